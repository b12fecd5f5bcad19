"""Mask families -> dense visibility (oracle; test infrastructure only).

A mask is described by a plain dict ``spec`` with key ``family`` and the
family's parameters (below).  ``dense_vis(spec, b, h, rows)`` returns the boolean
matrix vis[i, j] (True = query row i attends to key column j) for the requested
rows and every key column, straight from the family's definition.  Nothing here
knows about tiles, intervals or kernels.

Families and their definitions (r, c are 0-based positions):

causal                vis = c <= r.  Ascend sparseMode page, "leftUpCausal" (mode 2)
                      and the mode-0 case nextTokens = 0, preTokens >= Sq.
causal_bottom_right   vis = c <= r + (Skv - Sq).  Ascend sparseMode page,
                      "rightDownCausal" (mode 3).
document              vis = seg(r) == seg(c).  FlashMask rebuttal, "Document Mask".
causal_document       vis = seg(r) == seg(c) and c <= r.  FlashMask rebuttal,
                      "Causal Document Mask"; Binary Block Masking abstract
                      (sequence packing).
shared_question       segment 0 is the question, segments 1.. are answers:
                      vis = c <= r and (seg(c) == seg(r) or seg(c) == 0).
                      FlashMask rebuttal, "Shared Question Mask".
band                  with rr = r + Skv - Sq:  rr - pre <= c <= rr + next, both ends
                      inclusive.  Ascend sparseMode page, mode 0 band / negative
                      pre or next, and mode 4 (anchored at the lower right corner).
tree                  causal prefix of P tokens then n draft tokens with parents
                      parent[t] < t (-1 = root): prefix rows causal; a draft row
                      sees the whole prefix and its ancestors and itself.  Binary
                      Block Masking abstract (tree masking for Medusa).
block_bitmap          64 x 64 blocks with state SKIP(0) / PARTIAL(1) / FULL(2);
                      PARTIAL blocks take bit (c mod 64) of word (r mod 64) of
                      their pool entry; if force_diag, (r, r) is visible too.
                      Binary Block Masking abstract.
selected_key          per query a list of block indices of `sel_cells` cells;
                      vis = floor(c / cells) is a valid listed entry (entries
                      outside [0, ceil(Skv / cells)) ignored, duplicates count
                      once); no causal term.  llama.cpp PR 119 description of
                      flash_attn_sel (visibility lives only in the list; -1 and
                      duplicate entries skipped; 32-cell blocks).
intervals             raw per-column masked intervals: masked iff
                      UTS_c <= r < UTE_c or LTS_c <= r < LTE_c.
varlen                packed batch of segments (cumulative query lengths cu_q,
                      key lengths cu_k): row r of segment s sees only columns of
                      segment s; with ii, jj the positions inside the segment and
                      off = K_s - Q_s, mode "full" sees all, "causal" jj <= ii,
                      "causal_bottom_right" jj <= ii + off, "band" rr - pre <= jj
                      <= rr + next (rr = ii + off), "prefix" jj < prefix_s or
                      jj <= ii + off.  Ascend sparseMode page (actual_seq_qlen /
                      actual_seq_kvlen, modes 2, 3, 4, 5, 7, 8).
dense                 the mask element by element, dense [B][H][Sq][Skv], nonzero =
                      visible (Ascend sparseMode 1 "allMask"; Binary Block Masking's
                      full mask).

Spec keys: sq, skv and, per family, cu_seg (cumulative boundaries, first 0, last
Sq), pre, next, tree_prefix, tree_parent, blk_state [B][H][nbq][nbk],
blk_index (same shape), blk_bits [pool][64] (uint64), force_diag, sel [B][Sq][n],
sel_cells, raw_intervals [B][H][4][Skv], cu_q, cu_k, seg_mode, seg_prefix, dense.
"""

import numpy as np

SKIP, PARTIAL, FULL = 0, 1, 2
BLOCK = 64


def _segment_of(cu_seg, pos):
    """Index s with cu_seg[s] <= pos < cu_seg[s+1]."""
    cu = np.asarray(cu_seg, dtype=np.int64)
    return np.searchsorted(cu, pos, side="right") - 1


def ancestor_or_self(parent):
    """anc[t, c] = True iff node c lies on the path from node t up to its root."""
    n = len(parent)
    anc = np.zeros((n, n), dtype=bool)
    for t in range(n):
        c = t
        while c >= 0:
            anc[t, c] = True
            c = int(parent[c])
    return anc


def mask_index(spec, b, h):
    """(b_m, h_m) mask slice used by batch entry b and query head h."""
    nb = spec.get("batch", 1)
    nh = spec.get("heads", 1)
    return (b if nb > 1 else 0), (h if nh > 1 else 0)


def dense_vis(spec, b=0, h=0, rows=None):
    """Dense visibility rows [len(rows), Skv] of the mask for batch b, q head h."""
    sq, skv = int(spec["sq"]), int(spec["skv"])
    if rows is None:
        rows = np.arange(sq, dtype=np.int64)
    r = np.asarray(rows, dtype=np.int64)[:, None]
    c = np.arange(skv, dtype=np.int64)[None, :]
    fam = spec["family"]
    bm, hm = mask_index(spec, b, h)

    if fam == "causal":
        return c <= r
    if fam == "causal_bottom_right":
        return c <= r + (skv - sq)
    if fam in ("document", "causal_document", "shared_question"):
        seg_r = _segment_of(spec["cu_seg"], r)
        seg_c = _segment_of(spec["cu_seg"], c)
        if fam == "document":
            return seg_r == seg_c
        if fam == "causal_document":
            return (seg_r == seg_c) & (c <= r)
        return (c <= r) & ((seg_c == seg_r) | (seg_c == 0))
    if fam == "band":
        rr = r + (skv - sq)
        return (c >= rr - int(spec["pre"])) & (c <= rr + int(spec["next"]))
    if fam == "tree":
        p = int(spec["tree_prefix"])
        anc = ancestor_or_self(spec["tree_parent"])
        vis = c <= r  # prefix rows (and, below, prefix columns of draft rows)
        draft = (r >= p)[:, 0]
        if draft.any():
            rd = r[draft, 0] - p
            v = np.zeros((rd.size, skv), dtype=bool)
            v[:, :p] = True
            v[:, p:] = anc[rd][:, : skv - p]
            vis = np.broadcast_to(vis, (r.shape[0], skv)).copy()
            vis[draft] = v
        return np.broadcast_to(vis, (r.shape[0], skv))
    if fam == "block_bitmap":
        state = np.asarray(spec["blk_state"])[bm, hm]
        index = np.asarray(spec["blk_index"])[bm, hm]
        bits = np.asarray(spec["blk_bits"], dtype=np.uint64)
        bi, bj = r // BLOCK, c // BLOCK
        st = state[bi, bj]
        idx = index[bi, bj]
        vis = st == FULL
        part = st == PARTIAL
        if part.any() and bits.size:
            words = bits[np.where(part, idx, 0), r % BLOCK]
            bit = (words >> (c % BLOCK).astype(np.uint64)) & np.uint64(1)
            vis = vis | (part & (bit == 1))
        if spec.get("force_diag", False):
            vis = vis | (c == r)
        return vis
    if fam == "selected_key":
        cells = int(spec["sel_cells"])
        nblk = -(-skv // cells)
        lists = np.asarray(spec["sel"])[bm][r[:, 0]]  # [R, n]
        blockvis = np.zeros((lists.shape[0], nblk + 1), dtype=bool)
        valid = (lists >= 0) & (lists < nblk)
        rr = np.broadcast_to(np.arange(lists.shape[0])[:, None], lists.shape)
        blockvis[rr[valid], lists[valid]] = True
        return blockvis[:, c[0] // cells]
    if fam == "dense":
        # the mask given element by element (nonzero = visible)
        return np.asarray(spec["dense"])[bm, hm][r[:, 0]] != 0
    if fam == "varlen":
        # Packed variable-length batch (Ascend sparseMode page, actual_seq_qlen /
        # actual_seq_kvlen): row i of query segment s sees only the key columns
        # of segment s, under that segment's mode, with positions taken inside
        # the segment and the causal / band anchor at the segment's lower right
        # corner (upper left for "causal").
        cq = np.asarray(spec["cu_q"], dtype=np.int64)
        ck = np.asarray(spec["cu_k"], dtype=np.int64)
        modes = list(spec["seg_mode"])
        prefix = spec.get("seg_prefix")
        vis = np.zeros((r.shape[0], skv), dtype=bool)
        for s in range(len(modes)):
            rows_s = (r[:, 0] >= cq[s]) & (r[:, 0] < cq[s + 1])
            if not rows_s.any() or ck[s + 1] == ck[s]:
                continue
            ii = r[rows_s] - cq[s]                    # [R_s, 1]
            jj = np.arange(ck[s + 1] - ck[s])[None, :]  # [1, K_s]
            off = (ck[s + 1] - ck[s]) - (cq[s + 1] - cq[s])
            m = modes[s]
            if m == "full":
                v = np.ones((ii.shape[0], jj.shape[1]), dtype=bool)
            elif m == "causal":
                v = jj <= ii
            elif m == "causal_bottom_right":
                v = jj <= ii + off
            elif m == "band":
                rr = ii + off
                v = (jj >= rr - int(spec["pre"])) & (jj <= rr + int(spec["next"]))
            elif m == "prefix":
                v = (jj < int(prefix[s])) | (jj <= ii + off)
            else:
                raise ValueError(f"unknown varlen mode {m!r}")
            vis[np.nonzero(rows_s)[0], ck[s]:ck[s + 1]] = np.broadcast_to(v, (ii.shape[0], jj.shape[1]))
        return vis
    if fam == "intervals":
        raw = np.asarray(spec["raw_intervals"], dtype=np.int64)[bm, hm]
        uts, ute, lts, lte = raw[0][None, :], raw[1][None, :], raw[2][None, :], raw[3][None, :]
        masked = ((uts <= r) & (r < ute)) | ((lts <= r) & (r < lte))
        return ~masked
    raise ValueError(f"unknown mask family {fam!r}")


def pair_count(spec, b=0, h=0, chunk=2048):
    """Number of visible (i, j) pairs, counted from the dense rows chunk by chunk."""
    sq = int(spec["sq"])
    total = 0
    for r0 in range(0, sq, chunk):
        total += int(dense_vis(spec, b, h, np.arange(r0, min(sq, r0 + chunk))).sum())
    return total
