"""Seeded synthetic inputs for mask-aware attention (shared by tests and bench).

This module only draws random numbers and lays out the parameters of the
workloads; it holds none of the method's arithmetic (no masks are evaluated,
no encodings or attention are computed here).  Both the HIP path (through the
Python binding) and the oracle receive exactly the arrays produced here.

Recipe (stands in for the FlashMask evaluation dataset, which is not available,
and for the selected-key PR's model workload):
  * workload k draws from numpy Generator(PCG64) seeded with
    SeedSequence(1000 * k).spawn(4) -> independent streams for Q, K, V, mask;
  * Q, K, V entries are N(0, 1) drawn in float32; bf16 inputs are the round-to-
    nearest-even bf16 of those float32 values (kept as uint16 bit patterns);
  * document lengths: repeatedly a multiple of 64 drawn uniformly from
    [256, min(4096, rest)] among those that leave a rest of 0 or >= 256, until
    the sequence is filled (so every length is a multiple of 64, as on the
    FlashMask rebuttal page, and lies in [256, 4096]);
  * shared question: a 2048-token question followed by 8 answers whose lengths
    (multiples of 64) are a uniform random composition of the remaining tokens
    (7 distinct cut points among the 64-token units);
  * block bitmap: each 64 x 64 block independently FULL with probability 0.10,
    PARTIAL with 0.05 (elements Bernoulli(0.5)), else SKIP; the diagonal forced;
  * tree: 64 draft tokens, node 0 the root, node t's parent uniform among the
    earlier nodes of depth < 4, then renumbered stably by depth (breadth-first,
    Medusa-style) or in depth-first preorder;
  * selected key: per query 64 block indices uniform in [0, nblk), each replaced
    by -1 with probability 1/8; query 0 lists only -1, query 1 one block 64
    times, query 2 sixty-four distinct blocks (all blocks, repeated, if fewer).
"""

import math

import numpy as np

__all__ = [
    "streams", "normal_bf16", "normal_f32", "doc_lengths", "answer_lengths",
    "random_tree", "block_pattern", "selected_lists", "workload", "draw_qkv",
    "WORKLOADS",
]


def streams(k):
    """Four independent generators (Q, K, V, mask) for workload number k."""
    seqs = np.random.SeedSequence(1000 * k).spawn(4)
    return [np.random.Generator(np.random.PCG64(s)) for s in seqs]


def grad_stream(k):
    """A fifth independent generator (output gradient dO) for workload number k."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(1000 * k).spawn(5)[4]))


def _f32_to_bf16_bits(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def normal_f32(rng, shape, chunk=1 << 24):
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    for s in range(0, out.size, chunk):
        out[s: s + chunk] = rng.standard_normal(min(chunk, out.size - s), dtype=np.float32)
    return out.reshape(shape)


def normal_bf16(rng, shape, chunk=1 << 24):
    """bf16 bit patterns (uint16) of N(0, 1) float32 draws, rounded to nearest even."""
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    for s in range(0, out.size, chunk):
        n = min(chunk, out.size - s)
        out[s: s + n] = _f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32))
    return out.reshape(shape)


def doc_lengths(rng, total, lo=256, hi=4096, step=64):
    """Packed document lengths (multiples of step in [lo, hi]) summing to total."""
    assert total % step == 0 and total >= lo
    out, rest = [], total
    while rest > 0:
        cand = [L for L in range(lo, min(hi, rest) + 1, step)
                if rest - L == 0 or rest - L >= lo]
        L = int(cand[rng.integers(len(cand))])
        out.append(L)
        rest -= L
    return out


def answer_lengths(rng, total, parts=8, unit=64):
    """Uniform random composition of total (multiple of unit) into `parts` parts."""
    units = total // unit
    cuts = np.sort(rng.choice(np.arange(1, units), size=parts - 1, replace=False))
    bounds = np.concatenate(([0], cuts, [units]))
    return (np.diff(bounds) * unit).astype(int).tolist()


def random_tree(rng, n=64, max_depth=4, order="bfs"):
    """Parent array of a random draft tree (parent[t] < t, parent[0] = -1)."""
    parent = [-1]
    depth = [0]
    for t in range(1, n):
        cand = [u for u in range(t) if depth[u] < max_depth]
        p = int(cand[rng.integers(len(cand))])
        parent.append(p)
        depth.append(depth[p] + 1)
    if order == "bfs":
        new_of = {old: new for new, old in enumerate(sorted(range(n), key=lambda u: (depth[u], u)))}
    elif order == "dfs":
        children = [[] for _ in range(n)]
        for t in range(1, n):
            children[parent[t]].append(t)
        seq, stack = [], [0]
        while stack:
            u = stack.pop()
            seq.append(u)
            stack.extend(reversed(children[u]))
        new_of = {old: new for new, old in enumerate(seq)}
    else:
        raise ValueError(order)
    out = [0] * n
    for old in range(n):
        out[new_of[old]] = -1 if parent[old] < 0 else new_of[parent[old]]
    return np.array(out, dtype=np.int32)


def block_pattern(rng, nbq, nbk, p_full=0.10, p_partial=0.05, blk=64):
    """Random 64 x 64 block pattern: (state uint8 [nbq][nbk], index int32, bits uint64 [n][64])."""
    u = rng.random((nbq, nbk))
    state = np.where(u < p_full, 2, np.where(u < p_full + p_partial, 1, 0)).astype(np.uint8)
    index = np.full((nbq, nbk), -1, dtype=np.int32)
    npart = int((state == 1).sum())
    index[state == 1] = np.arange(npart, dtype=np.int32)
    bits = rng.integers(0, np.iinfo(np.uint64).max, size=(npart, blk), dtype=np.uint64,
                        endpoint=True)
    return state, index, bits


def selected_lists(rng, sq, nblk, n=64, p_invalid=1 / 8, edge_rows=True):
    """Per-query block lists int32 [sq][n] with duplicates, -1 entries and (unless
    edge_rows is false) the edge rows: query 0 all -1, query 1 one block
    repeated, query 2 distinct blocks."""
    sel = rng.integers(0, nblk, size=(sq, n), dtype=np.int64)
    sel[rng.random((sq, n)) < p_invalid] = -1
    if not edge_rows:
        return sel.astype(np.int32)
    if sq > 0:
        sel[0] = -1
    if sq > 1:
        sel[1] = int(rng.integers(0, nblk))
    if sq > 2:  # distinct entries (every block once, then repeats, if n > nblk)
        sel[2] = np.resize(rng.permutation(nblk), n)
    return sel.astype(np.int32)


# ----------------------------------------------------------------------------
# Workloads.  Each returns a dict: shapes, dtype, scale, workload number (seed)
# and a mask spec (family name + parameters).
# ----------------------------------------------------------------------------

def _base(name, k, B, Hq, Hkv, Sq, Skv, D, dtype):
    return dict(name=name, seed=k, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D,
                dtype=dtype, scale=1.0 / math.sqrt(D))


def workload(name, **over):
    """Workload dict by name; keyword overrides shrink shapes for tests."""
    if name == "tiny_causal_doc":
        w = _base(name, 1, 1, 1, 1, 256, 256, 64, "f32")
        w.update(over)
        w["mask"] = dict(family="causal_document", sq=w["Sq"], skv=w["Skv"],
                         cu_seg=np.array([0, 64, 192, 256], dtype=np.int32))
        return w
    if name in ("causal_doc_8k", "causal_doc_32k"):
        S = 8192 if name == "causal_doc_8k" else 32768
        w = _base(name, 2, 1, 32, 8, S, S, 128, "bf16")
        w.update(over)
        rng = streams(w["seed"])[3]
        lens = doc_lengths(rng, w["Sq"])
        w["mask"] = dict(family="causal_document", sq=w["Sq"], skv=w["Skv"],
                         cu_seg=np.cumsum([0] + lens).astype(np.int32))
        w["doc_lengths"] = lens
        return w
    if name == "shared_question_32k":
        w = _base(name, 3, 1, 32, 8, 32768, 32768, 128, "bf16")
        w.update(over)
        question = over.get("question", 2048)
        rng = streams(w["seed"])[3]
        ans = answer_lengths(rng, w["Sq"] - question, parts=over.get("answers", 8))
        w["mask"] = dict(family="shared_question", sq=w["Sq"], skv=w["Skv"],
                         cu_seg=np.cumsum([0, question] + ans).astype(np.int32))
        w["answer_lengths"] = ans
        return w
    if name == "band_32k":
        w = _base(name, 3, 1, 32, 8, 32768, 32768, 128, "bf16")
        w.update(over)
        w["mask"] = dict(family="band", sq=w["Sq"], skv=w["Skv"],
                         pre=over.get("pre", 4096), next=over.get("next", 0))
        return w
    if name == "band_neg_4k":
        w = _base(name, 3, 1, 32, 8, 4096, 4096, 128, "bf16")
        w.update(over)
        w["mask"] = dict(family="band", sq=w["Sq"], skv=w["Skv"],
                         pre=over.get("pre", 9), next=over.get("next", -3))
        return w
    if name == "block_bitmap_16k":
        w = _base(name, 4, 4, 16, 16, 16384, 16384, 128, "bf16")
        w.update(over)
        rng = streams(w["seed"])[3]
        nbq, nbk = -(-w["Sq"] // 64), -(-w["Skv"] // 64)
        states, indices, pools = [], [], []
        off = 0
        for _ in range(w["B"]):
            st, ix, bits = block_pattern(rng, nbq, nbk)
            states.append(st)
            indices.append(np.where(ix >= 0, ix + off, -1))
            pools.append(bits)
            off += bits.shape[0]
        w["mask"] = dict(family="block_bitmap", sq=w["Sq"], skv=w["Skv"],
                         batch=w["B"], heads=1,
                         blk_state=np.stack(states)[:, None],
                         blk_index=np.stack(indices)[:, None].astype(np.int32),
                         blk_bits=np.concatenate(pools).reshape(-1, 64).astype(np.uint64),
                         force_diag=True)
        return w
    if name in ("tree_4k", "tree_4k_dfs"):
        w = _base(name, 4, 4, 16, 16, 4096, 4096, 128, "bf16")
        w.update(over)
        n = over.get("tree_n", 64)
        rng = streams(w["seed"])[3]
        parent = random_tree(rng, n, order="dfs" if name.endswith("dfs") else "bfs")
        w["mask"] = dict(family="tree", sq=w["Sq"], skv=w["Skv"],
                         tree_prefix=w["Sq"] - n, tree_parent=parent)
        return w
    if name == "selected_key_128k":
        w = _base(name, 5, 1, 32, 8, 2048, 131072, 256, "bf16")
        w.update(over)
        cells = 32
        rng = streams(w["seed"])[3]
        nblk = -(-w["Skv"] // cells)
        w["mask"] = dict(family="selected_key", sq=w["Sq"], skv=w["Skv"], batch=1,
                         sel=selected_lists(rng, w["Sq"], nblk)[None], sel_cells=cells)
        return w
    if name == "varlen_prefill_32k":
        # packed batch of sequences with a KV cache (chunked prefill): sequence
        # lengths by the document law at 32768 keys; each sequence's new
        # queries are its last quarter (multiples of 64 stay multiples of 16),
        # bottom-right causal inside each sequence
        w = _base(name, 13, 1, 32, 8, 0, 32768, 128, "bf16")
        w.update(over)
        rng = streams(w["seed"])[3]
        klens = doc_lengths(rng, w["Skv"])
        qlens = [L // 4 for L in klens]
        w["Sq"] = int(sum(qlens))
        w["mask"] = dict(family="varlen", sq=w["Sq"], skv=w["Skv"],
                         cu_q=np.cumsum([0] + qlens).astype(np.int32),
                         cu_k=np.cumsum([0] + klens).astype(np.int32),
                         seg_mode=["causal_bottom_right"] * len(klens))
        w["seq_lengths"] = dict(q=qlens, kv=klens)
        return w
    if name in ("selected_key_decode_128k", "selected_key_decode16_128k"):
        # few-query (decode) form: 1 or 16 queries at the end of a 128K context,
        # ordinary lists (no forced edge rows)
        sq = 1 if name == "selected_key_decode_128k" else 16
        w = _base(name, 11 if sq == 1 else 12, 1, 32, 8, sq, 131072, 256, "bf16")
        w.update(over)
        cells = 32
        rng = streams(w["seed"])[3]
        nblk = -(-w["Skv"] // cells)
        w["mask"] = dict(family="selected_key", sq=w["Sq"], skv=w["Skv"], batch=1,
                         sel=selected_lists(rng, w["Sq"], nblk, edge_rows=False)[None], sel_cells=cells)
        return w
    raise KeyError(name)


WORKLOADS = ("tiny_causal_doc", "causal_doc_8k", "causal_doc_32k", "shared_question_32k",
             "band_32k", "band_neg_4k", "block_bitmap_16k", "tree_4k", "tree_4k_dfs",
             "selected_key_128k", "selected_key_decode_128k", "selected_key_decode16_128k",
             "varlen_prefill_32k")


def draw_qkv(w):
    """(q, k, v) arrays of workload w: uint16 bf16 bits or float32, [B][H][S][D]."""
    rq, rk, rv, _ = streams(w["seed"])
    qs = (w["B"], w["Hq"], w["Sq"], w["D"])
    ks = (w["B"], w["Hkv"], w["Skv"], w["D"])
    gen = normal_bf16 if w["dtype"] == "bf16" else normal_f32
    return gen(rq, qs), gen(rk, ks), gen(rv, ks)


def draw_dout(w):
    """Output gradient dO of workload w, shaped like Q: N(0, 1) as bf16 bits or float32."""
    gen = normal_bf16 if w["dtype"] == "bf16" else normal_f32
    return gen(grad_stream(w["seed"]), (w["B"], w["Hq"], w["Sq"], w["D"]))
