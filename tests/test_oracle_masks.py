"""Pins of the oracle's mask families and canonical encodings.

- special cases that reduce to another family (one document = causal, band with
  a huge preTokens and nextTokens = 0 = causal as the Ascend sparseMode page
  states for mode 0, tree as a chain = causal, ...);
- exact visible-pair counts of the workloads, from closed forms;
- the Ascend sparseMode page's worked varlen splits (tests/golden);
- the band's non-empty condition the Ascend page states for negative
  nextTokens / preTokens (which pins inclusive ends);
- dense -> canonical intervals -> dense round trips, closed-form intervals per
  family, closed-form causal / band tile states, brute-force tile states;
- the (batch, head) slice a mask given per batch entry and head is read at, and
  the broadcast of a mask given once, against element-by-element loops;
- the dense family (any nonzero byte visible) against the families it is built
  from.
"""

import json
import os

import numpy as np
import pytest

import synth
from oracle import encode as E
from oracle import masks as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dense(spec, b=0, h=0):
    return np.asarray(M.dense_vis(spec, b, h))


def causal(s):
    return np.tril(np.ones((s, s), dtype=bool))


# ---------------------------------------------------------------- families

def test_family_reductions():
    S = 40
    one_doc = np.array([0, S], dtype=np.int32)
    np.testing.assert_array_equal(dense(dict(family="causal_document", sq=S, skv=S, cu_seg=one_doc)), causal(S))
    assert dense(dict(family="document", sq=S, skv=S, cu_seg=one_doc)).all()
    np.testing.assert_array_equal(dense(dict(family="shared_question", sq=S, skv=S, cu_seg=one_doc)), causal(S))
    np.testing.assert_array_equal(dense(dict(family="causal", sq=S, skv=S)), causal(S))
    # Ascend mode 0: nextTokens = 0 and preTokens >= Sq is causal (diagonal included)
    np.testing.assert_array_equal(dense(dict(family="band", sq=S, skv=S, pre=S, next=0)), causal(S))
    np.testing.assert_array_equal(dense(dict(family="band", sq=S, skv=S, pre=10 ** 12, next=0)), causal(S))
    assert dense(dict(family="band", sq=S, skv=S, pre=S, next=S)).all()
    chain = np.arange(-1, 23, dtype=np.int32)  # parent[t] = t - 1
    np.testing.assert_array_equal(
        dense(dict(family="tree", sq=S, skv=S, tree_prefix=S - 24, tree_parent=chain)), causal(S))
    sel = np.tile(np.arange(4, dtype=np.int32), (1, S, 1))
    assert dense(dict(family="selected_key", sq=S, skv=100, sel=sel, sel_cells=32)).all()
    st = np.full((1, 1, 1, 2), 2, dtype=np.uint8)
    assert dense(dict(family="block_bitmap", sq=S, skv=100, blk_state=st,
                      blk_index=np.full((1, 1, 1, 2), -1, np.int32),
                      blk_bits=np.zeros((0, 64), np.uint64))).all()
    raw = np.zeros((1, 1, 4, S), dtype=np.int32)
    raw[0, 0, 1] = np.arange(S)       # UT = [0, j)
    raw[0, 0, 2:] = S                 # LT empty
    np.testing.assert_array_equal(dense(dict(family="intervals", sq=S, skv=S, raw_intervals=raw)), causal(S))
    np.testing.assert_array_equal(dense(dict(family="causal_bottom_right", sq=S, skv=S)), causal(S))


def test_family_definitions_small():
    cu = np.array([0, 3, 5, 8], dtype=np.int32)  # segments [0,3) [3,5) [5,8)
    seg = np.array([0, 0, 0, 1, 1, 2, 2, 2])
    doc = seg[:, None] == seg[None, :]
    np.testing.assert_array_equal(dense(dict(family="document", sq=8, skv=8, cu_seg=cu)), doc)
    np.testing.assert_array_equal(dense(dict(family="causal_document", sq=8, skv=8, cu_seg=cu)), doc & causal(8))
    sq_vis = causal(8) & (doc | (seg[None, :] == 0))
    np.testing.assert_array_equal(dense(dict(family="shared_question", sq=8, skv=8, cu_seg=cu)), sq_vis)
    # answers never see each other: row 6 (answer 2) sees the question and its own answer
    assert dense(dict(family="shared_question", sq=8, skv=8, cu_seg=cu))[6].tolist() == [1, 1, 1, 0, 0, 1, 1, 0]
    # tree: prefix 2, nodes 0..3 with parents -1, 0, 0, 1
    t = dense(dict(family="tree", sq=6, skv=6, tree_prefix=2, tree_parent=np.array([-1, 0, 0, 1])))
    exp = np.array([[1, 0, 0, 0, 0, 0],
                    [1, 1, 0, 0, 0, 0],
                    [1, 1, 1, 0, 0, 0],
                    [1, 1, 1, 1, 0, 0],
                    [1, 1, 1, 0, 1, 0],
                    [1, 1, 1, 1, 0, 1]], dtype=bool)
    np.testing.assert_array_equal(t, exp)
    # bitmap: one PARTIAL block with a known word, force_diag adds (i, i)
    bits = np.zeros((1, 64), dtype=np.uint64)
    bits[0, 1] = np.uint64(0b1010)
    st = np.array([[[[1]]]], dtype=np.uint8)
    spec = dict(family="block_bitmap", sq=3, skv=5, blk_state=st,
                blk_index=np.zeros((1, 1, 1, 1), np.int32), blk_bits=bits, force_diag=False)
    assert dense(spec).astype(int).tolist() == [[0] * 5, [0, 1, 0, 1, 0], [0] * 5]
    spec["force_diag"] = True
    assert dense(spec).astype(int).tolist() == [[1, 0, 0, 0, 0], [0, 1, 0, 1, 0], [0, 0, 1, 0, 0]]


def test_pair_counts_of_workloads():
    # tiny causal document, documents 64/128/64: 64*65/2 + 128*129/2 + 64*65/2
    w = synth.workload("tiny_causal_doc")
    assert M.pair_count(w["mask"]) == 12416
    # causal document at 8192: sum of L(L+1)/2 over the drawn documents
    w = synth.workload("causal_doc_8k")
    assert M.pair_count(w["mask"]) == sum(L * (L + 1) // 2 for L in w["doc_lengths"])
    # band preTokens 9, nextTokens -3 at 4096: rows 0..2 empty, 3..8 see 1..6 keys, others 7
    w = synth.workload("band_neg_4k")
    vis = dense(w["mask"])
    assert int(vis.sum()) == 28630
    assert not vis[:3].any() and vis[3:].any(axis=1).all()
    # band preTokens 4096, nextTokens 0 on a shorter sequence: closed form
    S, pre = 6144, 4096
    spec = dict(family="band", sq=S, skv=S, pre=pre, next=0)
    assert M.pair_count(spec) == (pre + 1) * (pre + 2) // 2 - (pre + 1) + (S - pre) * (pre + 1)


@pytest.mark.slow
def test_pair_count_band_32k():
    w = synth.workload("band_32k")
    assert M.pair_count(w["mask"], chunk=1024) == 125_859_840


def test_ascend_varlen_split_examples():
    with open(os.path.join(GOLDEN, "ascend_varlen_split.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        b = case["batch"]
        qlen = np.diff([0] + case["actual_seq_qlen"])
        kvlen = np.diff([0] + case["actual_seq_kvlen"])
        sq, skv = int(qlen[b]), int(kvlen[b])
        assert (sq, skv) == (case["sq"], case["skv"])
        spec = dict(family=case["family"], sq=sq, skv=skv, pre=case.get("pre"), next=case.get("next"))
        np.testing.assert_array_equal(dense(spec).astype(int), np.array(case["expected"]), err_msg=case["name"])


def test_band_nonempty_condition_pins_inclusive_ends():
    # Ascend sparseMode page: negative nextTokens needs preTokens >= |nextTokens|,
    # negative preTokens needs nextTokens >= |preTokens|: exactly the condition for
    # a non-empty band with both ends inclusive.
    S = 64
    for pre, nxt in [(3, -3), (2, -3), (9, -3), (-3, 7), (-3, 3), (-4, 3)]:
        vis = dense(dict(family="band", sq=S, skv=S, pre=pre, next=nxt))
        interior = vis[20:40]
        nonempty = interior.any(axis=1).all()
        assert nonempty == (pre + nxt >= 0), (pre, nxt)
        if nonempty:
            assert (interior.sum(axis=1) == pre + nxt + 1).all()


# ---------------------------------------------------------------- encodings

def _family_specs():
    S = 200
    cu = np.array([0, 64, 70, 150, 200], dtype=np.int32)
    return [
        dict(family="causal", sq=S, skv=S),
        dict(family="causal_bottom_right", sq=150, skv=S),
        dict(family="document", sq=S, skv=S, cu_seg=cu),
        dict(family="causal_document", sq=S, skv=S, cu_seg=cu),
        dict(family="shared_question", sq=S, skv=S, cu_seg=cu),
        dict(family="band", sq=S, skv=S, pre=17, next=4),
        dict(family="band", sq=S, skv=S, pre=9, next=-3),
        dict(family="band", sq=S, skv=S, pre=-3, next=7),
        dict(family="band", sq=120, skv=S, pre=30, next=0),
        dict(family="tree", sq=S, skv=S, tree_prefix=S - 40,
             tree_parent=synth.random_tree(np.random.default_rng(3), 40, order="dfs")),
    ]


def test_interval_round_trip_and_fast_path():
    for spec in _family_specs():
        vis = dense(spec)
        iv = E.intervals_from_dense(vis)
        np.testing.assert_array_equal(E.dense_from_intervals(iv, spec["sq"]), vis, err_msg=str(spec["family"]))
        np.testing.assert_array_equal(E.intervals_from_dense_fast(vis), iv, err_msg=str(spec["family"]))
        # canonical form: runs disjoint and non-abutting, UT starts at 0
        assert (iv[0] == 0).all()
        assert ((iv[1] < iv[2]) | (iv[2] == iv[3]) | (iv[0] == iv[1])).all()


def test_bfs_tree_not_interval_representable():
    spec = synth.workload("tree_4k", Sq=4096)["mask"]
    vis = dense(spec)
    with pytest.raises(E.NotRepresentable):
        E.intervals_from_dense(vis[:, 4032:])
    with pytest.raises(E.NotRepresentable):
        E.intervals_from_dense_fast(vis)


def test_closed_form_intervals():
    S = 200
    cu = np.array([0, 64, 70, 150, 200])
    j = np.arange(S)
    seg = np.searchsorted(cu, j, side="right") - 1
    ds, de = cu[seg], cu[seg + 1]
    # causal document: UT = [0, j), LT = [doc_end, S)
    iv = E.intervals_from_dense(dense(dict(family="causal_document", sq=S, skv=S, cu_seg=cu)))
    exp_ut_end = j
    exp_lt = np.where(de < S, de, S)
    np.testing.assert_array_equal(iv[1], exp_ut_end)
    np.testing.assert_array_equal(iv[2], exp_lt)
    np.testing.assert_array_equal(iv[3], np.full(S, S))
    # document: UT = [0, doc_start) and LT = [doc_end, S) (one-run cases canonicalised)
    iv = E.intervals_from_dense(dense(dict(family="document", sq=S, skv=S, cu_seg=cu)))
    for c in range(S):
        runs = []
        if ds[c] > 0:
            runs.append((0, ds[c]))
        if de[c] < S:
            runs.append((de[c], S))
        assert tuple(iv[:, c]) == E.canonical_from_runs(runs, S)
    # band next >= 0: UT = [0, max(0, j - next)), LT = [min(S, j + pre + 1), S)
    pre, nxt = 17, 4
    iv = E.intervals_from_dense(dense(dict(family="band", sq=S, skv=S, pre=pre, next=nxt)))
    ut_end = np.maximum(0, j - nxt)
    lt_start = np.minimum(S, j + pre + 1)
    for c in range(S):
        runs = ([(0, ut_end[c])] if ut_end[c] > 0 else []) + ([(lt_start[c], S)] if lt_start[c] < S else [])
        assert tuple(iv[:, c]) == E.canonical_from_runs(runs, S)
    # band pre = 9, next = -3: masked [0, min(S, j + 3)) and [min(S, j + 10), S)
    iv = E.intervals_from_dense(dense(dict(family="band", sq=S, skv=S, pre=9, next=-3)))
    np.testing.assert_array_equal(iv[1], np.minimum(S, j + 3))
    lt = np.minimum(S, j + 10)
    np.testing.assert_array_equal(iv[2], lt)


def test_tile_states_closed_form_and_bruteforce():
    S = 300
    vis = causal(S)
    for bm, bn in [(128, 64), (64, 64), (32, 48)]:
        st = E.tile_states(vis, bm, bn)
        nqt, nkt = st.shape
        for qt in range(nqt):
            r0, r1 = qt * bm, min(S, (qt + 1) * bm) - 1
            for kt in range(nkt):
                c0, c1 = kt * bn, min(S, (kt + 1) * bn) - 1
                exp = 2 if c1 <= r0 else (0 if c0 > r1 else 1)
                assert st[qt, kt] == exp
        np.testing.assert_array_equal(E.tile_states_fast(vis, bm, bn), st)
    rng = np.random.default_rng(9)
    for _ in range(5):
        sq, skv = rng.integers(1, 90, 2)
        v = rng.random((sq, skv)) < rng.random()
        st = E.tile_states(v, 16, 32)
        for qt in range(st.shape[0]):
            for kt in range(st.shape[1]):
                cells = [v[i, j] for i in range(qt * 16, min(sq, qt * 16 + 16))
                         for j in range(kt * 32, min(skv, kt * 32 + 32))]
                exp = 2 if all(cells) else (1 if any(cells) else 0)
                assert st[qt, kt] == exp
        np.testing.assert_array_equal(E.tile_states_fast(v, 16, 32), st)


def test_tile_lists_and_order():
    st = np.array([[0, 2, 1, 0], [0, 0, 0, 0], [2, 2, 2, 1], [1, 0, 0, 2]], dtype=np.uint8)
    lists, counts = E.tile_lists(st)
    assert counts.tolist() == [2, 0, 4, 2]
    full = 1 << 31
    assert (lists[0, :2].view(np.uint32).tolist() == [1 | full, 2])
    assert (lists[2].view(np.uint32).tolist() == [0 | full, 1 | full, 2 | full, 3])
    assert (lists[3, :2].view(np.uint32).tolist() == [0, 3 | full])
    assert E.tile_order(counts).tolist() == [2, 0, 3, 1]
    # per slice of 3 rows: slice [5, 1, 5] -> rows 0, 2 (tie, lower index
    # first), 1; slice [0, 7] -> rows 4, 3 (the slices are not merged)
    assert E.tile_order([5, 1, 5, 0, 7], 3).tolist() == [0, 2, 1, 4, 3]
    assert E.tile_order([5, 1, 5, 0, 7]).tolist() == [4, 0, 2, 1, 3]


def test_bitmap_round_trip():
    rng = np.random.default_rng(11)
    for sq, skv in [(130, 200), (64, 64), (1, 70)]:
        vis = rng.random((sq, skv)) < 0.2
        vis[:40, :40] = True
        vis[:, 128:192] = False
        st, ix, pool = E.bitmap_from_dense(vis)
        spec = dict(family="block_bitmap", sq=sq, skv=skv, blk_state=st[None, None],
                    blk_index=ix[None, None], blk_bits=np.array(pool, dtype=np.uint64).reshape(-1, 64))
        np.testing.assert_array_equal(dense(spec), vis)
        # pool entries in row-major order, partial blocks only
        order = [tuple(x) for x in np.argwhere(st == 1)]
        assert [int(ix[b]) for b in order] == list(range(len(pool)))


def test_canonical_lists():
    sel = np.array([[[5, -1, 3, 5, 9, 3], [-1, -1, -1, -1, -1, -1], [0, 8, 7, 7, 1, 2]]], dtype=np.int32)
    lists, counts = E.canonical_lists(sel, nblk=8)
    assert lists[0, 0].tolist() == [3, 5, -1, -1, -1, -1]
    assert lists[0, 1].tolist() == [-1] * 6 and counts[0, 1] == 0
    assert lists[0, 2].tolist() == [0, 1, 2, 7, -1, -1] and counts[0, 2] == 4


def test_varlen_single_segment_reduces_to_the_families():
    for sq, skv in [(7, 7), (5, 9), (9, 4)]:
        one = lambda mode, **kw: dict(family="varlen", sq=sq, skv=skv, cu_q=[0, sq], cu_k=[0, skv],
                                      seg_mode=[mode], **kw)
        np.testing.assert_array_equal(dense(one("full")), np.ones((sq, skv), dtype=bool))
        np.testing.assert_array_equal(dense(one("causal")), dense(dict(family="causal", sq=sq, skv=skv)))
        np.testing.assert_array_equal(dense(one("causal_bottom_right")),
                                      dense(dict(family="causal_bottom_right", sq=sq, skv=skv)))
        np.testing.assert_array_equal(dense(one("band", pre=2, next=1)),
                                      dense(dict(family="band", sq=sq, skv=skv, pre=2, next=1)))
        # prefix 0 is bottom-right causal; a prefix as wide as the keys is full
        np.testing.assert_array_equal(dense(one("prefix", seg_prefix=[0])),
                                      dense(dict(family="causal_bottom_right", sq=sq, skv=skv)))
        np.testing.assert_array_equal(dense(one("prefix", seg_prefix=[skv])), np.ones((sq, skv), dtype=bool))


def test_varlen_reproduces_the_ascend_split_examples():
    """The packed masks of the Ascend varlen split examples: the named batch's
    block equals the page's printed rows, every other batch follows its own
    mode, and nothing crosses segments."""
    with open(os.path.join(GOLDEN, "ascend_varlen_split.json")) as f:
        gold = json.load(f)
    # mode of the other batches on the same card: mode 7 comes from
    # rightDownCausal, mode 8 from leftUpCausal (the page's notes)
    base = {"mode7": "causal_bottom_right", "mode8": "causal"}
    fam_to_mode = {"band": "band", "causal": "causal", "causal_bottom_right": "causal_bottom_right"}
    for case in gold["cases"]:
        cq, ck = [0] + case["actual_seq_qlen"], [0] + case["actual_seq_kvlen"]
        n = len(cq) - 1
        modes = [base[case["name"][:5]]] * n
        modes[case["batch"]] = fam_to_mode[case["family"]]
        spec = dict(family="varlen", sq=cq[-1], skv=ck[-1], cu_q=cq, cu_k=ck, seg_mode=modes,
                    pre=case.get("pre", 0), next=case.get("next", 0))
        vis = dense(spec)
        b = case["batch"]
        block = vis[cq[b]:cq[b + 1], ck[b]:ck[b + 1]]
        np.testing.assert_array_equal(block.astype(int), np.array(case["expected"]), err_msg=case["name"])
        for s in range(n):  # nothing outside the diagonal blocks
            outside = np.ones(ck[-1], dtype=bool)
            outside[ck[s]:ck[s + 1]] = False
            assert not vis[cq[s]:cq[s + 1], outside].any(), case["name"]


def test_varlen_intervals_round_trip():
    rng = np.random.default_rng(9)
    for _ in range(20):
        n = int(rng.integers(1, 6))
        ql = rng.integers(0, 9, n)
        kl = rng.integers(0, 9, n)
        cq = np.concatenate(([0], np.cumsum(ql))).tolist()
        ck = np.concatenate(([0], np.cumsum(kl))).tolist()
        modes = [str(m) for m in rng.choice(["full", "causal", "causal_bottom_right", "band", "prefix"], n)]
        spec = dict(family="varlen", sq=cq[-1], skv=ck[-1], cu_q=cq, cu_k=ck, seg_mode=modes,
                    pre=int(rng.integers(-2, 6)), next=int(rng.integers(-2, 4)),
                    seg_prefix=rng.integers(0, 5, n).tolist())
        vis = dense(spec)
        if vis.size == 0:
            continue
        iv = E.intervals_from_dense(vis)  # every column stays within two masked runs
        np.testing.assert_array_equal(E.dense_from_intervals(iv, vis.shape[0]), vis)


# ------------------------------------------- per-(batch, head) slices, dense

def _masked_by_intervals_loop(raw_bh, sq, skv):
    """Visibility of one raw-interval slice, element by element (pure Python)."""
    out = np.ones((sq, skv), dtype=bool)
    for j in range(skv):
        uts, ute, lts, lte = (int(raw_bh[f][j]) for f in range(4))
        for i in range(sq):
            if uts <= i < ute or lts <= i < lte:
                out[i, j] = False
    return out


def _bitmap_loop(state_bh, index_bh, bits, sq, skv):
    """Visibility of one 64 x 64 bitmap slice, element by element (pure Python)."""
    out = np.zeros((sq, skv), dtype=bool)
    for i in range(sq):
        for j in range(skv):
            st = int(state_bh[i // 64, j // 64])
            if st == 2:
                out[i, j] = True
            elif st == 1:
                word = int(bits[int(index_bh[i // 64, j // 64]), i % 64])
                out[i, j] = bool((word >> (j % 64)) & 1)
    return out


def test_mask_index_selects_the_batch_head_slice():
    """A mask given per (batch, head) -- the Ascend sparseMode page's attenMask
    shapes [B, N, S, S] and the Binary Block Masking block matrix per sequence --
    is read at slice (b, h); a mask given once for the batch (or for all heads)
    serves every batch entry (or head) from slice 0."""
    rng = np.random.default_rng(5)
    sq, skv, B, H = 70, 90, 2, 3
    raw = np.zeros((B, H, 4, skv), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            a = rng.integers(0, sq, skv)
            raw[b, h, 0] = 0
            raw[b, h, 1] = a                                   # UT = [0, a)
            raw[b, h, 2] = np.minimum(sq, a + 1 + rng.integers(0, 20, skv))
            raw[b, h, 3] = sq                                  # LT = [a + 1 + g, sq)
    expect = {(b, h): _masked_by_intervals_loop(raw[b, h], sq, skv) for b in range(B) for h in range(H)}
    # the six slices really differ, so a wrong slice cannot pass by accident
    assert len({e.tobytes() for e in expect.values()}) == B * H
    spec = dict(family="intervals", sq=sq, skv=skv, raw_intervals=raw, batch=B, heads=H)
    for (b, h), e in expect.items():
        np.testing.assert_array_equal(dense(spec, b, h), e)
    # batch = 1: every batch entry uses slice 0 of the batch axis
    spec1 = dict(family="intervals", sq=sq, skv=skv, raw_intervals=raw[:1], batch=1, heads=H)
    for b in range(B):
        for h in range(H):
            np.testing.assert_array_equal(dense(spec1, b, h), expect[(0, h)])
    # heads = 1: every head uses slice 0 of the head axis
    spech = dict(family="intervals", sq=sq, skv=skv, raw_intervals=raw[:, :1], batch=B, heads=1)
    for b in range(B):
        for h in range(H):
            np.testing.assert_array_equal(dense(spech, b, h), expect[(b, 0)])

    # block bitmap, per (batch, head)
    sq, skv = 130, 150
    nbq, nbk = 3, 3
    st = rng.integers(0, 3, (B, H, nbq, nbk)).astype(np.uint8)
    ix = np.full(st.shape, -1, dtype=np.int32)
    npart = int((st == 1).sum())
    ix[st == 1] = np.arange(npart, dtype=np.int32)
    bits = rng.integers(0, 2 ** 63, (npart, 64), dtype=np.int64).astype(np.uint64)
    bits ^= rng.integers(0, 2, (npart, 64)).astype(np.uint64) << np.uint64(63)
    expect = {(b, h): _bitmap_loop(st[b, h], ix[b, h], bits, sq, skv) for b in range(B) for h in range(H)}
    assert len({e.tobytes() for e in expect.values()}) == B * H
    spec = dict(family="block_bitmap", sq=sq, skv=skv, blk_state=st, blk_index=ix, blk_bits=bits,
                batch=B, heads=H)
    for (b, h), e in expect.items():
        np.testing.assert_array_equal(dense(spec, b, h), e)
    spec1 = dict(spec, blk_state=st[:1], blk_index=ix[:1], batch=1)
    for b in range(B):
        for h in range(H):
            np.testing.assert_array_equal(dense(spec1, b, h), expect[(0, h)])
    spech = dict(spec, blk_state=st[:, :1], blk_index=ix[:, :1], heads=1)
    for b in range(B):
        for h in range(H):
            np.testing.assert_array_equal(dense(spech, b, h), expect[(b, 0)])


def test_dense_family_equals_the_families_it_is_built_from():
    """A dense uint8 mask (Ascend sparseMode 1 "allMask"; Binary Block Masking's
    full mask) holds any byte value; every nonzero byte means visible.  Built from
    six families with visible bytes drawn from 1..255, slice (b, h) must equal the
    family it was built from, and a zero written into a visible position hides
    exactly that position."""
    rng = np.random.default_rng(8)
    S = 96
    fams = [
        dict(family="causal", sq=S, skv=S),
        dict(family="causal_document", sq=S, skv=S, cu_seg=np.array([0, 20, 64, S], np.int32)),
        dict(family="shared_question", sq=S, skv=S, cu_seg=np.array([0, 32, 50, 80, S], np.int32)),
        dict(family="band", sq=S, skv=S, pre=9, next=-3),
        dict(family="tree", sq=S, skv=S, tree_prefix=S - 8,
             tree_parent=np.array([-1, 0, 0, 1, 1, 2, 3, 3], np.int32)),
        dict(family="document", sq=S, skv=S, cu_seg=np.array([0, 40, S], np.int32)),
    ]
    B, H = 2, 3
    vis = np.stack([np.asarray(M.dense_vis(f)) for f in fams]).reshape(B, H, S, S)
    val = rng.integers(1, 256, (B, H, S, S)).astype(np.uint8)   # 1..255, includes 1 and >= 2
    assert (val == 1).any() and (val >= 128).any()
    d = np.where(vis, val, 0).astype(np.uint8)
    spec = dict(family="dense", sq=S, skv=S, dense=d, batch=B, heads=H)
    for k, f in enumerate(fams):
        b, h = divmod(k, H)
        np.testing.assert_array_equal(dense(spec, b, h), np.asarray(M.dense_vis(f)))
    # polarity: clearing one visible byte hides exactly that element
    b, h = 1, 2
    i, j = map(int, np.argwhere(vis[b, h])[len(np.argwhere(vis[b, h])) // 2])
    d2 = d.copy()
    d2[b, h, i, j] = 0
    got = dense(dict(spec, dense=d2), b, h)
    want = vis[b, h].copy()
    want[i, j] = False
    np.testing.assert_array_equal(got, want)
    # a mask given once for all heads serves each head from head slice 0
    spech = dict(family="dense", sq=S, skv=S, dense=d[:, :1], batch=B, heads=1)
    for b in range(B):
        for h in range(H):
            np.testing.assert_array_equal(dense(spech, b, h), vis[b, 0])
