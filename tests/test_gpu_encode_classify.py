"""GPU encoder and tile classifier vs the oracle: bit-exact.

The expected values are derived by the oracle from the dense mask of each
family (canonical intervals / bitmap / lists, exact tile states, compact lists,
longest-first order); the GPU path computes them from the compressed
description only.
"""

import numpy as np
import pytest

import synth
from oracle import encode as OE
from oracle import masks as OM

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fm = pytest.importorskip("mask_aware_block_amd")

TILE_SHAPES_IV = [(128, 64), (64, 64), (256, 64), (16, 64), (48, 64), (32, 48), (16, 16), (256, 128), (48, 208)]
TILE_SHAPES_BM = [(128, 64), (64, 64), (64, 128), (256, 192)]


def _small_specs():
    rng = np.random.default_rng(123)
    out = []
    for S in (333, 64, 1):
        cu = np.unique(np.concatenate(([0, S], rng.integers(1, S, size=min(5, S - 1)) if S > 1 else [])))
        cu = cu.astype(np.int32)
        out += [
            dict(family="causal", sq=S, skv=S),
            dict(family="document", sq=S, skv=S, cu_seg=cu),
            dict(family="causal_document", sq=S, skv=S, cu_seg=cu),
            dict(family="shared_question", sq=S, skv=S, cu_seg=cu),
            dict(family="band", sq=S, skv=S, pre=37, next=5),
            dict(family="band", sq=S, skv=S, pre=9, next=-3),
            dict(family="band", sq=S, skv=S, pre=-3, next=7),
            dict(family="band", sq=S, skv=S, pre=2, next=-3),           # every row empty
            dict(family="band", sq=S, skv=S, pre=10 ** 15, next=-10 ** 15),
        ]
    out += [
        dict(family="causal", sq=200, skv=333),
        dict(family="causal_bottom_right", sq=200, skv=333),
        dict(family="band", sq=100, skv=300, pre=50, next=0),
        dict(family="band", sq=300, skv=100, pre=6, next=-2),
        dict(family="tree", sq=300, skv=300, tree_prefix=236,
             tree_parent=synth.random_tree(rng, 64, order="dfs")),
    ]
    # more segments than the encoder passes in its kernel arguments (64): the
    # segment starts go through a device copy instead
    cu_many = np.unique(np.concatenate(([0, 1500], rng.choice(np.arange(1, 1500), 99, replace=False))))
    cu_many = cu_many.astype(np.int32)
    out += [dict(family=f, sq=1500, skv=1500, cu_seg=cu_many)
            for f in ("document", "causal_document", "shared_question")]
    for n in (64, 65):  # the last count passed in the arguments, the first copied
        out.append(dict(family="causal_document", sq=1500, skv=1500,
                        cu_seg=np.array(cu_many[:n].tolist() + [1500], dtype=np.int32)))
    # packed variable-length batches: every mode, empty segments, Sq != Skv
    for trial in range(3):
        n = 6
        ql = rng.integers(0, 90, n)
        kl = rng.integers(0, 120, n)
        ql[1] = 0
        kl[3] = 0
        modes = ["full", "causal", "causal_bottom_right", "band", "prefix", "causal_bottom_right"]
        out.append(dict(family="varlen", sq=int(ql.sum()), skv=int(kl.sum()),
                        cu_q=np.concatenate(([0], np.cumsum(ql))).astype(np.int32),
                        cu_k=np.concatenate(([0], np.cumsum(kl))).astype(np.int32),
                        seg_mode=modes[trial:] + modes[:trial], pre=20 + trial, next=-2 + 3 * trial,
                        seg_prefix=rng.integers(0, 40, n).astype(np.int32)))
    return out


def _dense_all(spec, b=0, h=0):
    return np.asarray(OM.dense_vis(spec, b, h))


@pytest.mark.parametrize("spec", _small_specs(), ids=lambda s: f"{s['family']}-{s['sq']}x{s['skv']}")
def test_interval_families_exact(spec):
    enc = fm.encode(spec)
    assert enc.kind == fm.ENC_INTERVALS
    vis = _dense_all(spec)
    exp = OE.intervals_from_dense(vis)
    got = enc.intervals().cpu().numpy()[0, 0]
    np.testing.assert_array_equal(got, exp)
    for bm, bn in TILE_SHAPES_IV:
        t = fm.classify(enc, bm, bn)
        st, ls, cn, od = [x.cpu().numpy() for x in t.arrays()]
        exp_st = OE.tile_states(vis, bm, bn)
        np.testing.assert_array_equal(st[0, 0], exp_st, err_msg=f"states {bm}x{bn}")
        el, ec = OE.tile_lists(exp_st)
        np.testing.assert_array_equal(ls[0, 0], el, err_msg=f"lists {bm}x{bn}")
        np.testing.assert_array_equal(cn[0, 0], ec)
        np.testing.assert_array_equal(od, OE.tile_order(ec))


def test_raw_intervals_canonicalised():
    rng = np.random.default_rng(5)
    B, H, S, K = 2, 3, 150, 170
    raw = rng.integers(-20, S + 20, size=(B, H, 4, K)).astype(np.int32)
    # a few structured columns: abutting, overlapping, nested, empty
    raw[0, 0, :, 0] = [0, 10, 10, 20]
    raw[0, 0, :, 1] = [30, 50, 40, 60]
    raw[0, 0, :, 2] = [30, 80, 40, 60]
    raw[0, 0, :, 3] = [5, 5, 9, 3]
    raw[0, 0, :, 4] = [100, 120, 0, 10]
    spec = dict(family="intervals", sq=S, skv=K, batch=B, heads=H, raw_intervals=raw)
    enc = fm.encode(spec)
    got = enc.intervals().cpu().numpy()
    for b in range(B):
        for h in range(H):
            vis = _dense_all(spec, b, h)
            np.testing.assert_array_equal(got[b, h], OE.intervals_from_dense(vis), err_msg=f"{b},{h}")
    t = fm.classify(enc, 64, 64)
    st, ls, cn, od = [x.cpu().numpy() for x in t.arrays()]
    allc = []
    for b in range(B):
        for h in range(H):
            es = OE.tile_states(_dense_all(spec, b, h), 64, 64)
            np.testing.assert_array_equal(st[b, h], es)
            allc.append(OE.tile_lists(es)[1])
    np.testing.assert_array_equal(od, OE.tile_order(np.concatenate(allc), len(allc[0])))


def _bitmap_expect(spec, b, h):
    st, ix, pool = OE.bitmap_from_dense(_dense_all(spec, b, h))
    return st, ix, pool


def _check_bitmap(enc, spec, B, H):
    st, ix, bits, cnt = enc.bitmap()
    st, ix, bits = st.cpu().numpy(), ix.cpu().numpy(), bits.cpu().numpy().view(np.uint64)
    pool_all = []
    for b in range(B):
        for h in range(H):
            es, ei, ep = _bitmap_expect(spec, b, h)
            np.testing.assert_array_equal(st[b, h], es, err_msg=f"state {b},{h}")
            np.testing.assert_array_equal(ix[b, h] >= 0, ei >= 0)
            off = len(pool_all)
            np.testing.assert_array_equal(ix[b, h][ei >= 0], ei[ei >= 0] + off)
            pool_all += ep
    assert cnt == len(pool_all)
    if pool_all:
        np.testing.assert_array_equal(bits, np.array(pool_all, dtype=np.uint64))


@pytest.mark.parametrize("S,K,diag", [(300, 300, True), (130, 200, False), (64, 64, True), (1, 70, True)])
def test_block_bitmap_exact(S, K, diag):
    rng = np.random.default_rng(S + K)
    B = 2
    nbq, nbk = -(-S // 64), -(-K // 64)
    sts, ixs, pools, off = [], [], [], 0
    for _ in range(B):
        st, ix, bits = synth.block_pattern(rng, nbq, nbk, 0.3, 0.3)
        sts.append(st)
        ixs.append(np.where(ix >= 0, ix + off, -1))
        pools.append(bits)
        off += bits.shape[0]
    spec = dict(family="block_bitmap", sq=S, skv=K, batch=B, heads=1,
                blk_state=np.stack(sts)[:, None], blk_index=np.stack(ixs)[:, None].astype(np.int32),
                blk_bits=np.concatenate(pools).reshape(-1, 64), force_diag=diag)
    enc = fm.encode(spec)
    assert enc.kind == fm.ENC_BITMAP
    _check_bitmap(enc, spec, B, 1)
    for bm, bn in TILE_SHAPES_BM:
        t = fm.classify(enc, bm, bn)
        st, ls, cn, od = [x.cpu().numpy() for x in t.arrays()]
        allc = []
        for b in range(B):
            es = OE.tile_states(_dense_all(spec, b, 0), bm, bn)
            np.testing.assert_array_equal(st[b, 0], es, err_msg=f"{bm}x{bn}")
            el, ec = OE.tile_lists(es)
            np.testing.assert_array_equal(ls[b, 0], el)
            allc.append(ec)
        np.testing.assert_array_equal(od, OE.tile_order(np.concatenate(allc), len(allc[0])))


def test_tree_bfs_goes_bitmap_dfs_goes_intervals():
    for name, kind in (("tree_4k", fm.ENC_BITMAP), ("tree_4k_dfs", fm.ENC_INTERVALS)):
        w = synth.workload(name)
        spec = w["mask"]
        enc = fm.encode(spec)
        assert enc.kind == kind, name
        vis = _dense_all(spec)
        if kind == fm.ENC_BITMAP:
            _check_bitmap(enc, spec, 1, 1)
        else:
            np.testing.assert_array_equal(enc.intervals().cpu().numpy()[0, 0], OE.intervals_from_dense_fast(vis))
        bm, bn = fm.preferred_tile("bf16", 128, kind)
        t = fm.classify(enc, bm, bn)
        st = t.arrays()[0].cpu().numpy()[0, 0]
        np.testing.assert_array_equal(st, OE.tile_states_fast(vis, bm, bn))


def test_selected_lists_exact():
    rng = np.random.default_rng(8)
    for skv, cells, n in [(131072, 32, 64), (1000, 32, 17), (100, 7, 5)]:
        nblk = -(-skv // cells)
        sel = synth.selected_lists(rng, 300, nblk, n=n)
        sel[5, :3] = [nblk, nblk + 7, -5]  # out-of-range entries are ignored too
        sel = np.stack([sel, rng.permutation(sel)])
        spec = dict(family="selected_key", sq=300, skv=skv, batch=2, sel=sel, sel_cells=cells)
        enc = fm.encode(spec)
        ls, cn = [x.cpu().numpy() for x in enc.lists()]
        el, ec = OE.canonical_lists(sel, nblk)
        np.testing.assert_array_equal(ls, el)
        np.testing.assert_array_equal(cn, ec)


@pytest.mark.parametrize("name", ["causal_doc_8k", "causal_doc_32k", "shared_question_32k", "band_32k",
                                  "band_neg_4k", "block_bitmap_16k", "varlen_prefill_32k"])
def test_full_size_tables(name):
    """Full-size encodings and tile tables: every tile state, sampled columns."""
    w = synth.workload(name)
    spec = w["mask"]
    enc = fm.encode(spec)
    bm, bn = fm.preferred_tile(w["dtype"], w["D"], enc.kind)
    t = fm.classify(enc, bm, bn)
    st, ls, cn, od = [x.cpu().numpy() for x in t.arrays()]
    S = w["Sq"]
    rng = np.random.default_rng(0)
    nb = spec.get("batch", 1)
    cols = np.unique(np.concatenate((rng.integers(0, w["Skv"], 200), [0, w["Skv"] - 1])))
    if enc.kind == fm.ENC_INTERVALS:
        got_iv = enc.intervals().cpu().numpy()[0, 0][:, cols]
        colvis = np.zeros((S, cols.size), dtype=bool)
    allc = []
    for b in range(nb):
        exp_st = np.zeros((t.struct.nqt, t.struct.nkt), dtype=np.uint8)
        for qt in range(t.struct.nqt):
            rows = np.arange(qt * bm, min(S, (qt + 1) * bm))
            v = np.asarray(OM.dense_vis(spec, b, 0, rows))
            exp_st[qt] = OE.tile_states_fast(v, bm, bn)[0]
            if enc.kind == fm.ENC_INTERVALS and b == 0:
                colvis[rows] = v[:, cols]
        np.testing.assert_array_equal(st[b, 0], exp_st)
        el, ec = OE.tile_lists(exp_st)
        np.testing.assert_array_equal(ls[b, 0], el)
        np.testing.assert_array_equal(cn[b, 0], ec)
        allc.append(ec)
    np.testing.assert_array_equal(od, OE.tile_order(np.concatenate(allc), len(allc[0])))
    if enc.kind == fm.ENC_INTERVALS:
        np.testing.assert_array_equal(got_iv, OE.intervals_from_dense(colvis))


def _dense_spec(vis, form):
    vis = np.asarray(vis, dtype=np.uint8)
    B, H, S, K = vis.shape
    return dict(family="dense", sq=S, skv=K, batch=B, heads=H, dense=vis, dense_form=form)


def test_dense_masks_take_the_interval_form_when_they_can():
    """Dense input of interval-representable masks: the automatic and the interval
    forms both give the canonical intervals of the oracle; the bitmap form gives
    the canonical bitmap."""
    rng = np.random.default_rng(77)
    S, K = 333, 290
    fams = [dict(family="causal_bottom_right", sq=S, skv=K), dict(family="band", sq=S, skv=K, pre=40, next=-5)]
    vis = np.stack([np.stack([np.asarray(OM.dense_vis(f)) for f in fams])])  # [1][2][S][K]
    vis[0, 1, :, 7] = False  # a column with no visible row
    for form in (None, "intervals"):
        spec = _dense_spec(vis, form)
        enc = fm.encode(spec)
        assert enc.kind == fm.ENC_INTERVALS
        got = enc.intervals().cpu().numpy()
        for h in range(2):
            np.testing.assert_array_equal(got[0, h], OE.intervals_from_dense(vis[0, h]))
    spec = _dense_spec(vis, "bitmap")
    enc = fm.encode(spec)
    assert enc.kind == fm.ENC_BITMAP
    _check_bitmap(enc, spec, 1, 2)


def _runs_column(rng, S, cuts):
    """A column of S rows with 0, 1 or 2 masked runs whose ends are drawn from
    `cuts` (row indices that fall on the encoder's chunk edges) or at random."""
    col = np.ones(S, dtype=bool)
    n = rng.integers(0, 3)
    pts = sorted(rng.choice(np.concatenate([cuts, rng.integers(0, S + 1, 8)]), 2 * n, replace=False))
    for a, b in zip(pts[0::2], pts[1::2]):
        col[a:b] = False
    return col


@pytest.mark.parametrize("K", [300, 208, 256])
def test_dense_runs_across_row_chunks(K):
    """Masked runs that start, end or meet on 64-row chunk edges, on the edges
    of the encoder's per-wave row shares and of its row groups (whose partial
    runs a second kernel joins), at a ragged size: canonical
    intervals bit-exact; a third run far from the other two sends the automatic
    form to the bitmap and makes the interval form fail.  K = 300 takes the
    byte-per-lane path (64-column strips); 208 and 256 (multiples of 16) the
    16-byte row loads over 128-column strips, 208 with a strip that ends
    inside its second half."""
    rng = np.random.default_rng(79)
    S = 2500
    # 64-row chunks, per-wave shares and (896 rows each here) row groups
    cuts = np.array([0, 63, 64, 65, 128, 191, 192, 193, 384, 895, 896, 897, 1152, 1792, 2496, 2499, 2500])
    vis = np.stack([_runs_column(rng, S, cuts) for _ in range(K)], axis=1)[None, None]
    vis[0, 0, :, 5] = True
    vis[0, 0, :, 6] = False
    vis[0, 0, 192:384, 7] = False  # one run that fills exactly one wave's share
    vis[0, 0, :, 70] = False  # columns in the second half of a 128-column strip
    vis[0, 0, 896:1792, 199] = False
    spec = _dense_spec(vis, None)
    enc = fm.encode(spec)
    assert enc.kind == fm.ENC_INTERVALS
    np.testing.assert_array_equal(enc.intervals().cpu().numpy()[0, 0], OE.intervals_from_dense(vis[0, 0]))
    vis[0, 0, :, 9] = True
    vis[0, 0, 10:20, 9] = False
    vis[0, 0, 500:700, 9] = False
    vis[0, 0, 2400:2500, 9] = False
    enc = fm.encode(_dense_spec(vis, None))
    assert enc.kind == fm.ENC_BITMAP
    _check_bitmap(enc, _dense_spec(vis, None), 1, 1)
    with pytest.raises(fm.FmaskError) as ei:
        fm.encode(_dense_spec(vis, "intervals"))
    assert ei.value.status == fm.ERR_INVALID


@pytest.mark.parametrize("K", [208, 256])
def test_dense_row_loads_with_several_masks(K):
    """The 16-byte row-load path of the dense encoder with one mask per (batch,
    head) (2 x 2 distinct masks) and several row groups: the mask index taken
    from the workgroup, the per-mask row base and the per-(mask, group) partial
    runs; every slice bit-exact with the oracle's canonical intervals."""
    rng = np.random.default_rng(81)
    S = 2500
    cuts = np.array([0, 63, 64, 65, 191, 192, 384, 895, 896, 897, 1792, 2496, 2500])
    vis = np.stack([np.stack([np.stack([_runs_column(rng, S, cuts) for _ in range(K)], axis=1)
                              for _ in range(2)]) for _ in range(2)])
    assert len({vis[b, h].tobytes() for b in range(2) for h in range(2)}) == 4
    enc = fm.encode(_dense_spec(vis, "intervals"))
    got = enc.intervals().cpu().numpy()
    for b in range(2):
        for h in range(2):
            np.testing.assert_array_equal(got[b, h], OE.intervals_from_dense(vis[b, h]), err_msg=f"mask ({b}, {h})")


def test_dense_masks_fall_back_to_the_bitmap_form():
    rng = np.random.default_rng(78)
    S, K = 300, 260
    tree = dict(family="tree", sq=S, skv=S, tree_prefix=S - 64, tree_parent=synth.random_tree(rng, 64, order="bfs"))
    rand = rng.random((S, K)) < 0.3
    vis = np.zeros((2, 1, S, K), dtype=bool)
    vis[0, 0] = np.asarray(OM.dense_vis(tree))[:, :K]
    vis[1, 0] = rand
    spec = _dense_spec(vis, None)
    enc = fm.encode(spec)
    assert enc.kind == fm.ENC_BITMAP
    _check_bitmap(enc, spec, 2, 1)
    with pytest.raises(fm.FmaskError) as ei:
        fm.encode(_dense_spec(vis, "intervals"))
    assert ei.value.status == fm.ERR_INVALID
    # tables at the bitmap tile
    t = fm.classify(enc, 64, 64)
    st = t.arrays()[0].cpu().numpy()
    for b in range(2):
        np.testing.assert_array_equal(st[b, 0], OE.tile_states(vis[b, 0], 64, 64))


def test_caller_buffers_reused_across_calls():
    """encode / classify into caller-owned buffers (bigger than needed, reused
    for a second, different mask): the same encodings and tables as fresh ones."""
    a = dict(family="causal_document", sq=700, skv=700, cu_seg=np.array([0, 100, 450, 700], dtype=np.int32))
    b = dict(family="band", sq=650, skv=650, pre=40, next=3)
    ebuf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    tbuf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    for spec in (a, b):
        ref = fm.encode(spec)
        got = fm.encode(spec, out=ebuf)
        assert got.buf.data_ptr() == ebuf.data_ptr()
        assert torch.equal(got.intervals(), ref.intervals())
        tr = fm.classify(ref, 128, 64)
        tg = fm.classify(got, 128, 64, out=tbuf)
        assert tg.buf.data_ptr() == tbuf.data_ptr()
        for x, y in zip(tr.arrays(), tg.arrays()):
            assert torch.equal(x, y)


def test_tile_order_per_slice_at_scale():
    """The per-slice longest-first order when slices do not align with the
    order kernel's 256-row blocks: 2 x 2 mask slices of 300 tile rows each
    (64 x 64 tiles), raw intervals with row-dependent lengths; the order must
    equal the oracle's tile_order of the same counts, slice by slice."""
    rng = np.random.default_rng(77)
    B, H, S, K = 2, 2, 300 * 64, 5 * 64 + 9
    raw = np.zeros((B, H, 4, K), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            # column c masks rows [c_lo, c_hi): per-column random runs give rows
            # a spread of list lengths, with ties
            lo = rng.integers(0, S, size=K)
            raw[b, h, 0] = lo
            raw[b, h, 1] = np.minimum(S, lo + rng.integers(0, S // 2, size=K))
            raw[b, h, 2] = S
            raw[b, h, 3] = S
    enc = fm.encode(dict(family="intervals", sq=S, skv=K, batch=B, heads=H, raw_intervals=raw))
    t = fm.classify(enc, 64, 64)
    st, ls, cn, od = [x.cpu().numpy() for x in t.arrays()]
    assert cn.shape == (B, H, 300)
    np.testing.assert_array_equal(od, OE.tile_order(cn.ravel(), 300))
    assert sorted(od.tolist()) == list(range(B * H * 300))
