"""GPU masked attention (through the C ABI) vs the float64 oracle.

Small shapes (several tiles and a ragged tail) are compared element by element
over every output; the workloads at their full sizes are compared on sampled
rows that the oracle computes one by one.
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as OA
from oracle import masks as OM
from tests.helpers import TOL, compare, sample_rows, to_device, to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fm = pytest.importorskip("mask_aware_block_amd")


def _run(w, arrays, spec=None):
    spec = spec or w["mask"]
    q, k, v = to_device(w, arrays)
    enc = fm.encode(spec)
    tiles = None
    if enc.kind != fm.ENC_SELECTED:
        tiles = fm.classify(enc, dtype=w["dtype"], d=w["D"])
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _dense_check(w, spec=None, what=""):
    spec = spec or w["mask"]
    arrays = synth.draw_qkv(w)
    o, lse = _run(w, arrays, spec)
    q, k, v = (to_f64(w, a) for a in arrays)
    ro, rl = OA.attention_dense(q, k, v, OA.spec_vis_fn(spec), w["scale"])
    return compare(w, o, lse, ro, rl, what or spec["family"])


def test_tiny_causal_doc_fp32():
    w = synth.workload("tiny_causal_doc")
    err = _dense_check(w)
    assert err[0] <= 1e-5


def _small(dtype, D, S=333, K=None, Hq=4, Hkv=2, B=1, seed=11):
    K = K or S
    w = dict(name="small", seed=seed, B=B, Hq=Hq, Hkv=Hkv, Sq=S, Skv=K, D=D, dtype=dtype,
             scale=1 / math.sqrt(D))
    return w


def _specs(S, K):
    rng = np.random.default_rng(S * 7 + K)
    cu = np.unique(np.concatenate(([0, S], rng.integers(1, S, 6)))).astype(np.int32)
    out = [dict(family="causal", sq=S, skv=K),
           dict(family="band", sq=S, skv=K, pre=40, next=3),
           dict(family="band", sq=S, skv=K, pre=9, next=-3)]
    if S == K:
        out += [dict(family="document", sq=S, skv=K, cu_seg=cu),
                dict(family="causal_document", sq=S, skv=K, cu_seg=cu),
                dict(family="shared_question", sq=S, skv=K, cu_seg=cu),
                dict(family="tree", sq=S, skv=S, tree_prefix=S - 64,
                     tree_parent=synth.random_tree(rng, 64, order="bfs")),
                dict(family="tree", sq=S, skv=S, tree_prefix=S - 64,
                     tree_parent=synth.random_tree(rng, 64, order="dfs"))]
    else:
        out += [dict(family="causal_bottom_right", sq=S, skv=K)]
    # a packed variable-length batch over the same totals
    ql = np.diff(np.unique(np.concatenate(([0, S], rng.integers(0, S, 3))))).tolist()
    kl = np.diff(np.unique(np.concatenate(([0, K], rng.integers(0, K, len(ql) - 1))))).tolist()
    if len(kl) == len(ql):
        modes = (["causal_bottom_right", "band", "prefix", "full", "causal"] * 2)[:len(ql)]
        out += [dict(family="varlen", sq=S, skv=K, cu_q=np.cumsum([0] + ql).astype(np.int32),
                     cu_k=np.cumsum([0] + kl).astype(np.int32), seg_mode=modes, pre=30, next=2,
                     seg_prefix=[16] * len(ql))]
    return out


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("S,K", [(333, 333), (200, 461)])
def test_small_families(dtype, D, S, K):
    w = _small(dtype, D, S, K)
    for spec in _specs(S, K):
        _dense_check(w, spec, f"{spec['family']} {dtype} d{D} {S}x{K}")


@pytest.mark.parametrize("family", ["causal", "causal_document", "tree"])
def test_running_maximum_jumps(family):
    """Scores that grow from key tile to key tile by far more than the lazy
    bound (q.k rises by about 300, i.e. 38 in the exp2 domain, per 64 keys), so
    that the kernel's lazy maximum overflows and redoes the tile with its exact
    maximum on every tile after a row's first, and rescales O and l each time."""
    S, D = 512, 128
    w = _small("bf16", D, S, S, Hq=4, Hkv=2)
    rng = np.random.default_rng(5)
    u = np.ones(D, np.float32)
    q = (u + 0.1 * rng.standard_normal((1, 4, S, D))).astype(np.float32)
    tile = (np.arange(S) // 64).astype(np.float32)
    k = (rng.standard_normal((1, 2, S, D)) + (300.0 / D) * tile[None, None, :, None] * u).astype(np.float32)
    v = rng.standard_normal((1, 2, S, D)).astype(np.float32)
    arrays = tuple(synth._f32_to_bf16_bits(a) for a in (q, k, v))
    if family == "causal":
        spec = dict(family="causal", sq=S, skv=S)
    elif family == "causal_document":
        spec = dict(family="causal_document", sq=S, skv=S, cu_seg=np.array([0, 200, 330, S], np.int32))
    else:  # bitmap encoding
        spec = dict(family="tree", sq=S, skv=S, tree_prefix=S - 64,
                    tree_parent=synth.random_tree(np.random.default_rng(3), 64, order="bfs"))
    o, lse = _run(w, arrays, spec)
    qd, kd, vd = (to_f64(w, a) for a in arrays)
    ro, rl = OA.attention_dense(qd, kd, vd, OA.spec_vis_fn(spec), w["scale"])
    compare(w, o, lse, ro, rl, f"running maximum jumps, {family}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_bitmap_and_raw_intervals(dtype):
    S, K = 320, 260
    w = _small(dtype, 128, S, K, B=2, Hq=4, Hkv=4)
    rng = np.random.default_rng(3)
    nbq, nbk = -(-S // 64), -(-K // 64)
    sts, ixs, pools, off = [], [], [], 0
    for _ in range(2):
        st, ix, bits = synth.block_pattern(rng, nbq, nbk, 0.3, 0.3)
        sts.append(st)
        ixs.append(np.where(ix >= 0, ix + off, -1))
        pools.append(bits)
        off += bits.shape[0]
    spec = dict(family="block_bitmap", sq=S, skv=K, batch=2, heads=1,
                blk_state=np.stack(sts)[:, None], blk_index=np.stack(ixs)[:, None].astype(np.int32),
                blk_bits=np.concatenate(pools).reshape(-1, 64), force_diag=True)
    _dense_check(w, spec, "bitmap")
    raw = rng.integers(-10, S + 10, size=(2, 4, 4, K)).astype(np.int32)
    spec = dict(family="intervals", sq=S, skv=K, batch=2, heads=4, raw_intervals=raw)
    _dense_check(w, spec, "raw intervals per head")


@pytest.mark.parametrize("bm", [256, 128, 64])
def test_interval_tile_shapes(bm):
    """Every bf16 interval kernel (256-, 128- and 64-row tiles) on ragged shapes."""
    for S, K, spec in [(333, 333, dict(family="causal_document", sq=333, skv=333,
                                       cu_seg=np.array([0, 70, 200, 333], dtype=np.int32))),
                       (700, 700, dict(family="band", sq=700, skv=700, pre=100, next=5)),
                       (300, 520, dict(family="causal_bottom_right", sq=300, skv=520))]:
        w = _small("bf16", 128, S, K, Hq=8, Hkv=2, B=2)
        arrays = synth.draw_qkv(w)
        q, k, v = to_device(w, arrays)
        enc = fm.encode(spec)
        tiles = fm.classify(enc, bm, 64)
        o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
        torch.cuda.synchronize()
        qq, kk, vv = (to_f64(w, a) for a in arrays)
        ro, rl = OA.attention_dense(qq, kk, vv, OA.spec_vis_fn(spec), w["scale"])
        compare(w, o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"bm {bm} {spec['family']}")


@pytest.mark.parametrize("bm", [128, 64])
@pytest.mark.parametrize("D", [128, 64])
def test_bitmap_tile_shapes(bm, D):
    """Bitmap masks at the 64- and 128-row tiles (the 128-row kernel reads each
    wave's own 64 x 64 block: FULL, SKIP or PARTIAL words): random block
    patterns per batch on a ragged shape with GQA, and a BFS-numbered tree."""
    S, K = 330, 390
    w = _small("bf16", D, S, K, B=2, Hq=4, Hkv=2, seed=12)
    rng = np.random.default_rng(5)
    nbq, nbk = -(-S // 64), -(-K // 64)
    sts, ixs, pools, off = [], [], [], 0
    for _ in range(2):
        st, ix, bits = synth.block_pattern(rng, nbq, nbk, 0.3, 0.3)
        sts.append(st)
        ixs.append(np.where(ix >= 0, ix + off, -1))
        pools.append(bits)
        off += bits.shape[0]
    spec = dict(family="block_bitmap", sq=S, skv=K, batch=2, heads=1,
                blk_state=np.stack(sts)[:, None], blk_index=np.stack(ixs)[:, None].astype(np.int32),
                blk_bits=np.concatenate(pools).reshape(-1, 64), force_diag=False)
    tree = dict(family="tree", sq=S, skv=S, tree_prefix=S - 64,
                tree_parent=synth.random_tree(rng, 64, order="bfs"))
    for sp, what in ((spec, "block bitmap"), (tree, "tree")):
        ww = dict(w, Skv=sp["skv"])
        arrays = synth.draw_qkv(ww)
        q, k, v = to_device(ww, arrays)
        enc = fm.encode(sp)
        assert enc.kind == fm.ENC_BITMAP
        tiles = fm.classify(enc, bm, 64)
        o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
        torch.cuda.synchronize()
        qq, kk, vv = (to_f64(ww, a) for a in arrays)
        ro, rl = OA.attention_dense(qq, kk, vv, OA.spec_vis_fn(sp), w["scale"])
        compare(ww, o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"{what} bm {bm} d{D}")


def test_bitmap_long_tile_rows():
    """More than 256 non-SKIP tiles in a row (past the kernel's LDS list stage):
    a 16K+ key range of mostly FULL and some PARTIAL blocks."""
    S, K = 150, 16384 + 1000
    w = _small("bf16", 64, S, K, B=1, Hq=2, Hkv=1, seed=13)
    rng = np.random.default_rng(6)
    nbq, nbk = -(-S // 64), -(-K // 64)
    st, ix, bits = synth.block_pattern(rng, nbq, nbk, 0.9, 0.08)
    spec = dict(family="block_bitmap", sq=S, skv=K, batch=1, heads=1, blk_state=st[None, None],
                blk_index=ix[None, None].astype(np.int32), blk_bits=bits.reshape(-1, 64), force_diag=False)
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(spec)
    for bm in (128, 64):
        tiles = fm.classify(enc, bm, 64)
        assert int(tiles.arrays()[2].max()) > 256
        o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
        torch.cuda.synchronize()
        qq, kk, vv = (to_f64(w, a) for a in arrays)
        ro, rl = OA.attention_dense(qq, kk, vv, OA.spec_vis_fn(spec), w["scale"])
        compare(w, o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"long rows bm {bm}")


def test_bitmap_large_pool_path():
    """Bitmap encodings whose pool capacity passes 2^22 blocks go to the general
    tile kernel (the 128-row and pair kernels use 32-bit pool offsets).  The
    same small mask, with its descriptor's capacity raised past that bound,
    takes that path at 128 x 64 and 64 x 64 tiles and must match the oracle
    (the kernels index the pool only through its real entries)."""
    S, K = 300, 700
    w = _small("bf16", 128, S, K, B=1, Hq=4, Hkv=2, seed=17)
    rng = np.random.default_rng(17)
    nbq, nbk = -(-S // 64), -(-K // 64)
    st, ix, bits = synth.block_pattern(rng, nbq, nbk, 0.3, 0.4)
    spec = dict(family="block_bitmap", sq=S, skv=K, batch=1, heads=1, blk_state=st[None, None],
                blk_index=ix[None, None].astype(np.int32), blk_bits=bits.reshape(-1, 64), force_diag=True)
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(spec)
    enc.struct.pool_cap = (1 << 22) + 1
    qq, kk, vv = (to_f64(w, a) for a in arrays)
    ro, rl = OA.attention_dense(qq, kk, vv, OA.spec_vis_fn(spec), w["scale"])
    for bm in (128, 64):
        tiles = fm.classify(enc, bm, 64)
        o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
        torch.cuda.synchronize()
        compare(w, o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"large-pool path bm {bm}")


def _tile_check(w, spec, bm, what):
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(spec)
    tiles = fm.classify(enc, bm, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    qq, kk, vv = (to_f64(w, a) for a in arrays)
    ro, rl = OA.attention_dense(qq, kk, vv, OA.spec_vis_fn(spec), w["scale"])
    return compare(w, o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, what)


def test_bitmap_pairs_per_head_masks():
    """64 x 64 bitmap tables (two block rows per workgroup, each walking its
    own list): per-(batch, head) block patterns of different densities, GQA,
    ragged keys, one block row with an empty list."""
    S, K, B, Hq, Hkv = 450, 515, 2, 4, 2
    w = _small("bf16", 128, S, K, B=B, Hq=Hq, Hkv=Hkv, seed=31)
    rng = np.random.default_rng(32)
    nbq, nbk = -(-S // 64), -(-K // 64)
    sts, ixs, pools, off = [], [], [], 0
    for i in range(B * Hq):
        pf = (0.05, 0.2, 0.5, 0.9)[i % 4]
        st, ix, bits = synth.block_pattern(rng, nbq, nbk, pf, 0.1)
        if i == 1:
            st[3] = 0  # block row 3 of (batch 0, head 1): nothing visible
            npart = int((st == 1).sum())
            ix = np.full(st.shape, -1, dtype=np.int32)
            ix[st == 1] = np.arange(npart, dtype=np.int32)
            bits = np.resize(bits, (npart, 64))
        sts.append(st)
        ixs.append(np.where(ix >= 0, ix + off, -1))
        pools.append(np.asarray(bits, dtype=np.uint64).reshape(-1, 64))
        off += pools[-1].shape[0]
    spec = dict(family="block_bitmap", sq=S, skv=K, batch=B, heads=Hq,
                blk_state=np.stack(sts).reshape(B, Hq, nbq, nbk),
                blk_index=np.stack(ixs).reshape(B, Hq, nbq, nbk).astype(np.int32),
                blk_bits=np.concatenate(pools).reshape(-1, 64), force_diag=False)
    _tile_check(w, spec, 64, "bitmap pairs, per-head masks")


def test_xcd_set_major_items():
    """Items dealt to the XCDs by whole (K/V head, batch) sets (16 sets of
    6 tile rows x 16 heads, per-batch masks and one shared mask, ragged)."""
    S, B, Hq, Hkv = 700, 2, 128, 8
    w = _small("bf16", 64, S, S, Hq=Hq, Hkv=Hkv, B=B, seed=5)
    rng = np.random.default_rng(8)
    nb = -(-S // 64)
    sts, ixs, pools, off = [], [], [], 0
    for _ in range(B):
        st, ix, bits = synth.block_pattern(rng, nb, nb, 0.2, 0.2)
        sts.append(st)
        ixs.append(np.where(ix >= 0, ix + off, -1))
        pools.append(bits)
        off += bits.shape[0]
    spec = dict(family="block_bitmap", sq=S, skv=S, batch=B, heads=1,
                blk_state=np.stack(sts)[:, None], blk_index=np.stack(ixs)[:, None].astype(np.int32),
                blk_bits=np.concatenate(pools).reshape(-1, 64), force_diag=True)
    _dense_check(w, spec, "set-major bitmap per batch")
    # the 64 x 64 table: pairs of block rows (11 rows: the last pair has one)
    _tile_check(w, spec, 64, "set-major bitmap per batch, 64-row pairs")
    raw = rng.integers(-10, S + 10, size=(B, 1, 4, S)).astype(np.int32)
    _dense_check(w, dict(family="intervals", sq=S, skv=S, batch=B, heads=1, raw_intervals=raw),
                 "set-major intervals per batch")
    cu = np.array([0, 90, 300, 301, 640, S], dtype=np.int32)
    _dense_check(w, dict(family="causal_document", sq=S, skv=S, cu_seg=cu), "set-major shared mask")


def test_gqa_groups_and_batch():
    for Hq, Hkv in [(8, 1), (8, 8), (6, 2)]:
        w = _small("bf16", 128, 257, 257, Hq=Hq, Hkv=Hkv, B=2)
        _dense_check(w, dict(family="causal", sq=257, skv=257), f"gqa {Hq}/{Hkv}")


def test_empty_and_degenerate():
    # every row empty: zero output, LSE -inf
    w = _small("bf16", 128, 130, 130)
    _dense_check(w, dict(family="band", sq=130, skv=130, pre=2, next=-3), "all empty")
    # one query row, one key
    w = _small("bf16", 128, 1, 1)
    _dense_check(w, dict(family="causal", sq=1, skv=1), "1x1")
    w = _small("f32", 64, 1, 70)
    _dense_check(w, dict(family="causal_bottom_right", sq=1, skv=70), "1x70")


def test_selected_small():
    w = _small("bf16", 256, 40, 1000, Hq=8, Hkv=2)
    rng = np.random.default_rng(4)
    nblk = -(-1000 // 32)
    sel = synth.selected_lists(rng, 40, nblk, n=64)[None]
    spec = dict(family="selected_key", sq=40, skv=1000, batch=1, sel=sel, sel_cells=32)
    _dense_check(w, spec, "selected")
    w = _small("bf16", 128, 33, 300, Hq=4, Hkv=4, B=2)
    sel = np.stack([synth.selected_lists(rng, 33, 10, n=7) for _ in range(2)])
    spec = dict(family="selected_key", sq=33, skv=300, batch=2, sel=sel, sel_cells=32)
    _dense_check(w, spec, "selected per batch")


FULL = ["causal_doc_8k", "causal_doc_32k", "shared_question_32k", "band_32k", "band_neg_4k", "varlen_prefill_32k",
        "block_bitmap_16k", "tree_4k", "tree_4k_dfs", "selected_key_128k"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    w = synth.workload(name)
    spec = w["mask"]
    arrays = synth.draw_qkv(w)
    o, lse = _run(w, arrays)
    rng = np.random.default_rng(1)
    extra = []
    if "cu_seg" in spec or "cu_q" in spec:
        cu = np.asarray(spec.get("cu_seg", spec.get("cu_q")))
        extra = list(cu[1:-1]) + list(cu[1:-1] - 1)
    samples = sample_rows(w, 96, rng, extra=tuple(int(x) for x in extra[:40]))
    decode = OA.bf16_bits_to_f64 if w["dtype"] == "bf16" else None
    q, k, v = arrays
    if spec["family"] == "selected_key":
        ro, rl = OA.attention_listed_cells(q, k, v, spec["sel"], spec["sel_cells"], w["scale"],
                                           samples, decode=decode)
    else:
        ro, rl = OA.attention_rows(q, k, v, OA.spec_vis_fn(spec), w["scale"], samples, decode=decode)
    idx = tuple(np.array(samples).T)
    compare(w, o[idx], lse[idx], ro, rl, name)


def test_poison_masked_kv_does_not_leak():
    """NaN in K/V columns that no row can see (SKIP tiles) must not reach the output."""
    w = _small("bf16", 128, 192, 384, Hq=4, Hkv=2)
    spec = dict(family="causal", sq=192, skv=384)  # keys 192.. are visible to no row
    arrays = synth.draw_qkv(w)
    o1, l1 = _run(w, arrays, spec)
    k, v = arrays[1].copy(), arrays[2].copy()
    k[:, :, 192:] = 0x7FC0  # bf16 NaN
    v[:, :, 192:] = 0x7FC0
    o2, l2 = _run(w, (arrays[0], k, v), spec)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_poison_unselected_blocks_do_not_leak():
    """Selected-key lists (one-pass, split and block-major forms): NaN in every K/V block that
    no query lists must not reach the output (those blocks are never gathered;
    the selected-key PR's poison cases).  The lists hold -1 entries, duplicates
    and an out-of-range index; the last block is ragged."""
    S, K = 40, 32 * 40 + 5
    w = _small("bf16", 256, S, K, Hq=8, Hkv=2, seed=21)
    rng = np.random.default_rng(22)
    sel = synth.selected_lists(rng, S, 20, n=64)  # blocks 0..19 only
    sel[5, 3] = 999  # outside [0, nblk): skipped like -1
    spec = dict(family="selected_key", sq=S, skv=K, batch=1, sel=sel[None], sel_cells=32)
    arrays = synth.draw_qkv(w)
    k, v = arrays[1].copy(), arrays[2].copy()
    k[:, :, 20 * 32:] = 0x7FC0  # bf16 NaN in blocks 20..40
    v[:, :, 20 * 32:] = 0x7FC0
    enc = fm.encode(spec)
    outs = []
    for arr in (arrays, (arrays[0], k, v)):
        q_, k_, v_ = to_device(w, arr)
        o1, l1 = fm.attn_fwd(q_, k_, v_, enc, None, scale=w["scale"])
        o2, l2 = fm.attn_fwd_split(q_, k_, v_, enc, splits=3, scale=w["scale"])
        o3, l3 = fm.attn_fwd_blocks(q_, k_, v_, enc, scale=w["scale"])
        torch.cuda.synchronize()
        outs.append([t.float().cpu().numpy() for t in (o1, l1, o2, l2, o3, l3)])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
    assert np.isfinite(outs[1][0]).all() and np.isfinite(outs[1][4]).all()


@pytest.mark.parametrize("bm", [128, 64])
def test_poison_bitmap_skip_column_does_not_leak(bm):
    """Block bitmap: NaN in a 64-key column whose blocks are SKIP for every row
    (never loaded) leaves the output bit-identical."""
    S, K = 300, 640
    w = _small("bf16", 128, S, K, Hq=2, Hkv=2, seed=23)
    rng = np.random.default_rng(24)
    nbq, nbk = -(-S // 64), K // 64
    st, ix, bits = synth.block_pattern(rng, nbq, nbk, 0.3, 0.3)
    st[:, 5] = 0  # block column 5: keys 320..383, SKIP for every row
    npart = int((st == 1).sum())
    ix = np.full(st.shape, -1, dtype=np.int32)
    ix[st == 1] = np.arange(npart, dtype=np.int32)
    bits = bits[:npart] if len(bits) >= npart else np.resize(bits, (npart, 64))
    spec = dict(family="block_bitmap", sq=S, skv=K, batch=1, heads=1, blk_state=st[None, None],
                blk_index=ix[None, None], blk_bits=np.asarray(bits, dtype=np.uint64).reshape(-1, 64),
                force_diag=False)
    arrays = synth.draw_qkv(w)
    k, v = arrays[1].copy(), arrays[2].copy()
    k[:, :, 320:384] = 0x7FC0
    v[:, :, 320:384] = 0x7FC0
    enc = fm.encode(spec)
    tiles = fm.classify(enc, bm, 64)
    res = []
    for arr in (arrays, (arrays[0], k, v)):
        q_, k_, v_ = to_device(w, arr)
        o, lse = fm.attn_fwd(q_, k_, v_, enc, tiles, scale=w["scale"])
        torch.cuda.synchronize()
        res.append((o.float().cpu().numpy(), lse.cpu().numpy()))
    np.testing.assert_array_equal(res[0][0], res[1][0])
    np.testing.assert_array_equal(res[0][1], res[1][1])
    qq, kk, vv = (to_f64(w, a) for a in arrays)
    ro, rl = OA.attention_dense(qq, kk, vv, OA.spec_vis_fn(spec), w["scale"])
    compare(w, res[1][0], res[1][1], ro, rl, f"bitmap poison bm {bm}")


def test_interval_long_tile_rows():
    """Interval encoding with more than 256 non-SKIP tiles in a row, past the
    kernel's LDS list stage: bottom-right causal, 150 queries over 20000 keys."""
    S, K = 150, 20000
    w = _small("bf16", 128, S, K, B=1, Hq=2, Hkv=1, seed=25)
    spec = dict(family="causal_bottom_right", sq=S, skv=K)
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(spec)
    tiles = fm.classify(enc, 128, 64)
    assert int(tiles.arrays()[2].max()) > 256
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    qq, kk, vv = (to_f64(w, a) for a in arrays)
    ro, rl = OA.attention_dense(qq, kk, vv, OA.spec_vis_fn(spec), w["scale"])
    compare(w, o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "interval long rows")


def test_deterministic():
    w = synth.workload("causal_doc_8k", Hq=8, Hkv=2)
    arrays = synth.draw_qkv(w)
    o1, l1 = _run(w, arrays)
    o2, l2 = _run(w, arrays)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_dense_mask_input_both_forms():
    """Attention over masks handed over element by element: an interval-shaped
    mask (interval form) and a random one (bitmap form), per (batch, head)."""
    rng = np.random.default_rng(41)
    S, K = 300, 270
    w = _small("bf16", 128, S, K, B=2, Hq=2, Hkv=2)
    band = np.asarray(OM.dense_vis(dict(family="band", sq=S, skv=K, pre=50, next=3)))
    vis = np.zeros((2, 2, S, K), dtype=np.uint8)
    vis[0, 0] = band
    vis[0, 1] = np.asarray(OM.dense_vis(dict(family="causal_bottom_right", sq=S, skv=K)))
    vis[1, 0] = band
    vis[1, 1] = vis[1, 0]
    spec = dict(family="dense", sq=S, skv=K, batch=2, heads=2, dense=vis)
    _dense_check(w, spec, "dense (interval form)")
    vis2 = (rng.random((2, 2, S, K)) < 0.2).astype(np.uint8)
    spec2 = dict(family="dense", sq=S, skv=K, batch=2, heads=2, dense=vis2)
    _dense_check(w, spec2, "dense (bitmap form)")
