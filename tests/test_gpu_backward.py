"""GPU attention backward (fmask_attn_bwd, through the C ABI) vs the float64
oracle gradient (oracle.attention.attention_backward_dense).

The forward output O and LSE the backward consumes come from the GPU forward
(they are inputs of the operation, like dO); the reference gradient is the
oracle's, computed from the same bf16 Q, K, V and dO alone.  Small shapes span
several tiles with ragged tails, GQA and per-head masks; the 8K causal-document
workload is checked on one K/V head group at its full size, and the 32K one and
the two bitmap workloads on sampled rows and keys (attention_backward_sampled).
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as OA
from tests.helpers import GRAD_SCALE_FLOOR, to_device, to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fm = pytest.importorskip("mask_aware_block_amd")

# bf16 gradients with fp32 accumulation.  Relative to the largest reference
# magnitude of each tensor: every product P dO, dS Q, dS K enters the MFMA
# with P or dS rounded to bf16 (2^-9 relative) and the result is rounded to
# bf16 once more (2^-9), D_i comes from the bf16-rounded forward output.
GRAD_TOL = dict(max_rel=2e-2, mean_rel=2e-3)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _grad_check(w, spec, what, heads=None):
    arrays = synth.draw_qkv(w)
    do_bits = synth.draw_dout(w)
    q, k, v = to_device(w, arrays)
    do = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).cuda()
    enc = fm.encode(spec)
    tiles = fm.classify(enc, 128, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    dq, dk, dv = fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    qq, kk, vv, dd = (to_f64(w, a) for a in (*arrays, do_bits))
    hq0, hq1 = heads or (0, w["Hq"])
    G = w["Hq"] // w["Hkv"]
    sl_q = slice(hq0, hq1)
    sl_k = slice(hq0 // G, hq1 // G)
    vis = OA.spec_vis_fn(spec)
    fn = (lambda b, h, rows: vis(b, h + hq0, rows))
    rq, rk, rv = OA.attention_backward_dense(qq[:, sl_q], kk[:, sl_k], vv[:, sl_k], dd[:, sl_q], fn, w["scale"])
    out = {}
    for name, got, ref in (("dq", dq[:, sl_q], rq), ("dk", dk[:, sl_k], rk), ("dv", dv[:, sl_k], rv)):
        g = got.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all(), f"{what}: {name} not finite"
        scale = max(np.abs(ref).max(), GRAD_SCALE_FLOOR)
        err = np.abs(g - ref)
        out[name] = (err.max() / scale, err.mean() / scale)
        assert err.max() <= GRAD_TOL["max_rel"] * scale, f"{what}: {name} max err {err.max():.3e} (ref max {scale:.3e})"
        assert err.mean() <= GRAD_TOL["mean_rel"] * scale, f"{what}: {name} mean err {err.mean():.3e}"
    print(what, {k: (f"{a:.2e}", f"{b:.2e}") for k, (a, b) in out.items()}, flush=True)
    return out


def _small(D, S, K, Hq=4, Hkv=2, B=1, seed=21):
    return dict(name="small", seed=seed, B=B, Hq=Hq, Hkv=Hkv, Sq=S, Skv=K, D=D, dtype="bf16",
                scale=1 / math.sqrt(D))


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("S,K", [(333, 333), (200, 461)])
def test_small_families(D, S, K):
    w = _small(D, S, K)
    rng = np.random.default_rng(S + K)
    specs = [dict(family="causal", sq=S, skv=K), dict(family="band", sq=S, skv=K, pre=40, next=3),
             dict(family="band", sq=S, skv=K, pre=9, next=-3)]
    if S == K:
        cu = np.unique(np.concatenate(([0, S], rng.integers(1, S, 6)))).astype(np.int32)
        specs += [dict(family="causal_document", sq=S, skv=K, cu_seg=cu),
                  dict(family="shared_question", sq=S, skv=K, cu_seg=cu),
                  dict(family="document", sq=S, skv=K, cu_seg=cu)]
    else:
        specs += [dict(family="causal_bottom_right", sq=S, skv=K)]
    ql = [S // 3, S // 3, S - 2 * (S // 3)]
    kl = [K // 2, K // 4, K - K // 2 - K // 4]
    specs += [dict(family="varlen", sq=S, skv=K, cu_q=np.cumsum([0] + ql).astype(np.int32),
                   cu_k=np.cumsum([0] + kl).astype(np.int32),
                   seg_mode=["causal_bottom_right", "prefix", "band"], seg_prefix=[0, 20, 0], pre=25, next=1)]
    for spec in specs:
        _grad_check(w, spec, f"{spec['family']} d{D} {S}x{K}")


def test_gqa_batch_and_per_head_masks():
    S, K = 300, 260
    w = _small(128, S, K, Hq=4, Hkv=2, B=2, seed=22)
    rng = np.random.default_rng(5)
    raw = rng.integers(-10, S + 10, size=(2, 4, 4, K)).astype(np.int32)
    _grad_check(w, dict(family="intervals", sq=S, skv=K, batch=2, heads=4, raw_intervals=raw),
                "raw intervals per (batch, head)")
    w8 = _small(128, 257, 257, Hq=8, Hkv=1, B=2, seed=23)
    _grad_check(w8, dict(family="causal", sq=257, skv=257), "gqa 8/1")


@pytest.mark.parametrize("D", [128, 64])
def test_bitmap_masks(D):
    """Masks in the 64 x 64 bitmap form: a BFS-numbered tree (subtrees that
    are not contiguous), a random block pattern per batch entry with the
    diagonal forced visible, and a random dense mask; ragged sizes, GQA 4/2."""
    rng = np.random.default_rng(31 + D)
    n, prefix = 70, 150
    S = prefix + n
    spec = dict(family="tree", sq=S, skv=S, tree_prefix=prefix,
                tree_parent=synth.random_tree(rng, n, order="bfs"))
    assert fm.encode(spec).kind == fm.ENC_BITMAP
    _grad_check(_small(D, S, S, seed=31), spec, f"tree (bfs) D{D}")
    S, K = 300, 270
    nbq, nbk = -(-S // 64), -(-K // 64)
    sts, ixs, pools, off = [], [], [], 0
    for _ in range(2):
        st, ix, bits = synth.block_pattern(rng, nbq, nbk, 0.3, 0.3)
        sts.append(st)
        ixs.append(np.where(ix >= 0, ix + off, -1))
        pools.append(np.asarray(bits, dtype=np.uint64).reshape(-1, 64))
        off += pools[-1].shape[0]
    spec = dict(family="block_bitmap", sq=S, skv=K, batch=2, heads=1,
                blk_state=np.stack(sts).reshape(2, 1, nbq, nbk),
                blk_index=np.stack(ixs).reshape(2, 1, nbq, nbk).astype(np.int32),
                blk_bits=np.concatenate(pools) if off else np.zeros((1, 64), np.uint64), force_diag=True)
    _grad_check(_small(D, S, K, B=2, seed=32), spec, f"block pattern per batch D{D}")
    dense = (rng.random((1, 1, S, K)) < 0.3).astype(np.uint8)
    spec = dict(family="dense", sq=S, skv=K, dense=dense)
    assert fm.encode(spec).kind == fm.ENC_BITMAP
    _grad_check(_small(D, S, K, seed=33), spec, f"random dense (bitmap form) D{D}")


def test_full_size_causal_doc_8k_one_group():
    w = synth.workload("causal_doc_8k")
    _grad_check(w, w["mask"], "causal_doc_8k heads 0..3", heads=(0, 4))


def test_full_size_causal_doc_32k_sampled():
    """The 32K causal-document backward at the size the bench times, against
    the float64 oracle on sampled outputs (attention_backward_sampled, pinned to
    the dense gradient on the CPU): dQ of 35 rows of query heads 0..3 (the
    sequence's first and last rows, tile and document edges, seeded others) and
    dK, dV of 12 keys of K/V head 0 in three documents (their first, middle and
    last keys, and a tile edge)."""
    w = synth.workload("causal_doc_32k")
    spec = w["mask"]
    arrays = synth.draw_qkv(w)
    do_bits = synth.draw_dout(w)
    q, k, v = to_device(w, arrays)
    do = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).cuda()
    enc = fm.encode(spec)
    tiles = fm.classify(enc, 128, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    dq, dk, dv = fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    G = w["Hq"] // w["Hkv"]
    S = w["Sq"]
    L = np.array(w["doc_lengths"])
    st = np.concatenate([[0], np.cumsum(L)])
    rng = np.random.default_rng(7)
    rows = sorted(set([0, 1, 127, 128, S - 1] + [int(st[d]) for d in (1, 7, 14)] +
                      [int(st[d + 1] - 1) for d in (0, 7, 13)] + [int(x) for x in rng.choice(S, 24, replace=False)]))
    keys = sorted(set([0, 1, 63, 64, int(L[0] - 1), int(st[3]), int(st[3] + L[3] // 2), int(st[4] - 1),
                       int(st[13]), int(st[13] + 1), int(st[14] - 2), int(st[14] - 1)]))
    qq, dd = (to_f64(w, a[:, :G]) for a in (arrays[0], do_bits))
    kk, vv = (to_f64(w, a[:, :1]) for a in (arrays[1], arrays[2]))
    rq, rk, rv = OA.attention_backward_sampled(qq, kk, vv, dd, OA.spec_vis_fn(spec), w["scale"], 0, rows, keys)
    got = dict(dq=dq[0, :G][:, rows], dk=dk[0, :1][:, keys], dv=dv[0, :1][:, keys])
    for name, ref in (("dq", rq), ("dk", rk), ("dv", rv)):
        g = got[name].float().cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all(), f"{name} not finite"
        scale = max(np.abs(ref).max(), GRAD_SCALE_FLOOR)
        err = np.abs(g - ref)
        print(f"causal_doc_32k sampled {name}: max {err.max() / scale:.2e}, mean {err.mean() / scale:.2e} "
              f"of the largest sampled reference value", flush=True)
        assert err.max() <= GRAD_TOL["max_rel"] * scale, f"{name} max err {err.max():.3e} (ref max {scale:.3e})"
        assert err.mean() <= GRAD_TOL["mean_rel"] * scale, f"{name} mean err {err.mean():.3e}"


@pytest.mark.parametrize("name,b", [("tree_4k", 0), ("block_bitmap_16k", 2)])
def test_full_size_bitmap_sampled(name, b):
    """Bitmap masks at full size (the BFS-numbered tree, and one batch entry of
    the per-batch random block pattern) against the float64 oracle on sampled
    outputs: dQ of 28 rows and dK, dV of 12 keys of head 0 (block and tile
    edges, the last row and key, seeded others)."""
    w = synth.workload(name)
    spec = w["mask"]
    arrays = synth.draw_qkv(w)
    do_bits = synth.draw_dout(w)
    q, k, v = to_device(w, arrays)
    do = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).cuda()
    enc = fm.encode(spec)
    assert enc.kind == fm.ENC_BITMAP
    tiles = fm.classify(enc, 128, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    dq, dk, dv = fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    G = w["Hq"] // w["Hkv"]
    S, K = w["Sq"], w["Skv"]
    rng = np.random.default_rng(11)
    rows = sorted(set([0, 63, 64, 127, 128, S - 1] + [int(x) for x in rng.choice(S, 22, replace=False)]))
    keys = sorted(set([0, 63, 64, K // 2, K - 1] + [int(x) for x in rng.choice(K, 7, replace=False)]))
    qq, dd = (to_f64(w, a[:, :G]) for a in (arrays[0], do_bits))
    kk, vv = (to_f64(w, a[:, :1]) for a in (arrays[1], arrays[2]))
    rq, rk, rv = OA.attention_backward_sampled(qq, kk, vv, dd, OA.spec_vis_fn(spec), w["scale"], b, rows, keys)
    got = dict(dq=dq[b, :G][:, rows], dk=dk[b, :1][:, keys], dv=dv[b, :1][:, keys])
    for nm, ref in (("dq", rq), ("dk", rk), ("dv", rv)):
        g = got[nm].float().cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all(), f"{name} {nm} not finite"
        scale = max(np.abs(ref).max(), GRAD_SCALE_FLOOR)
        err = np.abs(g - ref)
        print(f"{name} batch {b} sampled {nm}: max {err.max() / scale:.2e}, mean {err.mean() / scale:.2e} "
              f"of the largest sampled reference value", flush=True)
        assert err.max() <= GRAD_TOL["max_rel"] * scale, f"{name} {nm} max err {err.max():.3e} (ref max {scale:.3e})"
        assert err.mean() <= GRAD_TOL["mean_rel"] * scale, f"{name} {nm} mean err {err.mean():.3e}"


@pytest.mark.parametrize("S,K", [(0, 100), (100, 0), (0, 0)])
def test_zero_length_sequences(S, K):
    """No query rows or no keys (empty device tensors, whose pointers are null):
    the forward writes O = 0 and LSE = -inf for every row, the backward zero
    dQ when there is no key and zero dK, dV when there is no row."""
    w = _small(128, S, K, Hq=4, Hkv=2, B=2, seed=3)
    q, k, v = to_device(w, synth.draw_qkv(w))
    do = torch.from_numpy(synth.draw_dout(w).view(np.int16)).view(torch.bfloat16).cuda()
    enc = fm.encode(dict(family="causal_bottom_right", sq=S, skv=K))
    tiles = fm.classify(enc, 128, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    dq, dk, dv = fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    assert o.shape == q.shape and dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())
    assert bool((dq == 0).all()) and bool((dk == 0).all()) and bool((dv == 0).all())


def test_unsupported_combinations_are_refused():
    w = _small(128, 64, 64)
    q, k, v = to_device(w, synth.draw_qkv(w))
    enc = fm.encode(dict(family="causal", sq=64, skv=64))
    t64 = fm.classify(enc, 64, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, fm.classify(enc, 128, 64), scale=w["scale"])
    with pytest.raises(fm.FmaskError) as ei:
        fm.attn_bwd(q, k, v, o, lse, torch.zeros_like(o), enc, t64)
    assert ei.value.status == fm.ERR_UNSUPPORTED


def test_workspace_reuse_and_size_check():
    """A caller's workspace is checked against fmask_attn_bwd_workspace_bytes and
    fully rewritten by each call: one buffer serves a larger then a smaller
    problem (with different masks) and gives the same gradients as a fresh one."""
    big = _small(128, 461, 461, seed=23)
    small = _small(128, 200, 333, seed=24)
    runs = []
    for w, spec in ((big, dict(family="causal", sq=461, skv=461)),
                    (small, dict(family="band", sq=200, skv=333, pre=30, next=2))):
        q, k, v = to_device(w, synth.draw_qkv(w))
        do = torch.from_numpy(synth.draw_dout(w).view(np.int16)).view(torch.bfloat16).cuda()
        enc = fm.encode(spec)
        tiles = fm.classify(enc, 128, 64)
        o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
        runs.append((q, k, v, o, lse, do, enc, tiles, w["scale"]))
    nbytes = [fm.attn_bwd_workspace_bytes(r[0], r[1], r[2], r[3], r[7]) for r in runs]
    assert nbytes[0] > nbytes[1] > 0
    ws = torch.full((nbytes[0],), 0x7f, dtype=torch.uint8, device="cuda")
    for (q, k, v, o, lse, do, enc, tiles, scale) in runs:
        ref = fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=scale)
        got = fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=scale, workspace=ws)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
    q, k, v, o, lse, do, enc, tiles, scale = runs[0]
    with pytest.raises(fm.FmaskError) as ei:
        fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=scale, workspace=ws[: nbytes[0] - 16])
    assert ei.value.status == fm.ERR_CAPACITY
