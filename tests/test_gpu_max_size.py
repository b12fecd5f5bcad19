"""The largest key range the bf16 interval kernels accept, through the C ABI.

The kernels address one (batch, K/V head) of K and V with 32-bit buffer
offsets, so the launcher accepts skv with (skv + 64) * 2 * D <= 2^31 - 1:
skv = 8,388,543 at D = 128, K and V 2 GiB each.  A band anchored at the lower
right corner (pre 100, next 0; Ascend sparseMode page, band and rightDownCausal)
over 200 queries makes only the last tiles visible, at byte offsets just
under 2^31, while every other K and V row holds NaN: a tile loaded or an
offset computed wrongly shows in the output.  The expected values come from
the float64 oracle on the last 512 keys with the same band, which has the same
visibility relative to the lower-right corner.  Forward on the 128-, 64- and
256-row interval tables and the backward (dK, dV exactly zero outside the band).
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as OA
from tests.helpers import compare, to_device, to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fm = pytest.importorskip("mask_aware_block_amd")

D = 128
SKV = (2 ** 31 - 1) // (2 * D) - 64  # 8,388,543: the launcher's limit at D = 128
SQ, TAIL, PRE = 200, 512, 100


def _problem():
    w = dict(name="max_size", seed=61, B=1, Hq=2, Hkv=1, Sq=SQ, Skv=TAIL, D=D, dtype="bf16",
             scale=1 / math.sqrt(D))
    arrays = synth.draw_qkv(w)  # Q and the last TAIL keys
    q, k_tail, v_tail = to_device(w, arrays)
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device="cuda")
    k = nan.expand(1, 1, SKV, D).contiguous()
    v = nan.expand(1, 1, SKV, D).contiguous()
    k[:, :, SKV - TAIL:] = k_tail
    v[:, :, SKV - TAIL:] = v_tail
    spec = dict(family="band", sq=SQ, skv=SKV, pre=PRE, next=0)
    tail_spec = dict(family="band", sq=SQ, skv=TAIL, pre=PRE, next=0)
    return w, arrays, q, k, v, spec, tail_spec


def test_largest_key_range_forward_and_backward():
    w, arrays, q, k, v, spec, tail_spec = _problem()
    enc = fm.encode(spec)
    assert enc.kind == fm.ENC_INTERVALS
    qq, kk, vv = (to_f64(w, a) for a in arrays)
    ro, rl = OA.attention_dense(qq, kk, vv, OA.spec_vis_fn(tail_spec), w["scale"])
    for bm in (128, 64, 256):
        tiles = fm.classify(enc, bm, 64)
        o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
        torch.cuda.synchronize()
        compare(w, o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"skv {SKV} bm {bm}")

    # backward on the 128-row table
    do_bits = synth.draw_dout(w)
    do = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).cuda()
    tiles = fm.classify(enc, 128, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    dq, dk, dv = fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    rq, rk, rv = OA.attention_backward_dense(qq, kk, vv, to_f64(w, do_bits), OA.spec_vis_fn(tail_spec),
                                             w["scale"])
    for name, got, ref in (("dq", dq, rq), ("dk", dk[:, :, SKV - TAIL:], rk), ("dv", dv[:, :, SKV - TAIL:], rv)):
        g = got.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all(), f"{name} not finite"
        scale = max(np.abs(ref).max(), 1e-6)
        err = np.abs(g - ref)
        assert err.max() <= 2e-2 * scale, f"{name} max err {err.max():.3e} (ref max {scale:.3e})"
        assert err.mean() <= 2e-3 * scale, f"{name} mean err {err.mean():.3e}"
    assert int(torch.count_nonzero(dk[:, :, :SKV - TAIL]).item()) == 0
    assert int(torch.count_nonzero(dv[:, :, :SKV - TAIL]).item()) == 0


def test_one_key_more_is_refused():
    """skv one past the limit: FMASK_ERR_UNSUPPORTED before any launch."""
    spec = dict(family="band", sq=8, skv=SKV + 1, pre=PRE, next=0)
    enc = fm.encode(spec)
    tiles = fm.classify(enc, 128, 64)
    q = torch.zeros(1, 1, 8, D, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(1, 1, SKV + 1, D, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    with pytest.raises(fm.FmaskError, match="2 GiB"):
        fm.attn_fwd(q, kv, kv, enc, tiles, out=out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
