"""No-allocation split form (fmask_attn_fwd_split_noalloc) through the C ABI.

The entry point runs the kernels of fmask_attn_fwd_split with the partial
states in the library's per-GPU scratch instead of a caller workspace, so its
output must be bit-identical to fmask_attn_fwd_split's on the same inputs and
split count.  Checked on two calls in a row, the second one smaller (the
scratch keeps the first call's contents), both also against the float64
oracle over the listed cells; and a problem whose partial states exceed the
scratch must be refused before any launch.
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as OA
from tests.helpers import compare, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fm = pytest.importorskip("mask_aware_block_amd")


def _workload(Sq, Skv, D, Hq, Hkv, seed):
    w = dict(name="decode", seed=seed, B=1, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D, dtype="bf16",
             scale=1 / math.sqrt(D))
    rng = synth.streams(seed)[3]
    sel = synth.selected_lists(rng, Sq, -(-Skv // 32), edge_rows=Sq >= 3)
    w["mask"] = dict(family="selected_key", sq=Sq, skv=Skv, batch=1, sel=sel[None], sel_cells=32)
    return w


def _one(w, splits):
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(w["mask"])
    o_ref, l_ref = fm.attn_fwd_split(q, k, v, enc, splits=splits, scale=w["scale"])
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    fm.attn_fwd_split_noalloc(q, k, v, enc, splits=splits, scale=w["scale"], out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "O differs from the workspace split form"
    assert torch.equal(lse, l_ref), "LSE differs from the workspace split form"
    samples = [(0, h, i) for h in range(w["Hq"]) for i in range(w["Sq"])]
    ro, rl = OA.attention_listed_cells(*arrays, w["mask"]["sel"], 32, w["scale"], samples,
                                       decode=OA.bf16_bits_to_f64)
    got_o = np.stack([o[0, h, i].float().cpu().numpy() for (_, h, i) in samples])
    got_l = np.array([lse[0, h, i].item() for (_, h, i) in samples])
    compare(w, got_o, got_l, ro, rl, f"noalloc splits {splits} Sq {w['Sq']}")


def test_noalloc_matches_workspace_form_twice_smaller_second():
    print("noalloc: call 1 (Sq 16, Skv 8192, D 256, GQA 4, automatic splits)", flush=True)
    _one(_workload(16, 8192, 256, 32, 8, 51), splits=0)
    print("noalloc: call 2 (Sq 1, Skv 4113, D 128, GQA 8, 3 splits)", flush=True)
    _one(_workload(1, 4096 + 17, 128, 16, 2, 52), splits=3)


def test_noalloc_refuses_more_than_its_scratch():
    w = _workload(64, 2048, 256, 32, 8, 53)
    q, k, v = to_device(w, synth.draw_qkv(w))
    enc = fm.encode(w["mask"])
    need = fm.lib().fmask_attn_split_workspace_bytes(
        __import__("ctypes").byref(fm.attn_args(q, k, v, q, w["scale"])),
        __import__("ctypes").byref(enc.struct), 64)
    assert need > fm.SPLIT_SCRATCH_BYTES
    o = torch.zeros_like(q)
    with pytest.raises(fm.FmaskError) as ei:
        fm.attn_fwd_split_noalloc(q, k, v, enc, splits=64, scale=w["scale"], out=o)
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert not o.any(), "a refused call wrote its output"
