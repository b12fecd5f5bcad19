"""Every output row of full-size workloads, at the bf16 tolerance.

The float64 oracle checks full-size workloads on sampled rows
(test_gpu_attention.py).  This test covers all rows: the mask rows come from
the oracle's visibility function (oracle.masks.dense_vis, chunk by chunk), and
the scores, softmax and P V are evaluated by plain PyTorch fp32 operations on
the GPU (rocBLAS matrix products, not this library's kernels), one chunk of
query rows and one K/V head group at a time.  The library's O and LSE must
agree with it within the same bounds as against the oracle (O max abs 2e-2,
mean abs 1e-3; LSE 2^-8 + 5e-4; rows with no visible key exactly zero with
LSE = -inf).
"""

import numpy as np
import pytest

import synth
from oracle import masks as OM
from tests.helpers import GRAD_SCALE_FLOOR, TOL, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fm = pytest.importorskip("mask_aware_block_amd")

WORKLOADS = ["causal_doc_32k", "shared_question_32k", "band_32k", "varlen_prefill_32k", "tree_4k",
             "block_bitmap_16k", "selected_key_128k"]
CHUNK = 1024


def _reference_chunk(q, k, v, vis, scale, G):
    """fp32 O [Hq, R, D] and LSE [Hq, R] of rows q [Hq, R, D] against k, v [Hkv, Skv, D] under vis [R, Skv]."""
    Hq = q.shape[0]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    masked = ~vis
    for g in range(Hq // G):
        s = torch.matmul(q[g * G:(g + 1) * G], k[g].t().contiguous()) * scale  # [G, R, Skv]
        s.masked_fill_(masked, float("-inf"))
        m = torch.logsumexp(s, dim=-1)  # -inf for rows with no visible key
        p = torch.exp(s - m[..., None])
        p = torch.nan_to_num(p, nan=0.0)
        o[g * G:(g + 1) * G] = torch.matmul(p, v[g])
        lse[g * G:(g + 1) * G] = m
        del s, p
    return o, lse


@pytest.mark.parametrize("name", WORKLOADS)
def test_every_row_full_size(name):
    w = synth.workload(name)
    spec = w["mask"]
    assert spec.get("heads", 1) == 1  # one mask slice per batch entry, shared by the heads
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(spec)
    if enc.kind == fm.ENC_SELECTED:  # the per-query walk and the block-major form
        forms = [("one-pass", *fm.attn_fwd(q, k, v, enc, None, scale=w["scale"])),
                 ("block-major", *fm.attn_fwd_blocks(q, k, v, enc, scale=w["scale"]))]
    else:
        forms = [("tiles", *fm.attn_fwd(q, k, v, enc, fm.classify(enc), scale=w["scale"]))]
    torch.cuda.synchronize()
    G = w["Hq"] // w["Hkv"]
    tol = TOL["bf16"]
    worst = {f[0]: 0.0 for f in forms}
    total = {f[0]: 0.0 for f in forms}
    n = 0
    fp32 = {}
    for b, r0 in ((b, r0) for b in range(w["B"]) for r0 in range(0, w["Sq"], CHUNK)):
        if b not in fp32:
            fp32 = {b: tuple(t[b].float().contiguous() for t in (q, k, v))}
        qf, kf, vf = fp32[b]
        rows = np.arange(r0, min(w["Sq"], r0 + CHUNK))
        vis = torch.from_numpy(np.array(OM.dense_vis(spec, b, 0, rows), dtype=bool)).cuda()
        ro, rl = _reference_chunk(qf[:, r0:r0 + len(rows)], kf, vf, vis, w["scale"], G)
        empty = torch.isneginf(rl)
        n += ro.numel()
        for form, o, lse in forms:
            what = f"{name} ({form}) batch {b} rows {r0}.."
            go = o[b, :, r0:r0 + len(rows)].float()
            gl = lse[b, :, r0:r0 + len(rows)]
            err = (go - ro).abs()
            worst[form] = max(worst[form], float(err.max()))
            total[form] += float(err.sum())
            assert bool((torch.isneginf(gl) == empty).all()), f"{what}: empty-row LSE mismatch"
            assert bool((go[empty] == 0).all()), f"{what}: empty rows must be exactly zero"
            if bool((~empty).any()):
                le = float((gl[~empty] - rl[~empty]).abs().max())
                assert le <= tol["lse"], f"{what}: LSE err {le:.3e}"
            assert worst[form] <= tol["max_abs"], f"{what}: max abs err {worst[form]:.3e}"
    for form, _, _ in forms:
        assert total[form] / n <= tol["mean_abs"], f"{name} ({form}): mean abs err {total[form] / n:.3e}"
        print(f"{name} ({form}): every row, max abs {worst[form]:.3e}, mean abs {total[form] / n:.3e}")


def _reference_backward(q, k, v, do, spec, b, scale, G):
    """fp32 dQ [Hq, Sq, D], dK and dV [Hkv, Skv, D] of one batch entry from the
    definition: P = softmax(scale Q K^T) on visible cells, O = P V,
    D_i = sum_d dO_id O_id, dS = P (dO V^T - D); dQ = scale dS K,
    dK = scale dS^T Q, dV = P^T dO (dK, dV summed over each group's heads)."""
    Hq, Sq, _ = q.shape
    dq = torch.empty_like(q)
    dk = torch.zeros_like(k)
    dv = torch.zeros_like(v)
    for r0 in range(0, Sq, CHUNK):
        rows = np.arange(r0, min(Sq, r0 + CHUNK))
        masked = ~torch.from_numpy(np.array(OM.dense_vis(spec, b, 0, rows), dtype=bool)).cuda()
        for g in range(Hq // G):
            qc = q[g * G:(g + 1) * G, r0:r0 + len(rows)]
            dc = do[g * G:(g + 1) * G, r0:r0 + len(rows)]
            s = torch.matmul(qc, k[g].t().contiguous()) * scale
            s.masked_fill_(masked, float("-inf"))
            p = torch.nan_to_num(torch.exp(s - torch.logsumexp(s, dim=-1, keepdim=True)), nan=0.0)
            del s
            o = torch.matmul(p, v[g])
            ds = p * (torch.matmul(dc, v[g].t().contiguous()) - (dc * o).sum(-1, keepdim=True))
            dq[g * G:(g + 1) * G, r0:r0 + len(rows)] = scale * torch.matmul(ds, k[g])
            dk[g] += scale * torch.matmul(ds.transpose(1, 2).contiguous(), qc).sum(0)
            dv[g] += torch.matmul(p.transpose(1, 2).contiguous(), dc).sum(0)
            del p, ds, o
    return dq, dk, dv


@pytest.mark.parametrize("name", ["causal_doc_32k", "shared_question_32k", "tree_4k", "block_bitmap_16k"])
def test_backward_every_row_full_size(name):
    """dQ, dK and dV of every row and key at full size, against the fp32
    evaluation above, within the backward's bounds (max abs 2e-2 and mean abs
    2e-3 of the largest reference magnitude, as in the other backward tests);
    the last two workloads have bitmap masks (one per batch entry for the
    block pattern)."""
    w = synth.workload(name)
    spec = w["mask"]
    assert spec.get("heads", 1) == 1
    q, k, v = to_device(w, synth.draw_qkv(w))
    do = torch.from_numpy(synth.draw_dout(w).view(np.int16)).view(torch.bfloat16).cuda()
    enc = fm.encode(spec)
    tiles = fm.classify(enc, 128, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    dq, dk, dv = fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    G = w["Hq"] // w["Hkv"]
    stats = {}
    for b in range(w["B"]):
        ref = _reference_backward(*(t[b].float().contiguous() for t in (q, k, v, do)), spec, b, w["scale"], G)
        for what, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
            g = got[b].float()
            assert bool(torch.isfinite(g).all()), f"{name} batch {b}: {what} not finite"
            mag = max(float(r.abs().max()), GRAD_SCALE_FLOOR)
            err = (g - r).abs()
            stats[(b, what)] = (float(err.max()) / mag, float(err.mean()) / mag)
            assert float(err.max()) <= 2e-2 * mag, f"{name} batch {b}: {what} max abs err {float(err.max()):.3e}"
            assert float(err.mean()) <= 2e-3 * mag, f"{name} batch {b}: {what} mean abs err {float(err.mean()):.3e}"
    for what in ("dq", "dk", "dv"):
        worst = max(v[0] for key, v in stats.items() if key[1] == what)
        print(f"{name} {what}: worst max abs {worst:.2e} of the largest reference gradient")
