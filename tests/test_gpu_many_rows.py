"""Forward and backward over 19.2M query rows: B = 1, Hq = 64 over one K/V
head, Sq = 300,032 (150,016 query-tile items per launch).

The backward's dQ kernel forms every row's D_i = sum_d dO_id O_id and LSE_i
log2(e) in its prologue and leaves them in the workspace, 8 bytes per
(batch, query head, row), for the dK/dV kernel, which sums over all 64 query
heads of the K/V head; a row term lost or misplaced anywhere in that range
shows in dK and dV of its document.

The mask packs 4,688 documents of 64 tokens, causal inside each (FlashMask
rebuttal, causal document mask), so each document is an independent 64 x 64
causal problem: the float64 oracle (attention_dense, attention_backward_dense)
runs on single documents, every head, and its O, LSE, dQ, dK and dV are compared
with the GPU's over those documents.  Q, K, V and dO are N(0, 1), drawn on the
device from a seeded generator in bf16 (the oracle gets the same values back).
"""

import math

import numpy as np
import pytest

from oracle import attention as OA
from tests.helpers import GRAD_SCALE_FLOOR, TOL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fm = pytest.importorskip("mask_aware_block_amd")

DOC, NDOC, HQ, D = 64, 4688, 64, 128
S = DOC * NDOC
# bf16 gradients with fp32 accumulation, relative to the largest reference
# magnitude of each tensor (the same bound as the other backward tests).
GRAD_TOL = dict(max_rel=2e-2, mean_rel=2e-3)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_many_rows_forward_and_backward():
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20240)
    draw = lambda *shape: torch.randn(*shape, generator=gen, device="cuda", dtype=torch.bfloat16)
    q, k, v, do = draw(1, HQ, S, D), draw(1, 1, S, D), draw(1, 1, S, D), draw(1, HQ, S, D)
    spec = dict(family="causal_document", sq=S, skv=S, cu_seg=np.arange(0, S + 1, DOC, dtype=np.int32))
    scale = 1 / math.sqrt(D)
    enc = fm.encode(spec)
    tiles = fm.classify(enc, 128, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=scale)
    dq, dk, dv = fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=scale)
    torch.cuda.synchronize()

    # documents at both ends, around the middle, and seeded others; every head
    rng = np.random.default_rng(5)
    docs = sorted({0, 1, NDOC // 2, NDOC - 2, NDOC - 1} | {int(x) for x in rng.choice(NDOC, 4, replace=False)})
    vis = OA.spec_vis_fn(dict(family="causal", sq=DOC, skv=DOC))
    tol = TOL["bf16"]
    for d in docs:
        r = slice(d * DOC, (d + 1) * DOC)
        qd, kd, vd, dod = (_f64(t[:, :, r]) for t in (q, k, v, do))
        ro, rl = OA.attention_dense(qd, kd, vd, vis, scale)
        oe = np.abs(_f64(o[:, :, r]) - ro)
        le = np.abs(lse[:, :, r].cpu().numpy().astype(np.float64) - rl).max()
        assert oe.max() <= tol["max_abs"] and oe.mean() <= tol["mean_abs"], f"doc {d}: O err {oe.max():.3e}"
        assert le <= tol["lse"], f"doc {d}: LSE err {le:.3e}"
        rq, rk, rv = OA.attention_backward_dense(qd, kd, vd, dod, vis, scale)
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            g = _f64(got[:, :, r])
            assert np.isfinite(g).all(), f"doc {d}: {name} not finite"
            ref_max = max(np.abs(ref).max(), GRAD_SCALE_FLOOR)
            err = np.abs(g - ref)
            assert err.max() <= GRAD_TOL["max_rel"] * ref_max, f"doc {d}: {name} max err {err.max():.3e}"
            assert err.mean() <= GRAD_TOL["mean_rel"] * ref_max, f"doc {d}: {name} mean err {err.mean():.3e}"
    print(f"{len(docs)} documents of {NDOC}, {HQ} heads ({HQ * S} rows): forward and backward within tolerance",
          flush=True)
