"""Pins of the oracle's attention gradient (oracle.attention.attention_backward_dense).

The gradient is pinned to things other than its own formula:
  * torch autograd (float64, CPU) through a plain masked-softmax forward: a
    derivation by the library, not by the closed form;
  * central finite differences of the oracle's own forward (attention_dense)
    along random directions, for Q, K and V;
  * invariants: sum over keys of dK is zero (each row of dS sums to zero);
    rows with no visible key contribute nothing; the gradient is linear in dO.
"""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import masks as OM

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(seed, B=2, Hq=4, Hkv=2, S=29, K=41, D=8, dens=0.45):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D))
    k = rng.standard_normal((B, Hkv, K, D))
    v = rng.standard_normal((B, Hkv, K, D))
    do = rng.standard_normal((B, Hq, S, D))
    vis = rng.random((B, Hq, S, K)) < dens
    vis[0, 1, 5] = False  # an empty row
    fn = lambda b, h, rows: vis[b, h, rows]
    return q, k, v, do, vis, fn


def test_matches_torch_autograd():
    q, k, v, do, vis, fn = _case(1)
    scale = 0.37
    dq, dk, dv = OA.attention_backward_dense(q, k, v, do, fn, scale, row_chunk=7)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    G = q.shape[1] // k.shape[1]
    kk = tk.repeat_interleave(G, dim=1)
    vv = tv.repeat_interleave(G, dim=1)
    s = scale * (tq @ kk.transpose(-1, -2))
    s = s.masked_fill(~torch.tensor(vis), float("-inf"))
    p = torch.nan_to_num(torch.softmax(s, dim=-1), nan=0.0)
    ((p @ vv) * torch.tensor(do)).sum().backward()
    assert np.abs(tq.grad.numpy() - dq).max() < 1e-12
    assert np.abs(tk.grad.numpy() - dk).max() < 1e-12
    assert np.abs(tv.grad.numpy() - dv).max() < 1e-12


def test_finite_differences_of_the_forward():
    q, k, v, do, vis, fn = _case(2, B=1, Hq=2, Hkv=1, S=9, K=11, D=4)
    scale = 0.5
    dq, dk, dv = OA.attention_backward_dense(q, k, v, do, fn, scale)

    def loss(q_, k_, v_):
        o, _ = OA.attention_dense(q_, k_, v_, fn, scale)
        return float((o * do).sum())

    rng = np.random.default_rng(3)
    eps = 1e-6
    for _ in range(3):
        uq, uk, uv = (rng.standard_normal(a.shape) for a in (q, k, v))
        fd_q = (loss(q + eps * uq, k, v) - loss(q - eps * uq, k, v)) / (2 * eps)
        fd_k = (loss(q, k + eps * uk, v) - loss(q, k - eps * uk, v)) / (2 * eps)
        fd_v = (loss(q, k, v + eps * uv) - loss(q, k, v - eps * uv)) / (2 * eps)
        assert abs(fd_q - (dq * uq).sum()) < 1e-6
        assert abs(fd_k - (dk * uk).sum()) < 1e-6
        assert abs(fd_v - (dv * uv).sum()) < 1e-6


def test_invariants():
    q, k, v, do, vis, fn = _case(4)
    dq, dk, dv = OA.attention_backward_dense(q, k, v, do, fn, 0.25)
    # each row of dS sums to zero, hence dK summed over keys vanishes
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    # the empty row has no gradient, and adds nothing to dK / dV
    assert np.abs(dq[0, 1, 5]).max() == 0.0
    do2 = do.copy()
    do2[0, 1, 5] = 1e3
    dq2, dk2, dv2 = OA.attention_backward_dense(q, k, v, do2, fn, 0.25)
    assert np.abs(dk2 - dk).max() < 1e-12 and np.abs(dv2 - dv).max() < 1e-12
    # linear in dO
    dqa, dka, dva = OA.attention_backward_dense(q, k, v, 2.5 * do, fn, 0.25)
    assert np.abs(dqa - 2.5 * dq).max() < 1e-12 and np.abs(dva - 2.5 * dv).max() < 1e-12


def test_causal_family_mask_matches_torch_causal_sdpa_gradient():
    # a family mask through the spec path: causal == torch's is_causal SDPA
    rng = np.random.default_rng(5)
    S, D = 33, 16
    q, k, v, do = (rng.standard_normal((1, 1, S, D)) for _ in range(4))
    spec = {"family": "causal", "sq": S, "skv": S}
    dq, dk, dv = OA.attention_backward_dense(q, k, v, do, OA.spec_vis_fn(spec), 1 / 4)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=1 / 4)
    (o * torch.tensor(do)).sum().backward()
    assert np.abs(tq.grad.numpy() - dq).max() < 1e-12
    assert np.abs(tk.grad.numpy() - dk).max() < 1e-12
    assert np.abs(tv.grad.numpy() - dv).max() < 1e-12


@pytest.mark.parametrize("seed", [4, 5, 6])
def test_sampled_gradient_matches_the_dense_one(seed):
    """attention_backward_sampled against the pinned dense gradient at every
    sampled row and key, per batch entry (random masks with an empty row and
    unseen keys, GQA 2)."""
    q, k, v, do, vis, fn = _case(seed)
    vis[1, :, :, 7] = False  # a key that no row sees
    scale = 0.41
    dq, dk, dv = OA.attention_backward_dense(q, k, v, do, fn, scale, row_chunk=6)
    rng = np.random.default_rng(seed)
    for b in range(q.shape[0]):
        rows = np.sort(rng.choice(q.shape[2], 9, replace=False))
        keys = np.sort(np.append(rng.choice(k.shape[2], 6, replace=False), 7))
        sq, sk, sv = OA.attention_backward_sampled(q, k, v, do, fn, scale, b, rows, keys, row_chunk=5)
        assert np.abs(sq - dq[b][:, rows]).max() < 1e-12
        assert np.abs(sk - dk[b][:, keys]).max() < 1e-12
        assert np.abs(sv - dv[b][:, keys]).max() < 1e-12
    assert np.abs(OA.attention_backward_sampled(q, k, v, do, fn, scale, 1, [], [7])[1]).max() == 0.0
