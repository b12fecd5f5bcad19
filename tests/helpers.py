"""Shared test helpers: move synth arrays to the device, compare with the oracle."""

import numpy as np

from oracle import attention as OA
from oracle import encode as OE
from oracle import masks as OM

# Agreement targets: fp32 inputs max abs <= 1e-5; bf16 inputs with fp32
# accumulation max abs <= 2e-2 and mean abs <= 1e-3 (against the float64 oracle
# run on the same bf16-rounded inputs).  LSE (no target is stated for it):
# fp32 1e-5; bf16 2^-8 + 5e-4: the bf16 kernel sums the bf16-rounded
# probabilities it multiplies into V (so O is normalised exactly by what it
# accumulated), and a bf16 rounding moves each term by at most 2^-8 relative,
# hence log(l) by at most 2^-8; fp32 score and log rounding add < 5e-4.
TOL = {"f32": dict(max_abs=1e-5, mean_abs=1e-5, lse=1e-5),
       "bf16": dict(max_abs=2e-2, mean_abs=1e-3, lse=2.0 ** -8 + 5e-4)}


# Gradient checks bound the error relative to the largest reference value of
# each tensor, that scale floored at GRAD_SCALE_FLOOR.  Where the exact gradient
# is zero by cancellation (a row with one visible key has dS = P (dP - D) = 0:
# dP_ij and D_i are the same dot product of dO with V_j = O_i), the kernel's
# fp32 dP and D, sums of D products of bf16 values, differ by rounding noise of
# up to about D 2^-24 max|dO| max|V|, times scale max|K| in dQ (~1e-4 at
# D = 128 for N(0,1) data).  The floor admits that noise (2e-2 x 5e-3 = 1e-4 max
# abs, 1e-5 mean abs), still inside the absolute bf16 bound of 2e-2 / 1e-3.
GRAD_SCALE_FLOOR = 5e-3


def to_device(w, arrays, device="cuda"):
    import torch
    q, k, v = arrays
    if w["dtype"] == "bf16":
        conv = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    else:
        conv = lambda a: torch.from_numpy(a).to(device)
    return conv(q), conv(k), conv(v)


def to_f64(w, a):
    return OA.bf16_bits_to_f64(a) if w["dtype"] == "bf16" else np.asarray(a, dtype=np.float64)


def compare(w, o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    """Assert the GPU output within the tolerance of the float64 oracle."""
    tol = TOL[w["dtype"]]
    o = np.asarray(o_gpu, dtype=np.float64)
    err = np.abs(o - o_ref)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert err.max() <= tol["max_abs"], f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= tol["mean_abs"], f"{what}: mean abs err {err.mean():.3e}"
    lg = np.asarray(lse_gpu, dtype=np.float64)
    inf_ref = np.isneginf(lse_ref)
    assert (np.isneginf(lg) == inf_ref).all(), f"{what}: empty-row LSE mismatch"
    if (~inf_ref).any():
        le = np.abs(lg[~inf_ref] - lse_ref[~inf_ref]).max()
        assert le <= tol["lse"], f"{what}: LSE err {le:.3e}"
    assert (o[inf_ref] == 0).all(), f"{what}: empty rows must be exactly zero"
    return float(err.max()), float(err.mean())


def sample_rows(w, n, rng, extra=()):
    """(b, h, i) samples: random rows plus edge rows."""
    B, Hq, Sq = w["B"], w["Hq"], w["Sq"]
    s = {(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(Sq))) for _ in range(n)}
    for i in (0, 1, Sq - 1, Sq // 2) + tuple(extra):
        if 0 <= i < Sq:
            s.add((int(rng.integers(B)), int(rng.integers(Hq)), int(i)))
    return sorted(s)
