"""Pins of the float64 attention oracle against things other than itself.

- scalar brute force (pure Python loops) on tiny shapes;
- torch.nn.functional.scaled_dot_product_attention in float64 on the CPU (a
  library routine) on rows with at least one visible key;
- closed forms: Q = 0 gives the mean of the visible V rows, constant V gives
  the constant, a single visible key gives its V row, one-hot V gives P;
- scipy.special.logsumexp for the LSE;
- invariants: rows of P sum to 1, GQA equals MHA with repeated K/V, permuting
  keys together with the mask columns changes nothing, empty rows are zero.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as A
from oracle import masks as M


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _random_vis(rng, sq, skv, p=0.5):
    vis = rng.random((sq, skv)) < p
    vis[0] = False  # an empty row
    return vis


def test_bruteforce_matches_vectorised():
    rng = np.random.default_rng(1)
    for sq, skv, d in [(1, 1, 1), (5, 7, 3), (17, 24, 8), (24, 24, 16)]:
        q, k, v = _rand(rng, sq, d), _rand(rng, skv, d), _rand(rng, skv, d)
        vis = _random_vis(rng, sq, skv)
        scale = 1 / math.sqrt(d)
        ob, lb = A.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), vis.tolist(), scale)
        o, l = A.attention_dense(q[None, None], k[None, None], v[None, None],
                                 lambda b, h, rows: vis[rows], scale)
        np.testing.assert_allclose(o[0, 0], ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(np.isinf(l[0, 0]), np.isinf(lb))
        fin = np.isfinite(lb)
        np.testing.assert_allclose(l[0, 0][fin], lb[fin], rtol=1e-12, atol=1e-12)


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(2)
    B, Hq, Hkv, sq, skv, d = 2, 4, 2, 40, 56, 16
    q, k, v = _rand(rng, B, Hq, sq, d), _rand(rng, B, Hkv, skv, d), _rand(rng, B, Hkv, skv, d)
    vis = rng.random((B, Hq, sq, skv)) < 0.3
    vis[:, :, 3] = False
    scale = 0.37
    o, lse = A.attention_dense(q, k, v, lambda b, h, rows: vis[b, h, rows], scale, row_chunk=16)
    G = Hq // Hkv
    kt = torch.from_numpy(np.repeat(k, G, axis=1))
    vt = torch.from_numpy(np.repeat(v, G, axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kt, vt, attn_mask=torch.from_numpy(vis), scale=scale).numpy()
    rows = vis.any(-1)
    np.testing.assert_allclose(o[rows], ref[rows], rtol=1e-11, atol=1e-12)
    assert np.all(o[~rows] == 0.0) and np.all(np.isneginf(lse[~rows]))
    s = scale * np.einsum("bhid,bhjd->bhij", q, np.repeat(k, G, axis=1))
    ref_lse = scipy.special.logsumexp(np.where(vis, s, -np.inf), axis=-1)
    np.testing.assert_allclose(lse[rows], ref_lse[rows], rtol=1e-12, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(3)
    sq, skv, d = 33, 45, 8
    vis = _random_vis(rng, sq, skv, 0.4)
    vf = lambda b, h, rows: vis[rows]
    k, v = _rand(rng, 1, 1, skv, d), _rand(rng, 1, 1, skv, d)
    # Q = 0: uniform weights over the visible set -> mean of the visible V rows;
    # LSE = log |V_i| exactly.
    o, lse = A.attention_dense(np.zeros((1, 1, sq, d)), k, v, vf, 0.5)
    for i in range(sq):
        n = vis[i].sum()
        if n:
            np.testing.assert_allclose(o[0, 0, i], v[0, 0][vis[i]].mean(axis=0), rtol=1e-13, atol=1e-14)
            assert abs(lse[0, 0, i] - math.log(n)) < 1e-13
        else:
            assert np.all(o[0, 0, i] == 0) and lse[0, 0, i] == -np.inf
    # constant V -> the constant on every non-empty row
    q = _rand(rng, 1, 1, sq, d)
    o, _ = A.attention_dense(q, k, np.full((1, 1, skv, d), 2.5), vf, 0.5)
    ne = vis.any(1)
    np.testing.assert_allclose(o[0, 0][ne], 2.5, rtol=1e-14)
    # a single visible key j -> exactly V_j, LSE = s_ij
    one = np.zeros((sq, skv), dtype=bool)
    js = rng.integers(0, skv, sq)
    one[np.arange(sq), js] = True
    o, lse = A.attention_dense(q, k, v, lambda b, h, rows: one[rows], 0.5)
    np.testing.assert_array_equal(o[0, 0], v[0, 0][js])
    np.testing.assert_allclose(lse[0, 0], 0.5 * np.einsum("id,id->i", q[0, 0], k[0, 0][js]), rtol=1e-14)


def test_probabilities_sum_to_one_and_match_softmax():
    rng = np.random.default_rng(4)
    sq, skv = 20, 16
    vis = _random_vis(rng, sq, skv, 0.6)
    q, k = _rand(rng, 1, 1, sq, 8), _rand(rng, 1, 1, skv, 8)
    eye = np.eye(skv)[None, None]  # one-hot V rows: O_i = P_i
    p, _ = A.attention_dense(q, k, eye, lambda b, h, rows: vis[rows], 0.25)
    ne = vis.any(1)
    np.testing.assert_allclose(p[0, 0][ne].sum(axis=1), 1.0, atol=1e-15)
    assert np.all(p[0, 0][~vis] == 0.0)
    s = 0.25 * q[0, 0] @ k[0, 0].T
    ref = scipy.special.softmax(np.where(vis, s, -np.inf)[ne], axis=1)
    np.testing.assert_allclose(p[0, 0][ne], ref, rtol=1e-13, atol=1e-16)


def test_gqa_equals_repeated_mha_and_key_permutation():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, sq, skv, d = 1, 6, 2, 24, 30, 8
    q, k, v = _rand(rng, B, Hq, sq, d), _rand(rng, B, Hkv, skv, d), _rand(rng, B, Hkv, skv, d)
    vis = _random_vis(rng, sq, skv)
    vf = lambda b, h, rows: vis[rows]
    o1, l1 = A.attention_dense(q, k, v, vf, 0.3)
    o2, l2 = A.attention_dense(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), vf, 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # head h reads K/V head h // 3: changing K/V head 1 leaves heads 0..2 untouched
    k2 = k.copy()
    k2[:, 1] += rng.standard_normal(k2[:, 1].shape)
    o3, _ = A.attention_dense(q, k2, v, vf, 0.3)
    np.testing.assert_array_equal(o3[:, :3], o1[:, :3])
    assert not np.allclose(o3[:, 3:], o1[:, 3:])
    perm = rng.permutation(skv)
    o4, l4 = A.attention_dense(q, k[:, :, perm], v[:, :, perm], lambda b, h, rows: vis[rows][:, perm], 0.3)
    np.testing.assert_allclose(o4, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l4[np.isfinite(l1)], l1[np.isfinite(l1)], rtol=1e-13)


def test_attention_rows_equals_dense():
    rng = np.random.default_rng(6)
    B, Hq, Hkv, sq, skv, d = 2, 4, 2, 50, 70, 8
    q, k, v = _rand(rng, B, Hq, sq, d), _rand(rng, B, Hkv, skv, d), _rand(rng, B, Hkv, skv, d)
    spec = dict(family="band", sq=sq, skv=skv, pre=5, next=-2)
    vf = A.spec_vis_fn(spec)
    o, l = A.attention_dense(q, k, v, vf, 0.4)
    samples = [(1, 3, 0), (0, 1, 49), (1, 2, 17), (0, 0, 1)]
    so, sl = A.attention_rows(q, k, v, vf, 0.4, samples)
    for n, (b, h, i) in enumerate(samples):
        np.testing.assert_allclose(so[n], o[b, h, i], rtol=1e-13, atol=1e-15)
        assert (sl[n] == l[b, h, i]) or abs(sl[n] - l[b, h, i]) < 1e-13


def test_listed_cells_equals_dense_union_and_dedup():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, sq, skv, d, cells = 1, 4, 1, 12, 100, 8, 32  # 4 blocks, the last one ragged
    q, k, v = _rand(rng, B, Hq, sq, d), _rand(rng, B, Hkv, skv, d), _rand(rng, B, Hkv, skv, d)
    sel = rng.integers(-2, 6, size=(1, sq, 5)).astype(np.int32)  # invalid -2, -1, 4, 5
    sel[0, 0] = -1
    sel[0, 1] = [3, 3, 3, 3, 3]
    spec = dict(family="selected_key", sq=sq, skv=skv, sel=sel, sel_cells=cells)
    o, l = A.attention_dense(q, k, v, A.spec_vis_fn(spec), 0.35)
    samples = [(0, h, i) for h in range(Hq) for i in range(sq)]
    so, sl = A.attention_listed_cells(q, k, v, sel, cells, 0.35, samples)
    for n, (b, h, i) in enumerate(samples):
        np.testing.assert_allclose(so[n], o[b, h, i], rtol=1e-12, atol=1e-14)
    assert np.all(so[:sq][0] == 0) and sl[0] == -np.inf
    # duplicates count once: a de-duplicated list gives the same rows
    dedup = np.array([sorted(set(r.tolist())) + [-1] * (5 - len(set(r.tolist()))) for r in sel[0]])[None]
    so2, _ = A.attention_listed_cells(q, k, v, dedup, cells, 0.35, samples)
    np.testing.assert_allclose(so2, so, rtol=1e-14, atol=0)
    # row 1 lists only block 3 = cells 96..99 (ragged last block)
    assert M.dense_vis(spec, 0, 0, np.array([1]))[0].nonzero()[0].tolist() == [96, 97, 98, 99]


def test_bf16_bits_conversion():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F80], dtype=np.uint16)
    vals = A.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[3] == 0.0 and vals[5] == np.inf
    assert vals[2] == 3.140625
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(vals, t)
