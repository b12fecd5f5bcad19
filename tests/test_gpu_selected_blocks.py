"""Block-major selected-key form, fmask_attn_fwd_blocks, through the C ABI.

The per-query block lists are inverted into, per 32-cell block, the (query,
entry) pairs that name it; each block's K and V are read once per K/V head and
scored against those queries' Q rows, and the per-entry partial states are
merged per query (the split-K merge of the selected-key PR).  Compared with
the float64 oracle over exactly the listed cells for every row: lists per
batch and shared by the batch, GQA groups of 1 to 16 query heads, a ragged
last block, queries with no valid entry, one block listed many times, all
blocks listed; the full 128K workload on sampled rows; bit-identical results
on a second call (the scatter's atomics order the pairs differently).
"""

import ctypes
import math

import numpy as np
import pytest

import synth
from oracle import attention as OA
from tests.helpers import compare, sample_rows, to_device, to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fm = pytest.importorskip("mask_aware_block_amd")


def _workload(B, Sq, Skv, D, Hq, Hkv, seed, per_batch, n=64):
    w = dict(name="blocks", seed=seed, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D, dtype="bf16",
             scale=1 / math.sqrt(D))
    rng = synth.streams(seed)[3]
    nblk = -(-Skv // 32)
    mb = B if per_batch else 1
    sel = np.stack([synth.selected_lists(rng, Sq, nblk, n=n) for _ in range(mb)])
    w["mask"] = dict(family="selected_key", sq=Sq, skv=Skv, batch=mb, sel=sel, sel_cells=32)
    return w


def _check_all_rows(w, what):
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(w["mask"])
    o, lse = fm.attn_fwd_blocks(q, k, v, enc, scale=w["scale"])
    torch.cuda.synchronize()
    qq, kk, vv = (to_f64(w, a) for a in arrays)
    ro, rl = OA.attention_dense(qq, kk, vv, OA.spec_vis_fn(w["mask"]), w["scale"])
    compare(w, o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, what)
    return q, k, v, enc, o, lse


@pytest.mark.parametrize("D", [256, 128])
def test_blocks_small_per_batch_lists(D):
    # rows 0..2 of each batch: no valid entry, one block 64 times, every block
    w = _workload(2, 40, 1000, D, 8, 2, 41, per_batch=True)
    _check_all_rows(w, f"blocks per-batch lists d{D}")


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 128), (8, 1, 256), (12, 1, 128), (16, 1, 256), (6, 3, 128)])
def test_blocks_gqa_groups_shared_lists(Hq, Hkv, D):
    # one list batch shared by two batches; ragged last block (skv = 777)
    w = _workload(2, 33, 777, D, Hq, Hkv, 43 + Hq, per_batch=False, n=24)
    _check_all_rows(w, f"blocks shared lists G {Hq // Hkv} d{D}")


def test_blocks_agree_with_one_pass_and_repeat_bit_identical():
    w = _workload(1, 300, 4096 + 64 + 5, 256, 32, 8, 47, per_batch=True)
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(w["mask"])
    ws = torch.empty(fm.attn_blocks_workspace_bytes(q, k, v, enc), dtype=torch.uint8, device="cuda")
    o1, l1 = fm.attn_fwd_blocks(q, k, v, enc, scale=w["scale"], workspace=ws)
    ws.fill_(0xA5)  # the workspace's contents on entry do not matter
    o2, l2 = fm.attn_fwd_blocks(q, k, v, enc, scale=w["scale"], workspace=ws)
    ob, lb = fm.attn_fwd(q, k, v, enc, None, scale=w["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert (o1.float() - ob.float()).abs().max().item() <= 2e-2
    fin = torch.isfinite(lb)
    assert torch.equal(torch.isfinite(l1), fin)
    assert (l1[fin] - lb[fin]).abs().max().item() <= 2.0 ** -8 + 5e-4
    samples = [(0, h, i) for h in (0, 5, 31) for i in range(w["Sq"])]
    ro, rl = OA.attention_listed_cells(*arrays, w["mask"]["sel"], 32, w["scale"], samples,
                                       decode=OA.bf16_bits_to_f64)
    idx = tuple(np.array(samples).T)
    compare(w, o1.float().cpu().numpy()[idx], l1.cpu().numpy()[idx], ro, rl, "blocks vs oracle, 4K")


def test_blocks_refuses_a_short_workspace():
    w = _workload(1, 16, 512, 128, 4, 1, 53, per_batch=True)
    q, k, v = to_device(w, synth.draw_qkv(w))
    enc = fm.encode(w["mask"])
    need = fm.attn_blocks_workspace_bytes(q, k, v, enc)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(fm.FmaskError, match="workspace"):
        fm.attn_fwd_blocks(q, k, v, enc, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_blocks_full_size_sampled():
    w = synth.workload("selected_key_128k")
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(w["mask"])
    o, lse = fm.attn_fwd_blocks(q, k, v, enc, scale=w["scale"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    samples = sample_rows(w, 96, rng, extra=(2, 3))
    ro, rl = OA.attention_listed_cells(*arrays, w["mask"]["sel"], w["mask"]["sel_cells"], w["scale"], samples,
                                       decode=OA.bf16_bits_to_f64)
    idx = tuple(np.array(samples).T)
    compare(w, o.float().cpu().numpy()[idx], lse.cpu().numpy()[idx], ro, rl, "selected_key_128k blocks")


def test_blocks_degenerate_sizes():
    """One key, one query; no key at all (every list empty: O = 0 and LSE =
    -inf, with no partial-state kernel launched); no query."""
    for sq, skv in ((5, 1), (1, 33)):
        _check_all_rows(_workload(1, sq, skv, 128, 4, 2, 59 + skv, per_batch=True, n=8), f"blocks sq {sq} skv {skv}")
    # no key, and no query: empty device tensors (null pointers) for K and V, or
    # for Q and O, through the one-pass, block-major and split forms
    for sq, skv in ((7, 0), (0, 64)):
        sel = np.full((1, sq, 8), -1, np.int32)
        spec = dict(family="selected_key", sq=sq, skv=skv, batch=1, sel=sel, sel_cells=32)
        enc = fm.encode(spec)
        q = torch.randn(1, 4, sq, 128, device="cuda").to(torch.bfloat16)
        kv = torch.randn(1, 2, skv, 128, device="cuda").to(torch.bfloat16)
        outs = [fm.attn_fwd(q, kv, kv, enc, None, scale=1 / math.sqrt(128)),
                fm.attn_fwd_blocks(q, kv, kv, enc, scale=1 / math.sqrt(128)),
                fm.attn_fwd_split(q, kv, kv, enc, splits=3, scale=1 / math.sqrt(128))]
        torch.cuda.synchronize()
        for o, lse in outs:
            assert o.shape == q.shape and lse.shape == q.shape[:3]
            assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())
