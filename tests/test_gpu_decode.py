"""Few-query (decode) selected-key path, fmask_attn_fwd_split, through the C ABI.

Each query's list is split over several workgroups and the partial states are
merged (the split-K combine of the selected-key PR).  Compared with the float64
oracle over exactly the listed cells (oracle.attention.attention_listed_cells)
for every row, for several split counts including the automatic one, lists
with no valid entry, and GQA groups of 4, 8 and 12 query heads.
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


def _workload(Sq, Skv, D, Hq, Hkv, seed, edge_rows):
    w = dict(name="decode", seed=seed, B=1, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D, dtype="bf16",
             scale=1 / math.sqrt(D))
    rng = synth.streams(seed)[3]
    nblk = -(-Skv // 32)
    sel = synth.selected_lists(rng, Sq, nblk, edge_rows=edge_rows)
    w["mask"] = dict(family="selected_key", sq=Sq, skv=Skv, batch=1, sel=sel[None], sel_cells=32)
    return w


def _check(w, splits_list):
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(w["mask"])
    samples = [(0, h, i) for h in range(w["Hq"]) for i in range(w["Sq"])]
    ro, rl = OA.attention_listed_cells(*arrays, w["mask"]["sel"], 32, w["scale"], samples,
                                       decode=OA.bf16_bits_to_f64)
    o1, l1 = fm.attn_fwd(q, k, v, enc, None, scale=w["scale"])
    for splits in splits_list:
        o, lse = fm.attn_fwd_split(q, k, v, enc, splits=splits, scale=w["scale"])
        torch.cuda.synchronize()
        got_o = np.stack([o[0, h, i].float().cpu().numpy() for (_, h, i) in samples])
        got_l = np.array([lse[0, h, i].item() for (_, h, i) in samples])
        compare(w, got_o, got_l, ro, rl, f"splits {splits} Sq {w['Sq']} G {w['Hq'] // w['Hkv']}")
        if splits == 1:  # one split is the one-pass kernel itself
            assert torch.equal(o, o1) and torch.equal(lse, l1)


@pytest.mark.parametrize("D", [256, 128])
def test_single_query(D):
    w = _workload(1, 4096 + 17, D, 32, 8, 31, edge_rows=False)
    _check(w, [1, 2, 3, 16, 0])


def test_few_queries_with_edge_rows():
    # query 0 lists nothing valid (empty row: O = 0, LSE = -inf), query 1 one
    # block repeated, query 2 distinct blocks
    w = _workload(16, 8192, 256, 32, 8, 32, edge_rows=True)
    _check(w, [1, 4, 7, 0])


@pytest.mark.parametrize("Hq,Hkv", [(24, 2), (16, 2), (8, 2)])
def test_gqa_groups(Hq, Hkv):
    w = _workload(3, 2048 + 5, 128, Hq, Hkv, 33, edge_rows=False)
    _check(w, [1, 5, 0])


def test_full_size_decode_rows():
    w = synth.workload("selected_key_decode16_128k")
    _check(w, [0])
