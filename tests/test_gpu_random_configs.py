"""Seeded random configurations through the C ABI against the float64 oracle.

Each case draws a mask family and its parameters, the shapes (ragged Sq and
Skv up to a few hundred, B and heads of 1 or 2 mask slices, GQA groups, head
size), whether masks are shared or per (batch, head), and the tile table the
kernels run on; every output row is compared with the oracle.  For every
family but the selected-key lists, half the seeds (the first 12 of each 24)
also run the backward on the 128 x 64 table.  The case
parameters are printed, and a failure names its seed.
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as OA
from oracle import masks as OM
from tests.helpers import GRAD_SCALE_FLOOR, compare, to_device, to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fm = pytest.importorskip("mask_aware_block_amd")

FAMILIES = ("causal", "causal_bottom_right", "band", "document", "causal_document", "shared_question", "tree",
            "varlen", "block_bitmap", "intervals", "dense", "selected_key")


def _cuts(rng, n, k):
    """Sorted cumulative boundaries 0 = c0 < ... < ck = n (k segments, k <= n)."""
    inner = np.sort(rng.choice(np.arange(1, n), size=k - 1, replace=False)) if k > 1 else np.array([], int)
    return np.concatenate(([0], inner, [n])).astype(np.int32)


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    fam = FAMILIES[seed % len(FAMILIES)]
    square = fam in ("document", "causal_document", "shared_question", "tree")
    sq = int(rng.integers(1, 400))
    skv = sq if square else int(rng.integers(1, 450))
    if fam == "tree":
        sq = skv = max(sq, 2)
    B = int(rng.integers(1, 3))
    if fam == "selected_key":
        D = int(rng.choice([128, 256]))
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 4, 8, 12, 16]))
    else:
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 3, 4]))
    Hq = Hkv * G
    spec = dict(family=fam, sq=sq, skv=skv)
    if fam == "band":
        spec.update(pre=int(rng.integers(-20, 300)), next=int(rng.integers(-20, 60)))
    elif fam in ("document", "causal_document", "shared_question"):
        spec["cu_seg"] = _cuts(rng, sq, int(rng.integers(1, min(8, sq) + 1)))
    elif fam == "tree":
        n = int(rng.integers(1, min(64, sq) + 1))
        spec.update(tree_prefix=sq - n, tree_parent=synth.random_tree(rng, n, order=str(rng.choice(["bfs", "dfs"]))))
    elif fam == "varlen":
        k = int(rng.integers(1, min(5, sq, skv) + 1))
        modes = ["full", "causal", "causal_bottom_right", "band", "prefix"]
        spec.update(cu_q=_cuts(rng, sq, k), cu_k=_cuts(rng, skv, k),
                    seg_mode=[str(m) for m in rng.choice(modes, size=k)],
                    pre=int(rng.integers(0, 80)), next=int(rng.integers(0, 10)),
                    seg_prefix=[int(x) for x in rng.integers(0, 40, size=k)])
    elif fam in ("block_bitmap", "intervals", "dense"):
        mb = B if rng.random() < 0.5 else 1
        mh = Hq if rng.random() < 0.5 else 1
        spec.update(batch=mb, heads=mh)
        if fam == "block_bitmap":
            nbq, nbk = -(-sq // 64), -(-skv // 64)
            sts, ixs, pools, off = [], [], [], 0
            pf, pp = float(rng.uniform(0, 0.6)), float(rng.uniform(0, 0.4))
            for _ in range(mb * mh):
                st, ix, bits = synth.block_pattern(rng, nbq, nbk, pf, pp)
                sts.append(st)
                ixs.append(np.where(ix >= 0, ix + off, -1))
                pools.append(np.asarray(bits, dtype=np.uint64).reshape(-1, 64))
                off += pools[-1].shape[0]
            pool = np.concatenate(pools) if off else np.zeros((1, 64), np.uint64)
            spec.update(blk_state=np.stack(sts).reshape(mb, mh, nbq, nbk),
                        blk_index=np.stack(ixs).reshape(mb, mh, nbq, nbk).astype(np.int32),
                        blk_bits=pool, force_diag=bool(rng.random() < 0.5))
        elif fam == "intervals":
            spec["raw_intervals"] = rng.integers(-10, sq + 10, size=(mb, mh, 4, skv)).astype(np.int32)
        else:
            if rng.random() < 0.5:  # an interval-shaped mask per slice
                base = dict(family="band", sq=sq, skv=skv, pre=int(rng.integers(0, 100)), next=int(rng.integers(0, 9)))
                vis = np.asarray(OM.dense_vis(base)).astype(np.uint8)
                spec["dense"] = np.broadcast_to(vis, (mb, mh, sq, skv)).copy()
            else:
                spec["dense"] = (rng.random((mb, mh, sq, skv)) < rng.uniform(0.05, 0.6)).astype(np.uint8)
    elif fam == "selected_key":
        mb = B if rng.random() < 0.5 else 1
        nblk = -(-skv // 32)
        n = int(rng.integers(1, 65))
        spec.update(batch=mb, sel_cells=32,
                    sel=np.stack([synth.selected_lists(rng, sq, nblk, n=n) for _ in range(mb)]))
    w = dict(name=f"random{seed}", seed=2000 + seed, B=B, Hq=Hq, Hkv=Hkv, Sq=sq, Skv=skv, D=D, dtype="bf16",
             scale=1 / math.sqrt(D))
    return w, spec, rng


@pytest.mark.parametrize("seed", list(range(96)) + [531, 700, 776])
def test_random_configuration(seed):
    w, spec, rng = _case(seed)
    desc = (f"seed {seed}: {spec['family']} B{w['B']} Hq{w['Hq']} Hkv{w['Hkv']} Sq{w['Sq']} Skv{w['Skv']} "
            f"D{w['D']} " + " ".join(f"{k}={spec[k]}" for k in ("pre", "next", "batch", "heads") if k in spec))
    print(desc, flush=True)
    arrays = synth.draw_qkv(w)
    q, k, v = to_device(w, arrays)
    enc = fm.encode(spec)
    qq, kk, vv = (to_f64(w, a) for a in arrays)
    ro, rl = OA.attention_dense(qq, kk, vv, OA.spec_vis_fn(spec), w["scale"])
    if enc.kind == fm.ENC_SELECTED:
        for form in ("one-pass", "blocks", "split"):
            if form == "one-pass":
                o, lse = fm.attn_fwd(q, k, v, enc, None, scale=w["scale"])
            elif form == "blocks":
                o, lse = fm.attn_fwd_blocks(q, k, v, enc, scale=w["scale"])
            else:
                o, lse = fm.attn_fwd_split(q, k, v, enc, splits=int(rng.integers(0, 6)), scale=w["scale"])
            torch.cuda.synchronize()
            compare(w, o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"{desc} {form}")
        return
    shapes = (128, 64, 256) if enc.kind == fm.ENC_INTERVALS else (128, 64)
    bm = int(rng.choice(shapes))
    tiles = fm.classify(enc, bm, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    torch.cuda.synchronize()
    compare(w, o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, f"{desc} bm {bm}")
    if enc.kind in (fm.ENC_INTERVALS, fm.ENC_BITMAP) and (seed // len(FAMILIES)) % 2 == 0:
        tiles = fm.classify(enc, 128, 64)
        o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
        do_bits = synth.draw_dout(w)
        do = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).cuda()
        dq, dk, dv = fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=w["scale"])
        torch.cuda.synchronize()
        rq, rk, rv = OA.attention_backward_dense(qq, kk, vv, to_f64(w, do_bits), OA.spec_vis_fn(spec), w["scale"])
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            g = got.float().cpu().numpy().astype(np.float64)
            assert np.isfinite(g).all(), f"{desc}: {name} not finite"
            scale = max(np.abs(ref).max(), GRAD_SCALE_FLOOR)
            err = np.abs(g - ref)
            assert err.max() <= 2e-2 * scale, f"{desc}: {name} max err {err.max():.3e} (ref max {scale:.3e})"
            assert err.mean() <= 2e-3 * scale, f"{desc}: {name} mean err {err.mean():.3e}"
