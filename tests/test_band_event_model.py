"""A CPU model of one unexplained GPU test failure, run on the oracle.

One GPU run of the interval tile-shape test failed on its band case (S = 700,
preTokens 100, nextTokens 5, 128 x 64 tiles, B 2, 8 query heads over 2 K/V
heads, head dim 128, seed 11) with an LSE error of 1.0e-2 against the bf16
bound 2^-8 + 5e-4, while O stayed inside 2e-2 max / 1e-3 mean.  The case did
not recur.  This module replays, in float64 on that case's exact inputs, every
way a single misdirected load or a single bookkeeping slip of the 128-row
kernel could have changed one workgroup's tile, and records which of them
give that signature:

  * direct-to-LDS hazard: a load that reads the previous value of M0 puts its
    1 KB (or 256 B) into the previous load's destination and leaves its own
    destination stale.  In the kernel's issue order (V(i), then K(i+1), then
    the interval field of i+1) that is: a V group of 4 keys moved one group
    down or onto the interval buffer, a K group of tile i+1 moved onto the V
    buffer or one group down, an interval field landing on a K row;
  * a stale tile-list entry: the tile's K, V and intervals are those of the
    previous list entry;
  * a row-sum slip: one wave's share of a tile counted in l but not in O, in O
    but not in l, or in l twice.

The model works with per-tile softmax partial states (m, l, unnormalised O) of
every row, so each candidate recomputes only the one tile it changes.  Stale
LDS content is the same buffer's content one or two list entries earlier, or
zeros where the buffer has not been written in this workgroup yet.
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as OA
from oracle import encode as OE
from oracle import masks as OM

S, PRE, NXT, B, HQ, HKV, D = 700, 100, 5, 2, 8, 2, 128
BM, BN = 128, 64
LSE_BOUND = 2.0 ** -8 + 5e-4


def _case():
    w = dict(name="small", seed=11, B=B, Hq=HQ, Hkv=HKV, Sq=S, Skv=S, D=D, dtype="bf16", scale=1 / math.sqrt(D))
    q, k, v = (OA.bf16_bits_to_f64(a) for a in synth.draw_qkv(w))
    spec = dict(family="band", sq=S, skv=S, pre=PRE, next=NXT)
    vis = np.asarray(OM.dense_vis(spec))
    iv = OE.intervals_from_dense(vis)  # canonical [4][S]: UTS, UTE, LTS, LTE
    return w, q, k, v, vis, iv


def _vis_from_iv(iv, rows, cols):
    r = rows[:, None]
    uts, ute, lts, lte = (iv[f][cols][None, :] for f in range(4))
    return ~(((uts <= r) & (r < ute)) | ((lts <= r) & (r < lte)))


def _tile_state(s, vis, vv):
    """Partial softmax state of scores s [R, n] under vis over values vv [n, D]."""
    sm = np.where(vis, s, -np.inf)
    m = sm.max(axis=1)
    mf = np.where(np.isfinite(m), m, 0.0)
    p = np.where(vis, np.exp(s - mf[:, None]), 0.0)
    return m, p.sum(axis=1), p @ vv


def _combine(states):
    ms = np.stack([st[0] for st in states])
    M = ms.max(axis=0)
    Mf = np.where(np.isfinite(M), M, 0.0)
    f = np.where(np.isfinite(ms), np.exp(ms - Mf[None]), 0.0)
    L = sum(fi * st[1] for fi, st in zip(f, states))
    O = sum(fi[:, None] * st[2] for fi, st in zip(f, states))
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(L[:, None] > 0, O / np.where(L > 0, L, 1)[:, None], 0.0)
        lse = np.where(L > 0, Mf + np.log(np.where(L > 0, L, 1)), -np.inf)
    return out, lse, L


def _model():
    w, q, k, v, vis, iv = _case()
    scale = w["scale"]
    nqt, nkt = -(-S // BM), -(-S // BN)
    ref_o, ref_l = OA.attention_dense(q, k, v, OA.spec_vis_fn(dict(family="band", sq=S, skv=S, pre=PRE, next=NXT)),
                                      scale)
    states = OE.tile_states(vis, BM, BN)
    results = []  # (kind, lse_err, o_max, o_mean_over_all_outputs)
    n_all = B * HQ * S * D
    for b in range(B):
        for h in range(HQ):
            g = h // (HQ // HKV)
            for qt in range(nqt):
                rows = np.arange(qt * BM, min(S, (qt + 1) * BM))
                lst = [kt for kt in range(nkt) if states[qt, kt] != 0]
                full = {kt: states[qt, kt] == 2 for kt in lst}
                cols_of = {kt: np.arange(kt * BN, min(S, (kt + 1) * BN)) for kt in lst}
                qq = q[b, h, rows] * scale

                def tile(kt, kk=None, vv=None, vmask=None):
                    c = cols_of[kt]
                    kk = k[b, g, c] if kk is None else kk
                    vv = v[b, g, c] if vv is None else vv
                    vm = vis[np.ix_(rows, c)] if vmask is None else vmask
                    return _tile_state(qq @ kk.T, vm, vv)

                base = {kt: tile(kt) for kt in lst}

                def score(kind, changed, wave_rows=None, l_only=None):
                    sts = [changed.get(kt, base[kt]) for kt in lst]
                    out, lse, L = _combine(sts)
                    if l_only is not None:  # row-sum slips on one wave's rows
                        out, lse = l_only(out, lse, L)
                    e_l = np.abs(lse - ref_l[b, h, rows])
                    e_l = np.where(np.isfinite(lse) | np.isfinite(ref_l[b, h, rows]), e_l, 0.0)
                    e_o = np.abs(out - ref_o[b, h, rows])
                    results.append((kind, float(np.nan_to_num(e_l, nan=np.inf).max()),
                                    float(np.nan_to_num(e_o, nan=np.inf).max()), float(e_o.sum() / n_all)))

                for i, kt in enumerate(lst):
                    c = cols_of[kt]
                    n = len(c)
                    nxt = lst[i + 1] if i + 1 < len(lst) else None
                    k_t, v_t = k[b, g, c], v[b, g, c]

                    def rows_of_group(grp):  # rows of the 64-row padded tile copies
                        return np.arange(4 * grp, 4 * grp + 4)

                    def pad(a):  # tile-shaped (64 rows) copy, zeros past the end
                        z = np.zeros((BN, D))
                        z[: len(a)] = a
                        return z

                    def stale(arr_getter, back):
                        j = i - back
                        return pad(arr_getter(lst[j])) if j >= 0 else np.zeros((BN, D))

                    kget = lambda t: k[b, g, cols_of[t]]
                    vget = lambda t: v[b, g, cols_of[t]]
                    for wv in range(4):
                        for ld in range(4):
                            grp = 4 * wv + ld
                            # V group grp of tile i moved one slot down (ld > 0) and left stale
                            vt = pad(v_t)
                            vs = stale(vget, 1)
                            if ld > 0:
                                vt[rows_of_group(grp - 1)] = pad(v_t)[rows_of_group(grp)]
                            vt[rows_of_group(grp)] = vs[rows_of_group(grp)]
                            score("M0: V group misplaced", {kt: tile(kt, vv=vt[:n])})
                            if nxt is not None:
                                # K group grp of tile i + 1: moved one slot down (ld > 0) or onto
                                # V group 4 wv + 3 of tile i (ld == 0), and left stale (K of i - 1)
                                cn = cols_of[nxt]
                                kn = pad(k[b, g, cn])
                                ks = stale(kget, 1)
                                changed = {}
                                if ld > 0:
                                    kn[rows_of_group(grp - 1)] = pad(k[b, g, cn])[rows_of_group(grp)]
                                else:
                                    vt2 = pad(v_t)
                                    vt2[rows_of_group(4 * wv + 3)] = pad(k[b, g, cn])[rows_of_group(grp)]
                                    changed[kt] = tile(kt, vv=vt2[:n])
                                kn[rows_of_group(grp)] = ks[rows_of_group(grp)]
                                changed[nxt] = tile(nxt, kk=kn[: len(cn)])
                                score("M0: K group misplaced", changed)
                        if nxt is not None and not full[nxt]:
                            # interval field wv of tile i + 1 stale (field of tile i - 1)
                            cn = cols_of[nxt]
                            ivn = [iv[f][cn].copy() for f in range(4)]
                            if i - 1 >= 0:
                                cs = cols_of[lst[i - 1]]
                                m_ = min(len(cs), len(cn))
                                ivn[wv][:m_] = iv[wv][cs][:m_]
                            else:
                                ivn[wv][:] = 0
                            r = rows[:, None]
                            vm = ~(((ivn[0][None] <= r) & (r < ivn[1][None])) | ((ivn[2][None] <= r) & (r < ivn[3][None])))
                            score("M0: interval field stale", {nxt: tile(nxt, vmask=vm)})
                        # row-sum slips on wave wv's 32 rows for tile i
                        wr = slice(32 * wv, 32 * wv + 32)
                        st = base[kt]
                        for slip in ("l only", "O only", "l twice"):
                            def fix(out, lse, L, st=st, wr=wr, slip=slip):
                                others = [base[t] for t in lst if t != kt]
                                o2, l2, L2 = _combine(others + [st])
                                M = np.maximum.reduce([s_[0] for s_ in others + [st]])
                                Mf = np.where(np.isfinite(M), M, 0.0)
                                ft = np.where(np.isfinite(st[0]), np.exp(st[0] - Mf), 0.0)
                                lt = ft * st[1]  # the tile's share of l
                                out, lse = out.copy(), lse.copy()
                                if slip == "l only":  # l counts the tile, O does not
                                    o_un = out * L[:, None] - ft[:, None] * st[2]
                                    Lw = L
                                elif slip == "O only":
                                    o_un = out * L[:, None]
                                    Lw = L - lt
                                else:
                                    o_un = out * L[:, None]
                                    Lw = L + lt
                                with np.errstate(invalid="ignore", divide="ignore"):
                                    out[wr] = np.where(Lw[wr, None] > 0, o_un[wr] / np.where(Lw[wr] > 0, Lw[wr], 1)[:, None], 0)
                                    lse[wr] = np.where(Lw[wr] > 0, Mf[wr] + np.log(np.where(Lw[wr] > 0, Lw[wr], 1)), -np.inf)
                                return out, lse
                            score(f"row sum: {slip}", {}, l_only=fix)
                    if i > 0:
                        # stale list entry: the tile's data are the previous entry's
                        pk = lst[i - 1]
                        cp = cols_of[pk]
                        m_ = min(len(cp), n)
                        kk = np.zeros((n, D)); kk[:m_] = k[b, g, cp][:m_]
                        vv = np.zeros((n, D)); vv[:m_] = v[b, g, cp][:m_]
                        vm = np.zeros((len(rows), n), dtype=bool)
                        vm[:, :m_] = vis[np.ix_(rows, cp)][:, :m_]
                        score("stale list entry", {kt: tile(kt, kk=kk, vv=vv, vmask=vm)})
    return results


@pytest.fixture(scope="module")
def outcomes():
    return _model()


def _summary(outcomes):
    kinds = sorted({r[0] for r in outcomes})
    table = {}
    for kd in kinds:
        rs = [r for r in outcomes if r[0] == kd]
        visible = [r for r in rs if r[1] > LSE_BOUND or r[2] > 2e-2 or r[3] > 1e-3]
        sig = [r for r in rs if 5e-3 <= r[1] <= 2e-2 and r[2] <= 2e-2 and r[3] <= 1e-3]
        table[kd] = (len(rs), len(visible), len(sig))
    return table


def test_clean_model_equals_the_oracle():
    """With nothing changed the per-tile combination is the oracle itself."""
    w, q, k, v, vis, iv = _case()
    np.testing.assert_array_equal(_vis_from_iv(iv, np.arange(S), np.arange(S)), vis)
    rows = np.arange(128, 256)
    qq = q[1, 5, rows] * w["scale"]
    sts = [_tile_state(qq @ k[1, 1][c].T, vis[np.ix_(rows, c)], v[1, 1][c])
           for c in (np.arange(t * 64, min(S, t * 64 + 64)) for t in range(11))]
    out, lse, _ = _combine(sts)
    ro, rl = OA.attention_rows(q, k, v, OA.spec_vis_fn(dict(family="band", sq=S, skv=S, pre=PRE, next=NXT)),
                               w["scale"], [(1, 5, r) for r in rows])
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


def test_which_slips_give_the_observed_signature(outcomes):
    """Signature: LSE error 0.5e-2 .. 2e-2 with O inside 2e-2 max and 1e-3 mean
    (over all outputs of the case).  Measured on this case: a K group moved by
    the M0 hazard gives it on a few instances (LSE 5e-3 .. 7e-3, O max up to
    1.9e-2: the moved keys carry a small share of the affected rows' weight);
    a row-sum slip (one wave's tile share in O but not l, or in l twice) gives
    it where that share is 1.6 .. 1.9 % of the row's weight; a moved V group
    only changes O, and a stale interval field or list entry always moves LSE
    by far more (>= 2.7e-2 and >= 0.43).  So the event was one of the first two
    kinds; only the first has a mechanism in the kernel (the load that issued
    without a wait state after its M0 write, padded since)."""
    table = _summary(outcomes)
    for kd, (n, visible, sig) in table.items():
        print(f"{kd:28s} instances {n:5d}  visible {visible:5d}  signature {sig:5d}")
    assert all(table[kd][0] > 0 for kd in table)
    assert table["M0: K group misplaced"][2] > 0
    assert table["row sum: O only"][2] > 0 and table["row sum: l twice"][2] > 0
    for kd in ("M0: V group misplaced", "M0: interval field stale", "stale list entry", "row sum: l only"):
        assert table[kd][2] == 0, kd
    lse_min = {kd: min(r[1] for r in outcomes if r[0] == kd and (r[1] > LSE_BOUND or r[2] > 2e-2))
               for kd in ("M0: interval field stale", "stale list entry")}
    assert lse_min["M0: interval field stale"] > 2e-2 and lse_min["stale list entry"] > 0.4
