"""Masked softmax attention in float64 (oracle; test infrastructure only).

Definition (the forward pass every page on the subject computes; the mask is
applied to the QK^T product as on the Ascend sparseMode page, masked positions
contributing nothing):
    g      = h // (Hq / Hkv)                       query head h reads K/V head g
    s_ij   = scale * sum_d Q[b,h,i,d] * K[b,g,j,d]
    V_i    = {j : vis(i, j)}
    V_i empty:  O_i = 0, LSE_i = -inf
    else:       m = max_{j in V_i} s_ij,  p_j = exp(s_ij - m) (0 off V_i),
                l = sum_j p_j,  O_i = sum_j (p_j / l) V[b,g,j,:],
                LSE_i = m + log(l)

``attention_dense`` evaluates this with dense QK^T over ALL key columns for a
chunk of rows, applies the materialised mask with np.where and multiplies the
dense P by V; ``attention_backward_dense`` gives its gradient the same way, and
``attention_backward_sampled`` that gradient at sampled rows and keys.
``attention_rows`` does the forward for a list of sampled rows,
``attention_bruteforce`` with scalar Python loops, and
``attention_listed_cells`` only over the cells a selected-key list names (the
host FP64 reference "over the listed cells" that the llama.cpp selected-key PR
tests its shader against).
"""

import math

import numpy as np

from . import masks


def bf16_bits_to_f64(bits):
    """float64 values of bfloat16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _softmax_rows(s, vis, vrows):
    """O and LSE of rows with scores s [R, Skv] (float64), mask vis [R, Skv]."""
    nonempty = vis.any(axis=1)
    s_m = np.where(vis, s, -np.inf)
    m = np.where(nonempty, s_m.max(axis=1, initial=-np.inf), 0.0)
    p = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    o = p @ vrows
    safe_l = np.where(nonempty, l, 1.0)
    o = np.where(nonempty[:, None], o / safe_l[:, None], 0.0)
    lse = np.where(nonempty, m + np.log(safe_l), -np.inf)
    return o, lse


def attention_dense(q, k, v, vis_fn, scale, row_chunk=512):
    """Dense masked attention.  q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D] (float64).

    vis_fn(b, h, rows) -> bool [len(rows), Skv].  Returns (O float64, LSE float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    O = np.zeros((B, Hq, Sq, v.shape[3]))
    LSE = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r0 in range(0, Sq, row_chunk):
                rows = np.arange(r0, min(Sq, r0 + row_chunk))
                vis = np.asarray(vis_fn(b, h, rows), dtype=bool)
                s = scale * (q[b, h, rows] @ k[b, g].T)
                O[b, h, rows], LSE[b, h, rows] = _softmax_rows(s, vis, v[b, g])
    return O, LSE


def spec_vis_fn(spec):
    """vis_fn for attention_dense from a mask spec (see oracle.masks)."""
    return lambda b, h, rows: masks.dense_vis(spec, b, h, rows)


def _f64(x, decode):
    return decode(x) if decode is not None else np.asarray(x, dtype=np.float64)


def attention_rows(q, k, v, vis_fn, scale, samples, decode=None):
    """O [n, D] and LSE [n] for sampled rows samples = [(b, h, i), ...].

    decode (optional) turns stored values into float64, e.g. bf16_bits_to_f64.
    """
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    outs, lses = [], []
    for b, h, i in samples:
        g = h // G
        vis = np.asarray(vis_fn(b, h, np.array([i])), dtype=bool)
        qi = _f64(q[b, h, i], decode)
        kk = _f64(k[b, g], decode)
        s = scale * (kk @ qi)[None, :]
        o, lse = _softmax_rows(s, vis, _f64(v[b, g], decode))
        outs.append(o[0])
        lses.append(lse[0])
    return np.array(outs), np.array(lses)


def attention_bruteforce(q, k, v, vis, scale):
    """Scalar Python evaluation for one (b, h) slice: q [Sq,D], k/v [Skv,D], vis [Sq,Skv]."""
    sq, d = len(q), len(q[0])
    skv = len(k)
    O = [[0.0] * d for _ in range(sq)]
    LSE = [-math.inf] * sq
    for i in range(sq):
        scores = {}
        for j in range(skv):
            if vis[i][j]:
                acc = 0.0
                for t in range(d):
                    acc += float(q[i][t]) * float(k[j][t])
                scores[j] = scale * acc
        if not scores:
            continue
        m = max(scores.values())
        w = {j: math.exp(s - m) for j, s in scores.items()}
        l = sum(w.values())
        for t in range(d):
            O[i][t] = sum(w[j] * float(v[j][t]) for j in w) / l
        LSE[i] = m + math.log(l)
    return np.array(O), np.array(LSE)


def listed_cells(entries, cells, skv):
    """Key cells named by one selected-key list: valid blocks, each once, ascending."""
    nblk = -(-skv // cells)
    blocks = sorted({int(e) for e in entries if 0 <= int(e) < nblk})
    out = [np.arange(e * cells, min(skv, (e + 1) * cells)) for e in blocks]
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def attention_listed_cells(q, k, v, sel, cells, scale, samples, decode=None):
    """Selected-key attention over exactly the listed cells, for sampled rows.

    sel [B_m][Sq][n] lists (shared by every head); samples = [(b, h, i), ...].
    """
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    skv = k.shape[2]
    sel = np.asarray(sel)
    outs, lses = [], []
    for b, h, i in samples:
        g = h // G
        bm = b if sel.shape[0] > 1 else 0
        keys = listed_cells(sel[bm, i], cells, skv)
        if keys.size == 0:
            outs.append(np.zeros(v.shape[3]))
            lses.append(-np.inf)
            continue
        kk = _f64(k[b, g, keys], decode)
        vv = _f64(v[b, g, keys], decode)
        s = scale * (kk @ _f64(q[b, h, i], decode))
        m = s.max()
        p = np.exp(s - m)
        l = p.sum()
        outs.append((p @ vv) / l)
        lses.append(m + math.log(l))
    return np.array(outs), np.array(lses)


def attention_backward_dense(q, k, v, do, vis_fn, scale, row_chunk=512):
    """Gradients (dQ, dK, dV) of the masked attention above w.r.t. Q, K and V,
    given the output gradient dO [B,Hq,Sq,Dv] (all float64).

    The analytic gradient of softmax attention, written per (b, h) over the
    materialised mask (rows with no visible key have P = 0 and contribute
    nothing, consistent with O_i = 0 there):
        P_ij   = exp(s_ij - LSE_i) on visible cells, 0 elsewhere
        dV_g  += P^T dO                       (summed over the heads of group g)
        dP     = dO V_g^T
        D_i    = sum_j P_ij dP_ij             (= sum_d dO_id O_id)
        dS     = P * (dP - D)
        dQ     = scale dS K_g
        dK_g  += scale dS^T Q
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r0 in range(0, Sq, row_chunk):
                rows = np.arange(r0, min(Sq, r0 + row_chunk))
                vis = np.asarray(vis_fn(b, h, rows), dtype=bool)
                s = scale * (q[b, h, rows] @ k[b, g].T)
                _, lse = _softmax_rows(s, vis, v[b, g])
                nonempty = np.isfinite(lse)
                p = np.where(vis & nonempty[:, None], np.exp(s - np.where(nonempty, lse, 0.0)[:, None]), 0.0)
                dor = do[b, h, rows]
                dv[b, g] += p.T @ dor
                dp = dor @ v[b, g].T
                delta = (p * dp).sum(axis=1)
                ds = p * (dp - delta[:, None])
                dq[b, h, rows] = scale * (ds @ k[b, g])
                dk[b, g] += scale * (ds.T @ q[b, h, rows])
    return dq, dk, dv


def attention_backward_sampled(q, k, v, do, vis_fn, scale, b, rows, keys, row_chunk=512):
    """The gradient of attention_backward_dense at sampled outputs of batch
    entry b: dQ at query rows `rows` (every head) and dK, dV at key positions
    `keys` (every K/V head), from the same definition, evaluated only where
    those outputs depend on it.

    dQ_i = scale sum_j dS_ij K_j needs row i alone (its P, dP and D_i).
    dK_j = scale sum_{h in group, i} dS_ij Q_i and dV_j = sum P_ij dO_i run over
    the rows with P_ij > 0, i.e. the rows whose mask shows key j (P is zero
    elsewhere): those rows are found from the materialised mask and evaluated
    whole (P_ij needs the row's LSE, dS_ij its D_i).
    Returns dq [Hq, len(rows), D], dk [Hkv, len(keys), D], dv [Hkv, len(keys), Dv].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)

    def row_terms(h, rr):
        """P and dS of rows rr of head h against every key."""
        g = h // G
        vis = np.asarray(vis_fn(b, h, rr), dtype=bool)
        s = scale * (q[b, h, rr] @ k[b, g].T)
        _, lse = _softmax_rows(s, vis, v[b, g])
        nonempty = np.isfinite(lse)
        p = np.where(vis & nonempty[:, None], np.exp(s - np.where(nonempty, lse, 0.0)[:, None]), 0.0)
        dp = do[b, h, rr] @ v[b, g].T
        delta = (p * dp).sum(axis=1)
        return p, p * (dp - delta[:, None])

    dq = np.zeros((Hq, len(rows), D))
    dk = np.zeros((Hkv, len(keys), D))
    dv = np.zeros((Hkv, len(keys), v.shape[3]))
    for h in range(Hq):
        g = h // G
        if len(rows):
            _, ds = row_terms(h, rows)
            dq[h] = scale * (ds @ k[b, g])
        if len(keys):
            for r0 in range(0, Sq, row_chunk):
                rr = np.arange(r0, min(Sq, r0 + row_chunk))
                rr = rr[np.asarray(vis_fn(b, h, rr), dtype=bool)[:, keys].any(axis=1)]
                if len(rr) == 0:
                    continue
                p, ds = row_terms(h, rr)
                dv[g] += p[:, keys].T @ do[b, h, rr]
                dk[g] += scale * (ds[:, keys].T @ q[b, h, rr])
    return dq, dk, dv
