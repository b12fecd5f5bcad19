"""Properties of the seeded workload generators (shared by tests and bench)."""

import numpy as np

import synth


def test_seed_determinism():
    a = synth.workload("causal_doc_8k")
    b = synth.workload("causal_doc_8k")
    assert a["doc_lengths"] == b["doc_lengths"]
    qa = synth.draw_qkv(synth.workload("tiny_causal_doc"))
    qb = synth.draw_qkv(synth.workload("tiny_causal_doc"))
    for x, y in zip(qa, qb):
        np.testing.assert_array_equal(x, y)


def test_doc_lengths_law():
    for S in (8192, 32768, 4096, 256):
        rng = np.random.default_rng(S)
        for _ in range(20):
            L = synth.doc_lengths(rng, S)
            assert sum(L) == S
            assert all(x % 64 == 0 and 256 <= x <= 4096 for x in L)


def test_answer_lengths_law():
    w = synth.workload("shared_question_32k")
    ans = w["answer_lengths"]
    assert len(ans) == 8 and sum(ans) == 32768 - 2048
    assert all(a % 64 == 0 and a > 0 for a in ans)
    assert w["mask"]["cu_seg"][1] == 2048 and w["mask"]["cu_seg"][-1] == 32768


def test_tree_orders():
    rng = np.random.default_rng(0)
    for order in ("bfs", "dfs"):
        p = synth.random_tree(rng, 64, order=order)
        assert p[0] == -1 and all(0 <= p[t] < t for t in range(1, 64))
        depth = [0] * 64
        for t in range(1, 64):
            depth[t] = depth[p[t]] + 1
        assert max(depth) <= 4
        if order == "bfs":
            assert depth == sorted(depth)
        else:  # preorder: every subtree is a contiguous range
            for c in range(64):
                desc = [t for t in range(64) if _is_anc(p, c, t)]
                assert desc == list(range(c, c + len(desc)))


def _is_anc(p, c, t):
    while t > c:
        t = p[t]
    return t == c


def test_block_pattern_and_lists():
    rng = np.random.default_rng(1)
    st, ix, bits = synth.block_pattern(rng, 256, 256)
    frac = np.bincount(st.ravel(), minlength=3) / st.size
    assert abs(frac[2] - 0.10) < 0.01 and abs(frac[1] - 0.05) < 0.01
    assert bits.shape == ((st == 1).sum(), 64) and bits.dtype == np.uint64
    assert (ix[st == 1] == np.arange(bits.shape[0])).all() and (ix[st != 1] == -1).all()
    ones = np.unpackbits(bits.view(np.uint8)).mean()
    assert abs(ones - 0.5) < 0.01
    sel = synth.selected_lists(rng, 2048, 4096)
    assert sel.shape == (2048, 64)
    assert (sel[0] == -1).all() and len(set(sel[1].tolist())) == 1 and len(set(sel[2].tolist())) == 64
    inv = (sel[3:] == -1).mean()
    assert abs(inv - 1 / 8) < 0.01
    assert sel.max() < 4096 and sel.min() >= -1


def test_bf16_generation_is_rne():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(10000).astype(np.float32)
    bits = synth._f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # nearest: no other bf16 value is closer
    up = ((bits.astype(np.uint32) + 1) << 16).view(np.float32)
    dn = ((bits.astype(np.uint32) - 1) << 16).view(np.float32)
    err = np.abs(back.astype(np.float64) - x)
    assert (err <= np.abs(up.astype(np.float64) - x)).all()
    assert (err <= np.abs(dn.astype(np.float64) - x)).all()
