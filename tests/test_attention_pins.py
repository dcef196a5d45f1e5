"""Pins of the tree-attention oracle: closed forms, a special case that reduces to
textbook causal attention, hand-listed visibility sets, and invariants that a
mistake in the mask or the head grouping would break."""
import numpy as np

from oracle import ddt_attention as A


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_chain_tree_is_causal_attention():
    # a chain (each position the child of the one before) sees exactly the
    # causal set: the prefix and every earlier tree position
    rng = np.random.default_rng(1)
    P, L, Hq, Hkv, D = 7, 5, 4, 2, 16
    q, kp, vp = _rand(rng, P, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    kt, vt = _rand(rng, P, Hkv, D), _rand(rng, P, Hkv, D)
    parent = np.arange(P) - 1
    scale = 0.3
    got = A.tree_attention(q, kp, vp, kt, vt, parent, P, scale)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        K = np.concatenate([kp[:, g], kt[:, g]])
        V = np.concatenate([vp[:, g], vt[:, g]])
        S = scale * q[:, h] @ K.T                              # [P][L + P]
        allowed = np.ones((P, L + P), bool)
        allowed[:, L:] = np.tril(np.ones((P, P), bool))
        S = np.where(allowed, S, -np.inf)
        W = np.exp(S - S.max(axis=1, keepdims=True))
        W /= W.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(got[:, h], W @ V, rtol=1e-12, atol=1e-13)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(2)
    q = _rand(rng, 1, 3, 8)
    kt, vt = _rand(rng, 1, 3, 8), _rand(rng, 1, 3, 8)
    empty = np.zeros((0, 3, 8))
    got = A.tree_attention(q, empty, empty, kt, vt, np.array([-1]), 1, 1.0)
    np.testing.assert_allclose(got[0], vt[0], rtol=0, atol=1e-15)


def test_zero_query_averages_the_visible_values():
    # q = 0 gives equal weights: the output is the mean of the prefix values and
    # of the values on the path to the root, listed here by hand
    rng = np.random.default_rng(3)
    parent = np.array([-1, 0, 0, 1, 2, 3])
    paths = {0: [0], 1: [1, 0], 2: [2, 0], 3: [3, 1, 0], 4: [4, 2, 0], 5: [5, 3, 1, 0]}
    P, L, H, D = 6, 3, 2, 4
    kp, vp = _rand(rng, L, H, D), _rand(rng, L, H, D)
    kt, vt = _rand(rng, P, H, D), _rand(rng, P, H, D)
    got = A.tree_attention(np.zeros((P, H, D)), kp, vp, kt, vt, parent, P, 0.7)
    for i, path in paths.items():
        for h in range(H):
            want = (vp[:, h].sum(axis=0) + vt[path, h].sum(axis=0)) / (L + len(path))
            np.testing.assert_allclose(got[i, h], want, rtol=1e-13, atol=1e-14)


def test_siblings_are_invisible():
    # branch {1, 3, 5} never sees branch {2, 4}: changing the other branch's keys
    # and values leaves it unchanged, while its own changes move it
    rng = np.random.default_rng(4)
    parent = np.array([-1, 0, 0, 1, 2, 3])
    P, L, Hq, Hkv, D = 6, 2, 2, 1, 8
    q, kp, vp = _rand(rng, P, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    kt, vt = _rand(rng, P, Hkv, D), _rand(rng, P, Hkv, D)
    base = A.tree_attention(q, kp, vp, kt, vt, parent, P, 0.5)
    kt2, vt2 = kt.copy(), vt.copy()
    kt2[[2, 4]] += 3.0
    vt2[[2, 4]] -= 2.0
    other = A.tree_attention(q, kp, vp, kt2, vt2, parent, P, 0.5)
    np.testing.assert_allclose(other[[0, 1, 3, 5]], base[[0, 1, 3, 5]], rtol=0, atol=1e-15)
    assert np.abs(other[[2, 4]] - base[[2, 4]]).max() > 1e-3


def test_grouped_heads_share_their_kv_head():
    rng = np.random.default_rng(5)
    P, L, Hq, Hkv, D = 4, 3, 4, 2, 8
    parent = np.array([-1, 0, 1, 1])
    q = _rand(rng, P, Hq, D)
    q[:, 1] = q[:, 0]                                          # heads 0 and 1 share kv head 0
    kp, vp = _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    kt, vt = _rand(rng, P, Hkv, D), _rand(rng, P, Hkv, D)
    a = A.tree_attention(q, kp, vp, kt, vt, parent, P, 0.4)
    np.testing.assert_allclose(a[:, 1], a[:, 0], rtol=0, atol=0)
    kp2, vt2 = kp.copy(), vt.copy()
    kp2[:, 1] += 1.0                                           # kv head 1 only
    vt2[:, 1] -= 1.0
    b = A.tree_attention(q, kp2, vp, kt, vt2, parent, P, 0.4)
    np.testing.assert_allclose(b[:, :2], a[:, :2], rtol=0, atol=0)
    assert np.abs(b[:, 2:] - a[:, 2:]).max() > 1e-3


def test_padding_positions_are_zero():
    rng = np.random.default_rng(6)
    P, H, D = 5, 2, 4
    out = A.tree_attention(_rand(rng, P, H, D), _rand(rng, 2, H, D), _rand(rng, 2, H, D),
                           _rand(rng, P, H, D), _rand(rng, P, H, D), np.array([-1, 0, 1, -1, -1]),
                           3, 1.0)
    assert not out[3:].any() and np.abs(out[:3]).min() > 0
