"""The seeded generator: determinism, keyed independence, dtype rounding, ranges."""
import numpy as np
import torch

from gen import configs, synth


def test_keyed_rows_are_deterministic_and_order_free():
    w = configs.shrink(configs.C2, V=3000, B=3)
    a = synth.draft_arena(w, 5, 1)
    b = synth.draft_arena(w, 5, 1)
    assert a.dtype == np.uint16 and a.shape == (w.D, 3, w.K_e, 3000)
    np.testing.assert_array_equal(a, b)
    sub = synth.draft_arena(w, 5, 1, rows=[2, 0])
    np.testing.assert_array_equal(sub[:, 0], a[:, 2])
    np.testing.assert_array_equal(sub[:, 1], a[:, 0])
    np.testing.assert_array_equal(synth.draft_row(w, 5, 1, 1, 3, 4), a[2, 1, 4])
    assert not np.array_equal(synth.draft_arena(w, 6, 1), a)
    att = np.array([0, 1, 0])
    c = synth.draft_arena(w, 5, 1, att)
    np.testing.assert_array_equal(c[:, 0], a[:, 0])
    assert not np.array_equal(c[:, 1], a[:, 1])


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = (g.standard_normal(100000) * g.uniform(0.01, 100, size=100000)).astype(np.float32)
    ours = synth.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.from_bf16_bits(ours),
                                  torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_planted_peak_probability_range():
    g = synth.keyed(1, 2, 3)
    probs = []
    for _ in range(200):
        row = synth.logit_row(g, 4000).astype(np.float64)
        p = np.exp(row - row.max())
        probs.append(p.max() / p.sum())
    probs = np.array(probs)
    # the planted token's probability spans the calibration range 0.05 .. 0.98
    assert probs.min() < 0.15 and probs.max() > 0.9
    assert probs.min() >= 0.04


def test_uniforms_temperatures_roots():
    w = configs.shrink(configs.C5, V=2000, B=64)
    U = synth.uniforms(w, 1, 0)
    assert U.shape == (64, w.m + 1, 2) and U.dtype == np.float32
    assert (U >= 0).all() and (U < 1).all()
    T = synth.temperatures(w, 1, 0)
    assert set(np.unique(T).tolist()) == {0.0, 1.0}
    assert set(np.unique(synth.temperatures(configs.C3, 1, 0)).tolist()) == {1.0}
    r = synth.root_tokens(w, 1, 0)
    assert r.min() >= 0 and r.max() < 2000
    np.testing.assert_array_equal(synth.root_tokens(w, 1, 0, rows=[5, 7]), r[[5, 7]])


def test_cost_tables_linear_and_seeded():
    S_T, S_D = synth.cost_tables(configs.C2)
    cw = S_D[3, 1:11] / S_T[3, 1]
    np.testing.assert_allclose(cw, 0.02 * np.arange(1, 11) + 1.0, rtol=1e-6)
    cv = S_T[0, 1:11] / S_T[0, 1]
    np.testing.assert_allclose(np.diff(cv), 0.02, rtol=1e-4)
    w = configs.Workload(**{**configs.C2.__dict__,
                            "cast": configs.CastSpec(table="seeded")})
    S_T, S_D = synth.cost_tables(w, 3)
    assert (np.diff(S_T[:, 1:], axis=1) >= 0).all() and (np.diff(S_D[:, 1:], axis=1) > 0).all()
    assert not np.allclose(S_T[0], S_T[5])


def test_succ_matrix0_shape_and_zipf_head():
    w = configs.shrink(configs.C4, V=5000, B=2)
    M = synth.succ_matrix0(w, 7)
    assert M.shape == (2, 5000, 8) and M.dtype == np.int32
    assert all(len(set(r)) == 8 for r in M[0].tolist()[:500])
    np.testing.assert_array_equal(M, synth.succ_matrix0(w, 7))


def test_roofline_cost_table_closed_form():
    # one layer of the 8B-class proxy: 4096*(48*128) + 4096*4096 + 3*4096*14336
    # = 218103808 weights, 436207616 bytes, 54.5259520 us at 8 TB/s; the LM head
    # 2*4096*128256 = 1050673152 bytes, 131.334144 us.  At batch 8 a forward of
    # one token with no context is HBM-bound: 32 * 54.525952 + 131.334144 us
    T = synth.roofline_table(configs.PROXY_TARGET, 8, 256, 16, 128)
    Dh = synth.roofline_table(configs.PROXY_DRAFT, 8, 256, 16, 128)
    assert T.shape == (16, 129) and (T[:, 0] == 0).all()
    np.testing.assert_allclose(T[0, 1], 32 * 54.525952 + 131.334144, rtol=1e-6)
    np.testing.assert_allclose(Dh[0, 1], 54.525952 + 131.334144, rtol=1e-6)
    # HBM-bound up to 312.5 token rows of a layer (2 flops per weight per row
    # against 2 bytes per weight: 2.5e15 / 8e12), so 39 tokens at batch 8 cost
    # the same as one, and the 40th costs more
    assert (T[0, 1:40] == T[0, 1]).all() and T[0, 40] > T[0, 39]
    # the context adds 2 * 2 * B * c * Hkv * D bytes of keys and values a layer
    np.testing.assert_allclose(T[1, 1] - T[0, 1], 32 * 2 * 2 * 8 * 256 * 8 * 128 / 8e12 * 1e6, rtol=1e-5)
    assert (np.diff(T[:, 1:], axis=1) >= 0).all() and (np.diff(T[:, 1:], axis=0) >= 0).all()
    w = configs.Workload(**{**configs.C2.__dict__,
                            "cast": configs.CastSpec(table="roofline", table_B=64)})
    S_T, S_D = synth.cost_tables(w)
    np.testing.assert_array_equal(S_T, synth.roofline_table(configs.PROXY_TARGET, 64, 256, 16, 128))
    np.testing.assert_array_equal(S_D, synth.roofline_table(configs.PROXY_DRAFT, 64, 256, 16, 128))
    assert (S_T[0, 1:5] == S_T[0, 1]).all() and S_T[0, 5] > S_T[0, 4]
