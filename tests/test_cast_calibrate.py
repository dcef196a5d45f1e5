"""CAST cost tables measured on the device (CAST notes, key design 1, and the
notes' limitations section: the table is measured per GPU and batch size).

CPU: table assembly from per-layer and LM-head times, pinned by hand.  GPU: a
small measured grid obeys what any measurement must (non-decreasing in the
token count, the target above the one-layer draft, never faster than the HBM
and MFMA roofline of the same shapes at MI355X's published peaks, more
context costing more), and a CAST round runs on the measured tables."""
import numpy as np
import pytest

from dynamic_draft_tree_row_amd import cast_calibrate as CC
from gen import configs, synth


def test_assemble_by_hand():
    lay = np.array([[1.0, 2.0, 1.0], [3.0, 3.0, 4.0]])
    head = np.array([10.0, 10.0, 10.0])
    t = CC.assemble(lay, head, n_layers=2)
    assert t.dtype == np.float32 and t.shape == (2, 4)
    # row 0: 12, 14, then 12 raised to 14 by the running maximum
    np.testing.assert_array_equal(t, [[0, 12, 14, 14], [0, 16, 16, 18]])
    with pytest.raises(ValueError):
        CC.assemble(lay, head[:2], 2)


def test_proxy_shapes_match_the_generator():
    for a, b in ((CC.TARGET_8B, configs.PROXY_TARGET), (CC.DRAFT_HEAD, configs.PROXY_DRAFT)):
        assert (a.d_model, a.n_layers, a.Hq, a.Hkv, a.D, a.ffn, a.V) == \
            (b.d_model, b.n_layers, b.Hq, b.Hkv, b.D, b.ffn, b.V)
    assert CC.TARGET_8B.layer_weight_bytes() == 2 * 218103808
    assert CC.TARGET_8B.head_weight_bytes() == 2 * 4096 * 128256


def test_tables_round_trip(tmp_path):
    S_T = CC.assemble(np.array([[10.0, 11.0], [12.0, 12.5]]), np.array([5.0, 6.0]), 32)
    S_D = CC.assemble(np.array([[1.0, 1.5], [1.2, 1.6]]), np.array([5.0, 6.0]), 1)
    p = str(tmp_path / "tables.npz")
    CC.save_tables(p, S_T, S_D, B=8, L=256, device="test device")
    got = CC.load_tables(p)
    np.testing.assert_array_equal(got["S_T"], S_T)
    np.testing.assert_array_equal(got["S_D"], S_D)
    assert (got["B"], got["L"], got["device"]) == (8, 256, "test device")
    assert got["target"] == CC.TARGET_8B and got["draft"] == CC.DRAFT_HEAD
    with pytest.raises(ValueError):
        CC.save_tables(p, S_T, S_D[:, :2], B=8, L=256)


def test_tables_round_trip_without_suffix(tmp_path):
    """A name with no .npz suffix is written and read back as given; a file
    that numpy's savez wrote as name.npz is found under the bare name too."""
    S_T = CC.assemble(np.array([[10.0, 11.0], [12.0, 12.5]]), np.array([5.0, 6.0]), 32)
    S_D = CC.assemble(np.array([[1.0, 1.5], [1.2, 1.6]]), np.array([5.0, 6.0]), 1)
    p = tmp_path / "tables_b8"
    CC.save_tables(str(p), S_T, S_D, B=8, L=256)
    assert p.exists() and not (tmp_path / "tables_b8.npz").exists()
    np.testing.assert_array_equal(CC.load_tables(str(p))["S_D"], S_D)
    q = tmp_path / "legacy"
    np.savez(str(q), S_T=S_T, S_D=S_D, B=np.int64(8), L=np.int64(256),
             target=np.array(CC.astuple(CC.TARGET_8B), np.int64),
             draft=np.array(CC.astuple(CC.DRAFT_HEAD), np.int64), device=np.array(""))
    assert CC.load_tables(str(q))["B"] == 8


def test_measure_rejects_bad_grids():
    with pytest.raises(ValueError):
        CC.measure_tables(B=1, L=16, M=1, N=300)
    with pytest.raises(ValueError):
        CC.measure_tables(B=1, L=16, M=1, N=4, target=CC.ProxyModel(512, 1, 4, 1, 64, 1024, 1000))


@pytest.mark.gpu
def test_measured_tables_on_device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    from dynamic_draft_tree_row_amd import _lib
    _lib.load()
    B, L, M, N = 4, 4096, 2, 4
    print(f"calibrate B={B} L={L} M={M} N={N}", flush=True)
    S_T, S_D = CC.measure_tables(B, L, M, N, reps=3, log=lambda s: print(s, flush=True))
    for t in (S_T, S_D):
        assert t.shape == (M, N + 1) and (t[:, 0] == 0).all()
        assert np.isfinite(t).all() and (t[:, 1:] > 0).all()
        assert (np.diff(t[:, 1:], axis=1) >= 0).all()
    assert (S_T[:, 1:] > S_D[:, 1:]).all()
    # no measurement beats the roofline of the same shapes (20% slack for the
    # published peaks being rounded and for clock boosts)
    assert (S_T >= 0.8 * synth.roofline_table(configs.PROXY_TARGET, B, L, M, N)).all()
    assert (S_D >= 0.8 * synth.roofline_table(configs.PROXY_DRAFT, B, L, M, N)).all()
    # 4096 context tokens add 64 MB of keys and values to each target layer
    assert S_T[1, 1] > S_T[0, 1]


@pytest.mark.gpu
def test_cast_round_on_measured_tables():
    # tables measured on this GPU are inputs like the logits: the oracle, fed
    # the same S_T and S_D, must reproduce the library's round exactly (CAST
    # key design 1: the tables are measured per GPU and batch size)
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    from tests import harness as H
    w = configs.shrink(configs.C2, V=17000)
    cs = w.cast
    print(f"calibrate B={w.B} L={cs.L} M=2 N=64 for a CAST round", flush=True)
    S_T, S_D = CC.measure_tables(w.B, cs.L, 2, 64, reps=2)
    cast = dict(S_T=S_T, S_D=S_D, L=cs.L, M=2, C1=[cs.C1] * w.D, C2=cs.C2, C3=[cs.C3] * w.B, R=cs.R)
    for rnd in range(2):
        case = H.oracle_case(w, 5, rnd, cast=cast)
        r = H.gpu_round(case)
        print(f"round {rnd}: measured S_T[0][1] {S_T[0, 1]:.1f} us, S_D[0][1] {S_D[0, 1]:.1f} us, "
              f"widths {r['widths'].tolist()}, verify counts {r['m_out'].tolist()}", flush=True)
        H.compare(case, r)
        m, n_nodes = r["m_out"], r["n_nodes"]
        assert (n_nodes >= 1).all() and ((m >= 1) & (m <= w.m_max)).all() and (m < n_nodes).all()
