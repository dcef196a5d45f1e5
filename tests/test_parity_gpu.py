"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Exact on token ids, tree structure, selections, flat layout, masks, retrieve
paths, argmaxes, accept lengths/paths, next tokens and successor-matrix rows;
rtol 1e-5 on fp32 path values and log confidences.  Small cases span several
vocab chunks and a ragged tail; full-size cases run the five workloads in the
launch configuration the bench times (the B=64 workload is compared on sampled
rows, every row checked for the method's invariants).
"""
import dataclasses
import json
import os
import sys

import numpy as np
import pytest
import torch

from gen import configs, synth
from oracle import ddt_oracle as O
from tests import harness as H

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    from dynamic_draft_tree_row_amd import _lib
    _lib.load()      # raises if the library was not built: no fallback


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------
# row reduction alone
# ---------------------------------------------------------------------------

def _rows_with_ties(V, dtype, seed):
    g = np.random.default_rng(seed)
    rows = [(g.standard_normal(V) * g.uniform(0.3, 3)).astype(np.float32) for _ in range(3)]
    rows.append(np.round(g.standard_normal(V) * 2).astype(np.float32))      # heavy ties
    rows.append(np.full(V, 1.5, np.float32))                                 # all equal
    r = (g.standard_normal(V)).astype(np.float32)
    r[g.integers(0, V, size=min(V, 5))] = 9.0                                # repeated max
    rows.append(r)
    return np.stack([synth.cast_row(x, dtype) for x in rows])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 7, 100, 4095, 4096, 8191, 8192, 8193, 33001, 128256])
def test_row_topk_parity(dtype, V):
    from dynamic_draft_tree_row_amd import api
    raw = _rows_with_ties(V, dtype, V)
    n = raw.shape[0]
    pad = 3                                   # row stride V + 3: unaligned rows too
    host = np.zeros((2, 3, V + pad), raw.dtype)
    host.reshape(6, V + pad)[:, :V] = raw
    x = H.to_dev(host, dtype)[:, :, :V]
    for K in sorted({1, min(8, V), min(10, V), min(32, V)}):
        say(f"row_topk dtype={dtype} V={V} K={K}")
        ws = torch.empty(api.workspace_bytes(6, V, x.dtype, K), dtype=torch.uint8, device="cuda")
        ids = torch.empty((6, K), dtype=torch.int32, device="cuda")
        lc = torch.empty((6, K), dtype=torch.float32, device="cuda")
        mx = torch.empty(6, dtype=torch.float32, device="cuda")
        sp = torch.empty(6, dtype=torch.float32, device="cuda")
        api.row_topk(x, K, ws, ids, lc, mx, sp)
        torch.cuda.synchronize()
        for i in range(n):
            l = O.decode(raw[i], dtype)
            m, _, s = O.row_stats(l)
            want = O.topk_ids(l, K)
            assert ids[i].cpu().tolist() == want.tolist(), f"row {i}"
            np.testing.assert_allclose(lc[i].cpu().numpy(), O.log_conf(l, want, m, s),
                                       rtol=1e-5, atol=1e-30)
            assert float(mx[i]) == np.float32(m)
            np.testing.assert_allclose(float(sp[i]), s, rtol=1e-5, atol=1e-30)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [8193, 33001])
def test_row_topk_parity_wide_launch(dtype, V):
    # 260 rows: launches of 256 rows or more reduce chunks of twice the length
    from dynamic_draft_tree_row_amd import api
    n = 260
    base = _rows_with_ties(V, dtype, V + 1)
    g = np.random.default_rng(V)
    extra = np.stack([synth.cast_row((g.standard_normal(V) * g.uniform(0.3, 3)).astype(np.float32), dtype)
                      for _ in range(n - base.shape[0])])
    raw = np.concatenate([base, extra])
    pad = 5
    host = np.zeros((1, n, V + pad), raw.dtype)
    host[0, :, :V] = raw
    x = H.to_dev(host, dtype)[:, :, :V]
    for K in (1, 10, 32):
        say(f"row_topk wide dtype={dtype} V={V} K={K}")
        ws = torch.empty(api.workspace_bytes(n, V, x.dtype, K), dtype=torch.uint8, device="cuda")
        ids = torch.empty((n, K), dtype=torch.int32, device="cuda")
        lc = torch.empty((n, K), dtype=torch.float32, device="cuda")
        mx = torch.empty(n, dtype=torch.float32, device="cuda")
        sp = torch.empty(n, dtype=torch.float32, device="cuda")
        api.row_topk(x, K, ws, ids, lc, mx, sp)
        torch.cuda.synchronize()
        ids_h, lc_h, mx_h, sp_h = ids.cpu().numpy(), lc.cpu().numpy(), mx.cpu().numpy(), sp.cpu().numpy()
        for i in range(n):
            l = O.decode(raw[i], dtype)
            m, _, s_ = O.row_stats(l)
            want = O.topk_ids(l, K)
            assert ids_h[i].tolist() == want.tolist(), f"row {i} K={K}"
            np.testing.assert_allclose(lc_h[i], O.log_conf(l, want, m, s_), rtol=1e-5, atol=1e-30)
            assert mx_h[i] == np.float32(m)
            np.testing.assert_allclose(sp_h[i], s_, rtol=1e-5, atol=1e-30)


# ---------------------------------------------------------------------------
# whole rounds, small vocabularies
# ---------------------------------------------------------------------------

def _case(w, seed, rnd, rows=None, M=None, tau=None):
    cast = H.cast_params(w) if w.cast else None
    graft = H.graft_params(w, tau) if w.graft else None
    M0 = M
    return H.oracle_case(w, seed, rnd, rows=rows, cast=cast, graft=graft, M=M, M0=M0)


SMALL = {
    "eagle2_f32": configs.shrink(configs.C1, V=5000, B=2),
    "cast": configs.shrink(configs.C2, V=17000),
    "cast_b12": configs.shrink(configs.C2, V=9000, B=12),       # more workgroups sharing the layer ticket
    "t1": configs.shrink(configs.C3, V=9001, B=4),            # odd V: unaligned bf16 rows
    "mixed_prefix": configs.shrink(configs.C5, V=4100, B=6),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_round_small(name, seed):
    w = SMALL[name]
    for rnd in range(2):
        case = _case(w, seed, rnd)
        say(f"round {name} seed={seed} round={rnd} B={w.B} V={w.V} tries={case.tries}")
        H.compare(case, H.gpu_round(case))


def test_cast_seeded_cost_table():
    cs = configs.CastSpec(table="seeded", C1=0.5, C2=0.05, C3=0.3)
    w = configs.Workload(**{**SMALL["cast"].__dict__, "cast": cs, "name": "cast_seeded"})
    cast = H.cast_params(w, seed=9)
    for seed in (3, 4):
        case = H.oracle_case(w, seed, 0, cast=cast)
        say(f"cast seeded table seed={seed}")
        H.compare(case, H.gpu_round(case))


@pytest.mark.parametrize("table_B,C1,C2,C3", [(64, 10.0, 0.5, 0.5), (16, 2.0, 1.0, 0.3)])
def test_cast_roofline_cost_table(table_B, C1, C2, C3):
    # MI355X-shaped costs: flat while a forward is HBM-bound (equal neighbouring
    # costs, the zero-cost-step branch of the width and verify scans), rising
    # once it is MFMA-bound
    cs = configs.CastSpec(table="roofline", table_B=table_B, C1=C1, C2=C2, C3=C3)
    w = configs.Workload(**{**SMALL["cast"].__dict__, "cast": cs, "name": f"cast_roofline_{table_B}"})
    cast = H.cast_params(w)
    for seed in (3, 4):
        case = H.oracle_case(w, seed, 0, cast=cast)
        say(f"cast roofline table B={table_B} seed={seed} m={case.out['m_rows'].tolist()}")
        H.compare(case, H.gpu_round(case))


def test_graft_small_multi_round():
    w = configs.shrink(configs.C4, V=6000, B=5)
    tau = H.calibrate_tau(w, 77, 4)
    M = synth.succ_matrix0(w, 77)
    M0 = M.copy()
    for rnd in range(3):
        case = H.oracle_case(w, 77, rnd, cast=None, graft=H.graft_params(w, tau), M=M, M0=M0)
        say(f"graft round {rnd} k_draft={case.out['draft'].k_draft}")
        H.compare(case, H.gpu_round(case))
        M = case.M_after


def test_graft_stochastic_verify_point_mass():
    # Graft with T > 0: retrieval nodes are verified with point-mass
    # proposals (accepted with probability p(x), rejected tokens leave the
    # residual), so a T = 1 request's walk can run through grafted chains
    # (seed 83: the T = 1 walks accept 8 retrieval nodes over the 3 rounds,
    # a chain of 3 among them, and reject others)
    base = configs.shrink(configs.C4, V=6000, B=6)
    w = configs.Workload(**{**base.__dict__, "verify": "t1", "name": base.name + "_t1"})
    tau = H.calibrate_tau(w, 83, 4)
    M = synth.succ_matrix0(w, 83)
    M0 = M.copy()
    for rnd in range(3):
        case = H.oracle_case(w, 83, rnd, cast=None, graft=H.graft_params(w, tau), M=M, M0=M0)
        say(f"graft T>0 round {rnd} k_draft={case.out['draft'].k_draft} "
            f"accept={case.out['accept_len'].tolist()}")
        H.compare(case, H.gpu_round(case))
        M = case.M_after


@pytest.mark.parametrize("verify", ["greedy", "t1"])
@pytest.mark.parametrize("mode", ["root_only", "tail_only"])
def test_graft_variants(mode, verify):
    # the two grafts prune-then-graft is compared with (Graft review, Fig. 2):
    # a fixed draft budget with no checkpoints, the template under the root or
    # under the tail of the selected draft tree
    base = configs.shrink(configs.C4, V=6000, B=5)
    gs = dataclasses.replace(base.graft, mode=mode)
    w = configs.Workload(**{**base.__dict__, "graft": gs, "verify": verify,
                            "name": f"{base.name}_{mode}_{verify}"})
    M = synth.succ_matrix0(w, 61)
    M0 = M.copy()
    for rnd in range(2):
        case = H.oracle_case(w, 61, rnd, graft=H.graft_params(w, None), M=M, M0=M0)
        say(f"graft {mode} {verify} round {rnd} m={case.out['m_rows'].tolist()} "
            f"accept={case.out['accept_len'].tolist()}")
        H.compare(case, H.gpu_round(case))
        M = case.M_after


def test_graft_shared_successor_matrix():
    # one successor matrix for the whole batch (row stride 0): every request
    # reads it in the draft phase, refreshes land in request order
    w = configs.shrink(configs.C4, V=5000, B=4)
    tau = H.calibrate_tau(w, 91, 4)
    M = synth.succ_matrix0(w, 91)[0].copy()
    M0 = M.copy()
    for rnd in range(2):
        case = H.oracle_case(w, 91, rnd, graft=H.graft_params(w, tau), M=M, M0=M0, shared_M=True)
        say(f"graft shared-M round {rnd} k_draft={case.out['draft'].k_draft}")
        H.compare(case, H.gpu_round(case))
        M = case.M_after


def test_determinism_bitwise():
    w = SMALL["mixed_prefix"]
    case = _case(w, 5, 0)
    a = H.gpu_round(case)
    b = H.gpu_round(case)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


@pytest.mark.parametrize("shape", [
    dict(V=16, D=2, K_e=2, K_n=2, m=60),        # fewer nodes than the budget
    dict(V=64, D=1, K_e=1, K_n=5, m=3),         # one layer
    dict(V=300, D=11, K_e=1, K_n=1, m=11),      # deepest chain
    dict(V=9000, D=3, K_e=32, K_n=32, m=255),   # widest frontier, largest budget
])
def test_round_edge_shapes(shape):
    w = configs.Workload("edge", B=3, dtype="bf16", verify="mixed", sigma=0.5, prefix=7, **shape)
    case = _case(w, 11, 0)
    say(f"edge {shape}")
    H.compare(case, H.gpu_round(case))


# ---------------------------------------------------------------------------
# full-size workloads, the bench's launch configuration
# ---------------------------------------------------------------------------

def _tau_golden():
    return json.load(open(os.path.join(GOLDEN, "graft_tau.json")))["tau"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [configs.C1, configs.C2, configs.C3, configs.C4],
                         ids=lambda c: c.name)
def test_round_full(cfg):
    M = synth.succ_matrix0(cfg, 1000) if cfg.graft else None
    case = _case(cfg, 1000 + configs.ORDER.index(cfg), 0, M=M,
                 tau=_tau_golden() if cfg.graft else None)
    say(f"full {cfg.name} tries={case.tries}")
    H.compare(case, H.gpu_round(case))


@pytest.mark.timeout(900)
def test_round_full_b64_sampled_rows():
    w = configs.C5
    rows = [0, 13, 27, 41, 63]
    case = _case(w, 1005, 0, rows=rows)
    say(f"full {w.name} sampled rows {rows} tries={case.tries}")
    r = H.gpu_round_full(case)
    sub = {k: (v[rows] if k != "widths" else v) for k, v in r.items()}
    H.compare(case, sub)
    H.check_invariants(r, w)
