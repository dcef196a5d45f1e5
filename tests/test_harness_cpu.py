"""CPU half of the parity harness: every workload shape yields margin-clean
oracle rounds whose outputs satisfy the method's invariants."""
import math

import numpy as np
import pytest

from gen import configs, synth
from oracle import ddt_oracle as O
from tests import harness as H


def small(cfg, V, B=None):
    return configs.shrink(cfg, V=V, B=B)


@pytest.mark.parametrize("cfg,V,B", [(configs.C1, 3000, None), (configs.C2, 2000, 4),
                                     (configs.C3, 2500, 3), (configs.C5, 1500, 4)])
def test_oracle_case_invariants(cfg, V, B):
    w = small(cfg, V, B)
    cast = H.cast_params(w) if w.cast else None
    case = H.oracle_case(w, seed=3, rnd=0, cast=cast)
    o = case.out
    assert not O.margin_failures(o["margins"])
    for b, t in enumerate(o["draft"].trees):
        f = o["flats"][b]
        m = int(o["m_rows"][b])
        assert 1 <= m <= w.m_max
        n = len([x for x in f.node if x >= 0])
        assert n == m + 1
        L = int(o["accept_len"][b])
        path = o["accept_path"][b]
        assert path[0] == 0 and (path[L + 1:] == -1).all()
        for s in range(1, L + 1):
            assert f.parent[path[s]] == path[s - 1]
    assert case.target.shape == (len(case.rows), w.m_max + 1, w.V)


def test_graft_case_runs_with_stages():
    w = small(configs.C4, 3000, 6)
    M0 = synth.succ_matrix0(w, 11)
    tau = [0.5, 0.3, 0.05]
    case = H.oracle_case(w, seed=4, rnd=0, graft=H.graft_params(w, tau), M=M0, M0=M0)
    o = case.out
    assert (o["m_rows"] == w.graft.K_max).all()
    assert set(o["draft"].k_draft) <= {8, 24, 40, 60}
    assert not np.array_equal(case.M_after, case.M_before)
