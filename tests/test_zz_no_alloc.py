"""ddt_row_topk_noalloc, the row reduction for callers that cannot allocate,
against ddt_row_topk on the same inputs, through the C ABI: two calls in a row,
the second on a smaller input, outputs bitwise equal to the workspace entry
point's (same kernels, same chunking) and equal to the oracle on sampled rows;
a request past the fixed array is refused on the host."""
import ctypes as C

import numpy as np
import pytest
import torch

from oracle import ddt_oracle as O
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    from dynamic_draft_tree_row_amd import _lib
    _lib.load()      # raises if the library was not built: no fallback


def _rows(n, V, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(n, V, device="cuda", generator=g)
    x = x * (0.3 + 2.7 * torch.rand(n, 1, device="cuda", generator=g))
    return x.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def _both(x, K):
    from dynamic_draft_tree_row_amd import api
    n0, n1, _ = x.shape
    out = []
    for noalloc in (False, True):
        ids = torch.full((n0 * n1, K), -7, dtype=torch.int32, device="cuda")
        lc = torch.full((n0 * n1, K), 7.0, dtype=torch.float32, device="cuda")
        mx = torch.full((n0 * n1,), 7.0, dtype=torch.float32, device="cuda")
        sp = torch.full((n0 * n1,), 7.0, dtype=torch.float32, device="cuda")
        if noalloc:
            api.row_topk_noalloc(x, K, ids, lc, mx, sp)
        else:
            ws = torch.empty(api.workspace_bytes(n0 * n1, x.shape[2], x.dtype, K), dtype=torch.uint8,
                             device="cuda")
            api.row_topk(x, K, ws, ids, lc, mx, sp)
        torch.cuda.synchronize()
        out.append([t.cpu().numpy() for t in (ids, lc, mx, sp)])
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_row_topk_matches_workspace_entry_point(dtype):
    # first call: 1024 rows of 128256 (the wide-chunk launch, K = 16); second
    # call: 15 rows of 33001 with K = 10, on the array the first call filled
    for n0, n1, V, K in ((64, 16, 128256, 16), (3, 5, 33001, 10)):
        print(f"noalloc row_topk dtype={dtype} rows={n0 * n1} V={V} K={K}", flush=True)
        x = _rows(n0 * n1, V, dtype, seed=V + K).view(n0, n1, V)
        (ia, la, ma, sa), (ib, lb, mb, sb) = _both(x, K)
        np.testing.assert_array_equal(ib, ia)
        np.testing.assert_array_equal(lb.view(np.uint32), la.view(np.uint32))
        np.testing.assert_array_equal(mb.view(np.uint32), ma.view(np.uint32))
        np.testing.assert_array_equal(sb.view(np.uint32), sa.view(np.uint32))
        host = x.reshape(n0 * n1, V).float().cpu().numpy().astype(np.float64)
        for r in (0, n0 * n1 // 2, n0 * n1 - 1):
            l = host[r]
            m, _, s = O.row_stats(l)
            want = O.topk_ids(l, K)
            assert ib[r].tolist() == want.tolist(), f"row {r}"
            np.testing.assert_allclose(lb[r], O.log_conf(l, want, m, s), rtol=1e-5, atol=1e-30)
            assert mb[r] == np.float32(m)
            np.testing.assert_allclose(sb[r], s, rtol=1e-5, atol=1e-30)


def test_noalloc_row_topk_refuses_past_the_array():
    from dynamic_draft_tree_row_amd import _lib
    lib = _lib.load()
    x = _rows(4, 128256, "bf16", seed=1)
    V = x.shape[1]
    rows, K = 2048, 32                      # 2048 x 16 chunks x 264 B > 8 MiB
    need = int(lib.ddt_workspace_bytes(rows, V, _lib.DDT_BF16, K))
    assert need > _lib.DDT_NOALLOC_SCRATCH_BYTES
    d = _lib.Logits(C.c_void_p(x.data_ptr()), _lib.DDT_BF16, V, 0, 0)   # stride 0: never read
    st = lib.ddt_row_topk_noalloc(C.byref(d), rows, 1, K, None, None, None, None, None)
    assert st == 3                          # DDT_ECAPACITY, refused before any launch
    ok = int(lib.ddt_workspace_bytes(1024, V, _lib.DDT_BF16, K))
    assert ok <= _lib.DDT_NOALLOC_SCRATCH_BYTES
