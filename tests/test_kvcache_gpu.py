"""GPU parity of the paged-KV calls (ddt_kv_commit / fork / release) against
the oracle: random sequences of operations on both sides from the same
start, the whole state compared after every call, bit for bit: the key and
value pools, block tables, lengths, holder counts, the free stack and its
count, and every status.  Key/value rows are random 16-bit patterns, so a
misplaced copy cannot hide behind equal values."""
import numpy as np
import pytest
import torch

from oracle import ddt_kvcache as KV

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    from dynamic_draft_tree_row_amd import _lib
    _lib.load()


def _bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)


def _i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to("cuda")


def _compare(kv, st, what):
    torch.cuda.synchronize()
    k = kv.k.view(torch.int16).cpu().numpy().view(np.uint16)
    v = kv.v.view(torch.int16).cpu().numpy().view(np.uint16)
    assert (k == st["k"]).all(), f"{what}: key pool"
    assert (v == st["v"]).all(), f"{what}: value pool"
    assert (kv.table.cpu().numpy() == st["table"]).all(), f"{what}: block table"
    assert (kv.len.cpu().numpy() == st["len"]).all(), f"{what}: lengths"
    assert (kv.ref.cpu().numpy() == st["ref"]).all(), f"{what}: holder counts"
    nf = int(kv.n_free.cpu()[0])
    assert nf == st["n_free"], f"{what}: free count {nf} vs {st['n_free']}"
    assert (kv.free_ids.cpu().numpy()[:nf] == st["free_ids"][:nf]).all(), f"{what}: free stack"


def _run(seed, B, P, Dp, Hkv, D, block, max_blocks, n_blocks, rounds, p_bad=0.0, forks=True):
    from dynamic_draft_tree_row_amd import api
    rng = np.random.default_rng(seed)
    kv = api.PagedKV(B, max_blocks, n_blocks, block, Hkv, D, "cuda")
    st = KV.new_state(B, max_blocks, n_blocks, block, Hkv, D)
    print(f"kv seed={seed} B={B} P={P} Dp={Dp} HD={Hkv * D} block={block} blocks={n_blocks}", flush=True)
    for rnd in range(rounds):
        kt = rng.integers(0, 1 << 16, size=(B, P, Hkv, D), dtype=np.uint16)
        vt = rng.integers(0, 1 << 16, size=(B, P, Hkv, D), dtype=np.uint16)
        acc = rng.integers(-1, Dp + 1, size=B).astype(np.int32)
        path = np.full((B, Dp + 1), -1, np.int32)
        for b in range(B):
            if acc[b] >= 0:
                path[b, :acc[b] + 1] = rng.permutation(P)[:acc[b] + 1]
                if rng.random() < p_bad:
                    path[b, rng.integers(0, acc[b] + 1)] = P + 3
        status = torch.full((B,), 99, dtype=torch.int32, device="cuda")
        kv.commit(_i32(acc), _i32(path), _bits(kt), _bits(vt), status)
        want = KV.commit(st, acc, path, kt, vt)
        torch.cuda.synchronize()
        assert (status.cpu().numpy() == want).all(), f"round {rnd}: status {status.cpu().numpy()} vs {want}"
        _compare(kv, st, f"round {rnd} commit")
        if forks and rnd % 3 == 1:
            empty = [b for b in range(B) if st["len"][b] == 0 and st["table"][b][0] == -1]
            full = [b for b in range(B) if st["len"][b] > 0]
            if empty and full:
                nf = min(len(empty), 3)
                src = np.array([full[rng.integers(len(full))] for _ in range(nf)], np.int32)
                dst = np.array(empty[:nf], np.int32)
                fs = torch.full((nf,), 99, dtype=torch.int32, device="cuda")
                kv.fork(_i32(src), _i32(dst), fs)
                want = KV.fork(st, src, dst)
                torch.cuda.synchronize()
                assert (fs.cpu().numpy() == want).all(), f"round {rnd}: fork status"
                _compare(kv, st, f"round {rnd} fork")
        if rnd % 4 == 3:
            req = rng.choice(B, size=max(1, B // 3), replace=True).astype(np.int32)
            kv.release(_i32(req))
            KV.release(st, req)
            _compare(kv, st, f"round {rnd} release")


@pytest.mark.parametrize("block", [1, 4, 16])
def test_kv_commit_fork_release_sequences(block):
    _run(seed=10 + block, B=7, P=12, Dp=9, Hkv=1, D=8, block=block, max_blocks=64 // block + 8,
         n_blocks=12 * (64 // block), rounds=12)


def test_kv_free_stack_exhaustion_and_bad_paths():
    # a pool too small for everyone: requests are refused in index order
    _run(seed=3, B=9, P=10, Dp=7, Hkv=2, D=8, block=4, max_blocks=16, n_blocks=14, rounds=10, p_bad=0.2)


def test_kv_context_capacity():
    _run(seed=4, B=5, P=10, Dp=8, Hkv=1, D=16, block=2, max_blocks=6, n_blocks=60, rounds=8)


def test_kv_full_size_mixed_workload_shape():
    # the B = 64 mixed shape: 129 flat positions, 8 key/value heads of 128,
    # 16-token blocks, accepted paths up to depth 10, forks and releases
    _run(seed=5, B=64, P=129, Dp=10, Hkv=8, D=128, block=16, max_blocks=64, n_blocks=2048, rounds=9)


def test_kv_shared_tails_copied_by_every_holder():
    # requests 0..3 get partly filled tails; each is forked to two more; then
    # for requests 0 and 2 every holder appends in one call (their old tails
    # lose all holders and go back on the stack, ordered by lowest copier),
    # for 1 and 3 only some holders do
    from dynamic_draft_tree_row_amd import api
    rng = np.random.default_rng(21)
    B, P, Dp, Hkv, D, block = 12, 9, 6, 2, 8, 4
    kv = api.PagedKV(B, 8, 64, block, Hkv, D, "cuda")
    st = KV.new_state(B, 8, 64, block, Hkv, D)

    def commit(acc):
        kt = rng.integers(0, 1 << 16, size=(B, P, Hkv, D), dtype=np.uint16)
        vt = rng.integers(0, 1 << 16, size=(B, P, Hkv, D), dtype=np.uint16)
        acc = np.asarray(acc, np.int32)
        path = np.full((B, Dp + 1), -1, np.int32)
        for b in range(B):
            if acc[b] >= 0:
                path[b, :acc[b] + 1] = rng.permutation(P)[:acc[b] + 1]
        status = torch.full((B,), 99, dtype=torch.int32, device="cuda")
        kv.commit(_i32(acc), _i32(path), _bits(kt), _bits(vt), status)
        want = KV.commit(st, acc, path, kt, vt)
        torch.cuda.synchronize()
        assert (status.cpu().numpy() == want).all()
        _compare(kv, st, "commit")

    commit([5, 2, 6, 0] + [-1] * 8)                     # tails at 2, 3, 3, 1 tokens
    src = np.array([0, 0, 1, 1, 2, 2, 3, 3], np.int32)
    dst = np.arange(4, 12, dtype=np.int32)
    fs = torch.full((8,), 99, dtype=torch.int32, device="cuda")
    kv.fork(_i32(src), _i32(dst), fs)
    assert (fs.cpu().numpy() == KV.fork(st, src, dst)).all()
    _compare(kv, st, "fork")
    tails = [int(st["table"][b][st["len"][b] // block]) for b in range(4)]
    assert all(st["ref"][t] == 3 for t in tails)
    # holders of 0: {0, 4, 5}; of 1: {1, 6, 7}; of 2: {2, 8, 9}; of 3: {3, 10, 11}
    acc = [1, 0, 2, -1, 0, 3, -1, 1, 0, 0, 2, -1]
    commit(acc)
    assert st["ref"][tails[0]] == 0 and st["ref"][tails[2]] == 0
    assert st["ref"][tails[1]] == 1 and st["ref"][tails[3]] == 2
    top = st["free_ids"][st["n_free"] - 2:st["n_free"]].tolist()
    assert top == [tails[0], tails[2]]                  # pushed by lowest copier: request 0, then 2
    kv.release(_i32(np.arange(B)))
    KV.release(st, np.arange(B))
    _compare(kv, st, "release all")
    assert st["n_free"] == 64


def test_kv_admission_boundaries():
    # the blocks a commit takes are the prefix sum at the last request whose
    # prefix fits: exercised with a stack that runs out part-way, with the
    # first request not fitting (nothing taken; the requests after it that
    # need no block are refused too, admission being in index order), and
    # with admitted requests that take no block before a refused one
    from dynamic_draft_tree_row_amd import api
    rng = np.random.default_rng(33)
    B, P, Dp, Hkv, D, block = 4, 12, 10, 1, 8, 4
    kv = api.PagedKV(B, 8, 3, block, Hkv, D, "cuda")
    st = KV.new_state(B, 8, 3, block, Hkv, D)

    def commit(acc, want_status):
        kt = rng.integers(0, 1 << 16, size=(B, P, Hkv, D), dtype=np.uint16)
        vt = rng.integers(0, 1 << 16, size=(B, P, Hkv, D), dtype=np.uint16)
        acc = np.asarray(acc, np.int32)
        path = np.full((B, Dp + 1), -1, np.int32)
        for b in range(B):
            if acc[b] >= 0:
                path[b, :acc[b] + 1] = rng.permutation(P)[:acc[b] + 1]
        status = torch.full((B,), 99, dtype=torch.int32, device="cuda")
        kv.commit(_i32(acc), _i32(path), _bits(kt), _bits(vt), status)
        want = KV.commit(st, acc, path, kt, vt)
        torch.cuda.synchronize()
        assert list(want) == want_status
        assert (status.cpu().numpy() == want).all(), f"status {status.cpu().numpy()} vs {want}"
        _compare(kv, st, f"commit {list(acc)}")

    commit([1, 1, 1, 1], [2, 2, 2, -2])                 # one block each; the stack runs out at request 3
    assert st["n_free"] == 0
    commit([9, 0, 0, -1], [-2, -2, -2, 0])              # 0 does not fit: nothing is taken, and 1 and 2,
                                                        # which need no block, come after a refusal
    commit([1, 0, 0, 0], [2, 1, 1, -2])                 # 0..2 fit in their tails: the last fitting prefix is 0
    kv.release(_i32(np.array([1], np.int32)))
    KV.release(st, np.array([1], np.int32))
    _compare(kv, st, "release 1")
    assert st["n_free"] == 1
    commit([0, -1, 5, 0], [1, 0, -2, -2])               # 0 takes the one block; 2 needs two more
