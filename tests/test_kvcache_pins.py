"""Pins of the paged-KV commit oracle: a hand-worked example whose block ids
follow from the free-stack discipline by hand, closed forms (a context is the
concatenation of everything committed to it), holder-count invariants after
every operation, copy-on-write isolation, and each status case."""
import numpy as np

from oracle import ddt_kvcache as KV


def _rows(rng, B, P, H, D):
    k = rng.integers(0, 1 << 16, size=(B, P, H, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(B, P, H, D), dtype=np.uint16)
    return k, v


def _check_invariants(st):
    n_blocks = st["ref"].shape[0]
    holders = np.zeros(n_blocks, np.int64)
    bs = st["block"]
    for b in range(st["table"].shape[0]):
        row = st["table"][b]
        used = -(-int(st["len"][b]) // bs)
        assert (row[:used] >= 0).all() and (row[used:] == -1).all(), f"table row {b} vs len"
        assert len(set(row[:used].tolist())) == used, "a block twice in one row"
        for x in row[:used]:
            holders[x] += 1
    assert (holders == st["ref"]).all(), "ref differs from the number of holders"
    free = st["free_ids"][:st["n_free"]].tolist()
    assert len(free) == len(set(free)), "a block twice on the free stack"
    assert set(free) == set(np.flatnonzero(st["ref"] == 0).tolist()), "free stack != blocks with no holder"


def test_hand_worked_example():
    # 3 requests, blocks of 4 tokens, 6 blocks; the stack starts [5 4 3 2 1 0]
    # with block 0 on top
    st = KV.new_state(B=3, max_blocks=4, n_blocks=6, block=4, Hkv=1, D=8)
    rng = np.random.default_rng(0)
    k, v = _rows(rng, 3, 7, 1, 8)
    path = np.array([[0, 2, 5, -1, -1, -1, -1], [0, 1, 3, 4, 5, 6, -1], [0, -1, -1, -1, -1, -1, -1]])
    # request 0 commits 3 tokens (one block: 0), request 1 six tokens (blocks
    # 1 then 2), request 2 nothing
    s = KV.commit(st, np.array([2, 5, -1]), path, k, v)
    assert s.tolist() == [3, 6, 0]
    assert st["table"][0].tolist() == [0, -1, -1, -1]
    assert st["table"][1].tolist() == [1, 2, -1, -1]
    assert st["n_free"] == 3 and st["free_ids"][:3].tolist() == [5, 4, 3]
    # request 2 shares request 0's context
    assert KV.fork(st, np.array([0]), np.array([2])).tolist() == [0]
    assert st["table"][2].tolist() == [0, -1, -1, -1] and st["ref"][0] == 2
    # request 2 appends 2 tokens: block 0 is shared and partly filled, so it is
    # copied to block 3 (top of the stack), and token 4 goes to block 4
    path2 = np.array([[-1] * 7, [-1] * 7, [1, 6, -1, -1, -1, -1, -1]])
    assert KV.commit(st, np.array([-1, -1, 1]), path2, k, v).tolist() == [0, 0, 2]
    assert st["table"][2].tolist() == [3, 4, -1, -1]
    assert st["ref"][0] == 1 and st["ref"][3] == 1 and st["ref"][4] == 1
    assert st["n_free"] == 1 and st["free_ids"][0] == 5
    k2, _ = KV.context(st, 2)
    assert (k2[:3] == k[0, [0, 2, 5]]).all() and (k2[3:] == k[2, [1, 6]]).all()
    k0, _ = KV.context(st, 0)
    assert (k0 == k[0, [0, 2, 5]]).all()
    # releasing request 0 frees block 0 (pushed on top of block 5)
    KV.release(st, np.array([0]))
    assert st["n_free"] == 2 and st["free_ids"][:2].tolist() == [5, 0]
    _check_invariants(st)


def test_context_is_the_concatenation_of_commits():
    rng = np.random.default_rng(1)
    B, P, H, D, bs = 5, 9, 2, 8, 4
    st = KV.new_state(B, max_blocks=12, n_blocks=64, block=bs, Hkv=H, D=D)
    want = [[] for _ in range(B)]
    for _ in range(8):
        k, v = _rows(rng, B, P, H, D)
        acc = rng.integers(-1, 6, size=B)
        path = np.full((B, P), -1)
        for b in range(B):
            if acc[b] >= 0:
                path[b, :acc[b] + 1] = rng.permutation(P)[:acc[b] + 1]
        s = KV.commit(st, acc, path, k, v)
        for b in range(B):
            assert s[b] == max(acc[b] + 1, 0)
            for p in path[b, :max(acc[b] + 1, 0)]:
                want[b].append((k[b, p], v[b, p]))
        _check_invariants(st)
    for b in range(B):
        kb, vb = KV.context(st, b)
        assert len(kb) == len(want[b])
        for t, (kk, vv) in enumerate(want[b]):
            assert (kb[t] == kk).all() and (vb[t] == vv).all()


def test_copy_on_write_isolates_forks():
    rng = np.random.default_rng(2)
    B, P, H, D, bs = 4, 8, 1, 8, 4
    st = KV.new_state(B, max_blocks=8, n_blocks=32, block=bs, Hkv=H, D=D)
    k, v = _rows(rng, B, P, H, D)
    KV.commit(st, np.array([5, -1, -1, -1]), np.tile(np.arange(P), (B, 1)), k, v)   # 6 tokens: 1.5 blocks
    assert KV.fork(st, np.array([0, 0]), np.array([1, 2])).tolist() == [0, 0]
    full, tail = st["table"][0][0], st["table"][0][1]
    assert st["ref"][full] == 3 and st["ref"][tail] == 3
    before, _ = KV.context(st, 0)
    # requests 1 and 2 append in the same call: both copy the shared tail,
    # the full block stays shared
    k2, v2 = _rows(rng, B, P, H, D)
    s = KV.commit(st, np.array([-1, 2, 1, -1]), np.tile(np.arange(P), (B, 1)), k2, v2)
    assert s.tolist() == [0, 3, 2, 0]
    assert st["ref"][full] == 3 and st["ref"][tail] == 1
    after, _ = KV.context(st, 0)
    assert (after == before).all()
    for b, n in ((1, 3), (2, 2)):
        kb, _ = KV.context(st, b)
        assert (kb[:6] == before).all() and (kb[6:] == k2[b, :n]).all()
        assert st["table"][b][0] == full and st["table"][b][1] != tail
    _check_invariants(st)
    # all holders appending at once: the tail is copied by every one of them
    # and, left with no holder, goes back on the stack
    st2 = KV.new_state(B, max_blocks=8, n_blocks=32, block=bs, Hkv=H, D=D)
    KV.commit(st2, np.array([5, -1, -1, -1]), np.tile(np.arange(P), (B, 1)), k, v)
    KV.fork(st2, np.array([0]), np.array([1]))
    t2 = st2["table"][0][1]
    n_free = st2["n_free"]
    KV.commit(st2, np.array([0, 0, -1, -1]), np.tile(np.arange(P), (B, 1)), k2, v2)
    assert st2["ref"][t2] == 0 and st2["free_ids"][st2["n_free"] - 1] == t2
    assert st2["n_free"] == n_free - 2 + 1
    _check_invariants(st2)


def test_release_returns_blocks_only_after_the_last_holder():
    rng = np.random.default_rng(3)
    B, P, bs = 3, 10, 4
    st = KV.new_state(B, max_blocks=4, n_blocks=16, block=bs, Hkv=1, D=8)
    k, v = _rows(rng, B, P, 1, 8)
    KV.commit(st, np.array([8, -1, -1]), np.tile(np.arange(P), (B, 1)), k, v)      # 9 tokens, 3 blocks
    KV.fork(st, np.array([0]), np.array([1]))
    n0 = st["n_free"]
    KV.release(st, np.array([0]))
    assert st["n_free"] == n0 and st["len"][0] == 0
    KV.release(st, np.array([1, 1]))
    assert st["n_free"] == n0 + 3
    _check_invariants(st)
    assert st["n_free"] == 16


def test_status_cases():
    rng = np.random.default_rng(4)
    B, P, bs = 4, 6, 2
    k, v = _rows(rng, B, P, 1, 8)
    path = np.tile(np.arange(P), (B, 1))
    # capacity: max_blocks * block = 4 tokens
    st = KV.new_state(B, max_blocks=2, n_blocks=40, block=bs, Hkv=1, D=8)
    assert KV.commit(st, np.array([4, 3, -1, 0]), path, k, v).tolist() == [-1, 4, 0, 1]
    # invalid path entries
    bad = path.copy()
    bad[1, 1] = P
    st = KV.new_state(B, max_blocks=8, n_blocks=40, block=bs, Hkv=1, D=8)
    assert KV.commit(st, np.array([1, 1, 1, 1]), bad, k, v).tolist() == [2, -3, 2, 2]
    # exhaustion: 5 free blocks; requests need 2, 3, 1, 1 -> the third does
    # not fit, and the fourth is refused after it although it would fit
    st = KV.new_state(B, max_blocks=8, n_blocks=5, block=bs, Hkv=1, D=8)
    assert KV.commit(st, np.array([3, 5, 1, 0]), path, k, v).tolist() == [4, 6, -2, -2]
    assert st["n_free"] == 0 and st["len"].tolist() == [4, 6, 0, 0]
    _check_invariants(st)
    # a fork onto a non-empty request or onto a source is refused
    assert KV.fork(st, np.array([0, 1]), np.array([1, 0])).tolist() == [-1, -1]
    assert KV.fork(st, np.array([0]), np.array([2])).tolist() == [0]
    _check_invariants(st)
