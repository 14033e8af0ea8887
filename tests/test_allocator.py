"""Allocator: the oracle model pinned to the page-4 queue semantics worked by
hand and to invariants; then libpkv's host allocator (host-only pools, no
GPU) against the oracle on random operation scripts, bit for bit."""
import numpy as np
import pytest

from oracle import oracle as orc


def test_page4_queue_walkthrough(oracle_lib):
    """allocate takes from the front, free returns to the back, append_block
    takes the front or reports 'wait' ("连续批处理与KV缓存" §4.2), worked by hand
    for 8 blocks of 4 tokens."""
    a = orc.Allocator(8, 4)
    st, slots = a.allocate(100, 12)            # A: 3 blocks -> 0, 1, 2
    assert st == orc.OK and list(slots) == list(range(12))
    st, slots = a.allocate(200, 5)             # B: 2 blocks -> 3, 4
    assert st == orc.OK and list(slots) == [12, 13, 14, 15, 16]
    assert list(a.free_queue()) == [5, 6, 7]
    assert a.free(100) == orc.OK               # A's blocks go to the back
    assert list(a.free_queue()) == [5, 6, 7, 0, 1, 2]
    st, slots = a.append([200], [4])           # B grows 5 -> 9 tokens: row 1 of 4, then block 5
    assert st == orc.OK and list(slots) == [17, 18, 19, 20]
    st, _, _ = a.table([200], 4)
    st, table, lens = a.table([200], 4)
    assert list(table[0]) == [3, 4, 5, -1] and lens[0] == 9
    st, slots = a.allocate(300, 16)            # C: 4 blocks -> 6, 7, 0, 1
    assert st == orc.OK and list(slots[::4]) == [24, 28, 0, 4]
    assert list(a.free_queue()) == [2]
    st, _ = a.allocate(400, 5)                 # needs 2, one free: out of memory, no change
    assert st == orc.OOM and list(a.free_queue()) == [2] and a.stats()["seqs"] == 2
    st, _ = a.append([200, 300], [3, 1])       # B: 9 -> 12 fits block 5; C: 16 -> 17 needs one
    assert st == orc.OK and list(a.free_queue()) == []
    st, _ = a.append([300], [3])               # C: 17 -> 20 fills block 2; one more needs a block
    assert st == orc.OK
    st, _ = a.append([300], [1])
    assert st == orc.NO_FREE_BLOCK              # "return False: needs to wait"
    assert a.free(999) == orc.OK                # unknown id: no-op
    assert a.allocate(200, 1)[0] == orc.SEQ_EXISTS


def test_600_token_sequence_uses_38_blocks(oracle_lib):
    a = orc.Allocator(64, 16)
    st, slots = a.allocate(0, 600)
    assert st == orc.OK and a.stats()["used"] == 38
    st, table, lens = a.table([0], 40)
    assert (table[0] >= 0).sum() == 38 and lens[0] == 600
    assert 38 * 16 - 600 == 8


def test_shared_prefix_copy_on_write(oracle_lib):
    """200-token prefix at bs 16 (12 full blocks + 8 rows), forked 127 times;
    every sequence then appends. The first 127 writers find the partial block
    shared and copy it; the last one writes in place."""
    a = orc.Allocator(2000, 16)
    assert a.allocate(0, 200)[0] == orc.OK
    for c in range(1, 128):
        assert a.fork(0, c) == orc.OK
    s = a.stats()
    assert s["used"] == 13 and s["shared"] == 13
    assert all(a.refcount(b) == 128 for b in range(13))
    st, slots = a.append(list(range(128)), [1] * 128)
    assert st == orc.OK
    cows = a.take_cows()
    assert len(cows) == 127 and a.stats()["cow"] == 127
    assert set(cows[:, 0]) == {12} and set(cows[:, 2]) == {8}   # the partial block, 8 rows
    assert slots[127] == 12 * 16 + 8                              # last writer: in place
    assert a.refcount(12) == 1 and a.refcount(0) == 128
    s = a.stats()
    assert s["used"] == 13 + 127 and s["shared"] == 12


def test_append_all_or_nothing(oracle_lib):
    a = orc.Allocator(4, 16)
    assert a.allocate(0, 24)[0] == orc.OK  # 2 blocks
    assert a.fork(0, 1) == orc.OK
    before = (list(a.free_queue()), a.stats())
    # seq 0 needs a copy (shared partial block), seq 1 then writes in place,
    # and 30 more tokens for seq 1 (24 -> 54) need 2 new blocks: 3 > 2 free
    st, _ = a.append([0, 1], [1, 30])
    assert st == orc.NO_FREE_BLOCK
    assert (list(a.free_queue()), a.stats()) == before
    st, _ = a.append([0, 1], [1, 9])        # 1 copy + 1 new block (24 -> 33) = 2
    assert st == orc.OK and a.stats()["free"] == 0


def _invariants(a: orc.Allocator, live):
    N = a.num_blocks
    fq = list(a.free_queue())
    assert len(set(fq)) == len(fq)
    holders = {}
    if live:
        st, table, lens = a.table(sorted(live), N)
        assert st == orc.OK
        for i, s in enumerate(sorted(live)):
            nb = (int(lens[i]) + a.block_size - 1) // a.block_size
            assert (table[i] >= 0).sum() == nb
            for b in table[i, :nb]:
                holders[int(b)] = holders.get(int(b), 0) + 1
    for b in range(N):
        assert a.refcount(b) == holders.get(b, 0)
        assert (b in fq) == (holders.get(b, 0) == 0)
    assert len(fq) + len(holders) == N


def random_script(rng, steps, max_seq=12):
    ops = []
    live, nxt = set(), 0
    for _ in range(steps):
        r = rng.random()
        if r < 0.3 or not live:
            ops.append(("allocate", nxt, int(rng.integers(0, 70))))
            live.add(nxt)
            nxt += 1
        elif r < 0.45:
            p = int(rng.choice(sorted(live)))
            ops.append(("fork", p, nxt))
            live.add(nxt)
            nxt += 1
        elif r < 0.6:
            s = int(rng.choice(sorted(live)))
            ops.append(("free", s))
            live.discard(s)
        else:
            k = int(rng.integers(1, min(len(live), 5) + 1))
            seqs = [int(x) for x in rng.choice(sorted(live), size=k, replace=False)]
            ops.append(("append", seqs, [int(rng.integers(0, 20)) for _ in seqs]))
        if len(live) > max_seq:
            s = int(rng.choice(sorted(live)))
            ops.append(("free", s))
            live.discard(s)
    return ops


@pytest.mark.parametrize("seed", range(6))
def test_oracle_invariants_random_scripts(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    N, bs = int(rng.integers(8, 65)), int(rng.choice([16, 32]))
    a = orc.Allocator(N, bs, rng.permutation(N))
    live = set()
    for op in random_script(rng, 300):
        if op[0] == "allocate":
            st, _ = a.allocate(op[1], op[2])
            if st == orc.OK:
                live.add(op[1])
        elif op[0] == "fork":
            if op[1] in live and a.fork(op[1], op[2]) == orc.OK:
                live.add(op[2])
        elif op[0] == "free":
            a.free(op[1])
            live.discard(op[1])
        else:
            seqs = [s for s in op[1] if s in live]
            a.append(seqs, op[2][: len(seqs)])
        _invariants(a, live)


def _lib_pool(N, bs, order):
    from paged_kv_cache_62_amd import pkv
    return pkv.Pool(1, 2, 64, bs, N, pkv.PKV_I8, initial_free_order=order, host_only=True)


@pytest.mark.parametrize("seed", range(8))
def test_library_allocator_matches_oracle(oracle_lib, seed):
    """Same script on libpkv's host allocator and the oracle: identical
    statuses, slots, tables, lengths, free queues and statistics."""
    from paged_kv_cache_62_amd import pkv
    rng = np.random.default_rng(200 + seed)
    N, bs = int(rng.integers(8, 97)), int(rng.choice([16, 32, 64]))
    order = rng.permutation(N).astype(np.int32)
    a = orc.Allocator(N, bs, order)
    p = _lib_pool(N, bs, order)
    codes = {orc.OK: pkv.PKV_OK, orc.OOM: pkv.PKV_ERR_OOM, orc.NO_FREE_BLOCK: pkv.PKV_ERR_NO_FREE_BLOCK,
             orc.UNKNOWN_SEQ: pkv.PKV_ERR_UNKNOWN_SEQ, orc.SEQ_EXISTS: pkv.PKV_ERR_SEQ_EXISTS,
             orc.INVALID: pkv.PKV_ERR_INVALID_ARG}
    live = set()

    def lib_call(fn, *args):
        try:
            return pkv.PKV_OK, fn(*args)
        except pkv.PkvError as e:
            return e.status, None

    for op in random_script(rng, 400):
        if op[0] == "allocate":
            st, slots = a.allocate(op[1], op[2])
            gst, gslots = lib_call(p.allocate, op[1], op[2])
            assert gst == codes[st]
            if st == orc.OK:
                np.testing.assert_array_equal(gslots, slots)
                live.add(op[1])
        elif op[0] == "fork":
            st = a.fork(op[1], op[2])
            gst, _ = lib_call(p.fork, op[1], op[2])
            assert gst == codes[st]
            if st == orc.OK:
                live.add(op[2])
        elif op[0] == "free":
            assert a.free(op[1]) == orc.OK
            assert lib_call(p.free, op[1])[0] == pkv.PKV_OK
            live.discard(op[1])
        else:
            st, slots = a.append(op[1], op[2])
            gst, gslots = lib_call(p.append_slots, op[1], op[2])
            assert gst == codes[st]
            if st == orc.OK:
                np.testing.assert_array_equal(gslots, slots)
        np.testing.assert_array_equal(p.free_queue(), a.free_queue())
        s, gs = a.stats(), p.stats()
        assert (gs["free_blocks"], gs["used_blocks"], gs["shared_blocks"], gs["cow_copies"], gs["num_seqs"]) == \
            (s["free"], s["used"], s["shared"], s["cow"], s["seqs"])
        if live:
            seqs = sorted(live)
            st, table, lens = a.table(seqs, N)
            gt, gl = p.block_table(seqs, N)
            np.testing.assert_array_equal(gt, table)
            np.testing.assert_array_equal(gl, lens)


def test_library_error_paths_leave_state_unchanged(oracle_lib):
    from paged_kv_cache_62_amd import pkv
    p = _lib_pool(6, 16, None)
    p.allocate(1, 40)                       # 3 blocks
    before = (p.free_queue().tolist(), p.stats())
    with pytest.raises(pkv.PkvError) as e:
        p.allocate(2, 64)                   # 4 > 3 free
    assert e.value.status == pkv.PKV_ERR_OOM
    with pytest.raises(pkv.PkvError) as e:
        p.append_slots([1], [60])           # 40 -> 100 tokens needs 4 more
    assert e.value.status == pkv.PKV_ERR_NO_FREE_BLOCK
    with pytest.raises(pkv.PkvError) as e:
        p.append_slots([1, 9], [1, 1])
    assert e.value.status == pkv.PKV_ERR_UNKNOWN_SEQ
    with pytest.raises(pkv.PkvError) as e:
        p.append_slots([1, 1], [1, 1])
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        p.fork(1, 1)
    assert e.value.status == pkv.PKV_ERR_SEQ_EXISTS
    with pytest.raises(pkv.PkvError) as e:
        p.fork(7, 8)
    assert e.value.status == pkv.PKV_ERR_UNKNOWN_SEQ
    with pytest.raises(pkv.PkvError) as e:
        p.block_table([1], 2)               # holds 3 blocks
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    assert (p.free_queue().tolist(), p.stats()) == before
    p.free(12345)                           # unknown: no-op
    assert (p.free_queue().tolist(), p.stats()) == before


def test_order_longest_first(oracle_lib):
    """pkv_seq_order_longest_first: the ids sorted by current length, longest
    first, equal lengths in the given order (stable); lengths as the pool
    holds them after forks and appends; an unknown id is an error."""
    from paged_kv_cache_62_amd import pkv
    p = _lib_pool(64, 16, None)
    lens = {10: 33, 11: 200, 12: 33, 13: 1, 14: 200, 15: 64}
    for s, n in lens.items():
        p.allocate(s, n)
    ids = [13, 10, 15, 12, 11, 14]
    got = p.order_longest_first(ids).tolist()
    assert got == [11, 14, 15, 10, 12, 13]
    assert got == sorted(ids, key=lambda s: (-lens[s], ids.index(s)))
    p.fork(13, 20)                          # 1 token, shares the block
    p.append_slots([20], [99])              # 100 tokens now
    assert p.order_longest_first([13, 20, 15]).tolist() == [20, 15, 13]
    assert p.order_longest_first([]).tolist() == []
    with pytest.raises(pkv.PkvError) as e:
        p.order_longest_first([10, 99])
    assert e.value.status == pkv.PKV_ERR_UNKNOWN_SEQ
