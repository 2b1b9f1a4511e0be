"""CPU checks of the per-layer memory policy's host side: the library's ring sizing and block
accounting against the oracle, the block manager's tables and slots against the ring
definition (the oracle's ring columns), all-or-nothing errors, and the validation of ring
tables in the decode calls. Nothing here launches a kernel."""
import ctypes
import json
import os

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_16_amd as m
    return m


def test_ring_sizing_and_blocks_match_the_oracle(pkv):
    with open(os.path.join(ROOT, "tests", "golden", "ring_policy.json")) as f:
        g = json.load(f)
    for c in g["ring_pages"]:
        assert pkv.ring_pages(c["W"], c["P"]) == c["R"], c["what"]
    for c in g["blocks"]:
        assert pkv.policy_blocks(c["L"], c["P"], c["W"], c["S"]) == c["n"], c["what"]
    rng = np.random.default_rng(3)
    for _ in range(2000):
        P = int(rng.choice([16, 32, 48, 256]))
        W = int(rng.integers(-2, 3000))
        S = int(rng.integers(0, 300))
        L = int(rng.integers(0, 40000))
        assert pkv.ring_pages(W, P) == oracle.ring_pages(W, P), (W, P)
        R = 0 if W <= 0 else oracle.ring_pages(W, P) + int(rng.integers(0, 4))
        assert pkv.policy_blocks(L, P, W, S, R) == oracle.policy_blocks(L, P=P, window=W, sinks=S, ring_pages=R)


def _check_state(pkv, bm, groups, lens, P):
    """Blocks in use equal the oracle's count; no block is held twice within a group; every
    held block is in range; free + held = pool."""
    for g, spec in enumerate(groups):
        want = sum(oracle.policy_blocks(L, P=P, window=spec.get("window", 0), sinks=spec.get("num_sinks", 0),
                                        ring_pages=spec.get("ring_pages", 0)) for L in lens.values())
        assert bm.blocks_in_use(g) == want
        ids = sorted(lens)
        if not ids:
            continue
        t = bm.block_table(g, ids)
        held = t[t >= 0]
        assert held.size == want and np.unique(held).size == held.size
        assert held.min(initial=0) >= 0 and held.max(initial=0) < spec["num_blocks"]


def _expected_slots(pkv, bm, group, spec, seq, L0, L1, P):
    """Slots of tokens [L0, L1) of one sequence from its table row and the oracle's ring
    columns; -1 for a window group's token out of sinks and window at L1."""
    row = bm.block_table(group, [seq])[0]
    W, S = spec.get("window", 0), spec.get("num_sinks", 0)
    R = bm.ring_pages(group)
    out = []
    for t in range(L0, L1):
        col = t // P if W <= 0 else oracle.ring_column(t // P, sinks=S, P=P, ring_pages=R)
        live = W <= 0 or t < S or t >= L1 - W
        out.append(int(row[col]) * P + t % P if live else -1)
    return out


def test_block_manager_random_walk(pkv):
    """Random prefills, decode steps and releases over a full group and two window groups:
    slots follow the ring definition, counts follow the oracle, no block is shared."""
    P = 16
    groups = [dict(num_blocks=400), dict(window=40, num_sinks=3, num_blocks=120),
              dict(window=23, num_sinks=20, ring_pages=5, num_blocks=100)]
    bm = pkv.BlockManager(P, 8, 64, groups)
    assert bm.table_cols(0) == 64 and bm.ring_pages(1) == oracle.ring_pages(40, P)
    assert bm.table_cols(1) == 1 + oracle.ring_pages(40, P) and bm.table_cols(2) == 2 + 5
    rng = np.random.default_rng(11)
    lens = {}
    for it in range(300):
        op = rng.random()
        if op < 0.15 and lens:
            s = int(rng.choice(sorted(lens)))
            bm.release(s)
            del lens[s]
            assert bm.context_len(s) == 0
        else:
            ids = rng.choice(8, size=int(rng.integers(1, 5)), replace=False).astype(np.int32)
            cnt = rng.integers(0, 60 if op < 0.5 else 2, size=ids.size).astype(np.int32)
            before = {int(s): lens.get(int(s), 0) for s in ids}
            if any(before[int(s)] + int(c) > 64 * P for s, c in zip(ids, cnt)):
                continue
            try:
                slots, new_lens = bm.append(ids, cnt)
            except pkv.PagedKVError as e:
                assert e.status == 7  # too few blocks: nothing changed
                for s in ids:
                    assert bm.context_len(int(s)) == before[int(s)]
                _check_state(pkv, bm, groups, lens, P)
                continue
            k = 0
            for s, c, nl in zip(ids, cnt, new_lens):
                s, c = int(s), int(c)
                assert nl == before[s] + c
                lens[s] = before[s] + c
                for g, spec in enumerate(groups):
                    assert slots[g, k:k + c].tolist() == _expected_slots(pkv, bm, g, spec, s, before[s], lens[s], P)
                k += c
            for g in range(len(groups)):
                live = slots[g][slots[g] >= 0]
                assert np.unique(live).size == live.size
        _check_state(pkv, bm, groups, lens, P)
    bm.close()


def test_block_manager_errors_change_nothing(pkv):
    P = 16
    bm = pkv.BlockManager(P, 4, 4, [dict(num_blocks=6), dict(window=16, num_blocks=5)])
    bm.append([0], [40])                                   # 3 blocks of the full group, 2 ring blocks
    t0 = [bm.block_table(g, [0, 1, 2, 3]).copy() for g in range(2)]
    for ids, cnt, code in (([1], [60], 7),                 # 4 more full blocks: only 3 free
                           ([0], [40], 2),                 # 80 tokens exceed 4 pages of the full row
                           ([1, 1], [1, 1], 2),            # repeated id
                           ([4], [1], 2),                  # id out of range
                           ([1], [-1], 2)):                # negative count
        with pytest.raises(pkv.PagedKVError) as e:
            bm.append(ids, cnt)
        assert e.value.status == code
        for g in range(2):
            assert np.array_equal(bm.block_table(g, [0, 1, 2, 3]), t0[g])
        assert bm.context_len(0) == 40 and bm.context_len(1) == 0
    assert bm.blocks_in_use(0) == 3 and bm.blocks_in_use(1) == 2
    # released blocks are handed out again, lowest column first
    first = bm.block_table(0, [0])[0, :3].tolist()
    bm.release(0)
    assert bm.blocks_in_use(0) == 0 and bm.blocks_in_use(1) == 0
    bm.append([2], [33])
    assert bm.block_table(0, [2])[0, :3].tolist() == first


def test_block_manager_create_validation(pkv):
    lib = pkv._lib
    h = ctypes.c_void_p()
    G = pkv.LayerGroup

    def create(P=16, seqs=4, pages=8, groups=(G(0, 0, 0, 8),)):
        arr = (G * len(groups))(*groups)
        return lib.pkv_bm_create(P, seqs, pages, arr, len(groups), ctypes.byref(h))

    assert create() == 0
    lib.pkv_bm_destroy(h)
    assert create(P=24) == 3 and create(P=512) == 3
    assert create(seqs=0) == 2 and create(pages=0) == 2
    assert create(groups=(G(0, -1, 0, 8),)) == 2
    assert create(groups=(G(0, 0, 0, -1),)) == 2
    assert create(groups=(G(512, 4, 32, 8),)) == 4       # ring below the least size (33 at P=16)
    assert create(groups=(G(512, 4, 33, 8),)) == 0
    lib.pkv_bm_destroy(h)
    assert create(groups=(G(0, 0, 0, 2 ** 30),)) == 3    # slots would overflow int32
    assert lib.pkv_bm_create(16, 4, 8, None, 1, ctypes.byref(h)) == 1


def test_ring_table_validation_in_decode_calls(pkv):
    """Ring options are checked on the host before any launch."""
    lib = pkv._lib
    d = pkv.CacheDesc(64, 16, 8, 128, 2)
    fake = ctypes.c_void_p(256)  # never dereferenced
    call = lib.paged_decode_attention

    def run(opts, mb):
        return call(ctypes.byref(d), fake, fake, fake, fake, mb, fake, 2, 32, 9000, 0.0, ctypes.byref(opts), fake,
                    2, None, None, 0, None)

    def opts(window, sinks, ring):
        o = pkv.DecodeOpts(window, sinks, None, 0, 0)
        o.ring_pages = ring
        return o

    assert run(opts(0, 0, 33), 40) == 4          # ring without a window
    assert run(opts(512, 4, -1), 40) == 4        # negative ring
    assert run(opts(512, 4, 32), 40) == 4        # below the least ring (33)
    assert run(opts(512, 4, 33), 33) == 2        # row narrower than 1 sink page + 33
    assert run(opts(512, 20, 33), 34) == 2       # 20 sinks take 2 pages
    # a valid ring with a 34-column row passes validation and then needs a workspace for this size
    assert run(opts(512, 4, 33), 34) == 5
    assert lib.paged_decode_attention_workspace_size(ctypes.byref(d), 2, 32, 9000, ctypes.byref(opts(0, 0, 5))) == 0
    assert lib.paged_decode_attention_workspace_size(ctypes.byref(d), 2, 32, 9000, ctypes.byref(opts(512, 4, 33))) > 0
