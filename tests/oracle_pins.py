"""Pins that tie the CPU oracle to facts fixed outside itself.

Each pin takes an ``oracle.Oracle`` instance and raises AssertionError (or lets an
OracleError through) when the oracle disagrees with what the pages or the
mathematics fix: the primer's worked KV-size values, hand-computed layout
positions, closed forms of softmax attention, invariances, and a brute-force
contiguous-cache evaluation in long double. The same pins run against mutated
copies of the oracle (test_oracle_pins.py) to show that each plausible mistake is
caught by at least one of them.
"""
from __future__ import annotations

import json
import os
from types import SimpleNamespace

import numpy as np
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NAN_BITS = {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}
TOL = 1e-12


def _raw_dtype(dtype):
    return np.float32 if dtype == "f32" else np.uint16


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact decode of a CPU tensor of any cache dtype (torch's own conversion)."""
    return t.to(torch.float64).numpy()


def build(o, seed, *, B, Hq, Hkv, d, dtype, P, lens, spare=1, q=None, K=None, V=None,
          table_seed=None):
    """A paged problem: logical K/V rows appended through the oracle into NaN-filled pools."""
    lens = [int(x) for x in lens]
    Lmax = max(lens + [1])
    q = synth.normal((B, Hq, d), seed, "q", dtype=dtype) if q is None else q
    K = synth.normal((B, Lmax, Hkv, d), seed, "k", dtype=dtype) if K is None else K
    V = synth.normal((B, Lmax, Hkv, d), seed, "v", dtype=dtype) if V is None else V
    bt, nb = synth.block_tables(lens, P, seed if table_seed is None else table_seed,
                                spare_blocks=spare)
    n_el = nb * Hkv * P * d
    kpool = np.full(n_el, NAN_BITS[dtype], dtype=_raw_dtype(dtype))
    vpool = np.full(n_el, NAN_BITS[dtype], dtype=_raw_dtype(dtype))
    slots = synth.token_slots(bt, lens, P)
    k_new = torch.cat([K[b, :L] for b, L in enumerate(lens)]) if lens else K[:0, 0]
    v_new = torch.cat([V[b, :L] for b, L in enumerate(lens)]) if lens else V[:0, 0]
    o.kv_append(dtype, kpool, vpool, synth.raw_numpy(k_new), synth.raw_numpy(v_new),
                slots.numpy(), P=P, Hkv=Hkv, d=d)
    return SimpleNamespace(q=q, K=K, V=V, bt=bt, nb=nb, lens=lens, kpool=kpool, vpool=vpool,
                           P=P, Hkv=Hkv, Hq=Hq, d=d, dtype=dtype, B=B, slots=slots)


def attend(o, pr, **kw):
    return o.decode_attention(pr.dtype, pr.kpool, pr.vpool, synth.raw_numpy(pr.q), pr.bt.numpy(),
                              np.array(pr.lens, np.int32), P=pr.P, Hkv=pr.Hkv, d=pr.d, **kw)


def brute(o, pr, **kw):
    return o.bruteforce(pr.dtype, synth.raw_numpy(pr.K), synth.raw_numpy(pr.V),
                        synth.raw_numpy(pr.q), np.array(pr.lens, np.int32), Hkv=pr.Hkv, d=pr.d,
                        P=pr.P, **kw)


# ---------------------------------------------------------------------------------------
def pin_kv_bytes(o):
    """The primer's worked KV-size values (§3.2, §3.3, §5.3), exact."""
    with open(os.path.join(GOLDEN, "kv_cache_bytes.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = o.kv_cache_bytes(c["batch"], c["layers"], c["heads"], c["head_dim"], c["seq_len"],
                               c["dtype_bytes"])
        assert got == c["bytes"], (c["where"], got, c["bytes"])
    # Paged allocation rounds the sequence up to whole blocks: 4001 tokens -> 251 blocks of 16.
    assert o.kv_cache_bytes(1, 1, 8, 128, 4001, 2, 16) == 2 * 8 * 128 * 4016 * 2
    assert o.kv_cache_bytes(1, 1, 8, 128, 4096, 2, 16) == 2 * 8 * 128 * 4096 * 2


def pin_layout_golden(o):
    """Hand-computed element positions of the documented cache layout."""
    with open(os.path.join(GOLDEN, "layout_positions.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        args = (c["blk"], c["h"], c["t"], c["x"], c["Hkv"], c["P"], c["d"], c["dtype"])
        assert o.k_index(*args) == c["k"], ("K", c)
        assert o.v_index(*args) == c["v"], ("V", c)


def pin_layout_bijection(o):
    """Each tile of the layout is a permutation of its P*d element slots."""
    for dtype in ("f32", "f16", "bf16"):
        for d in (64, 128):
            for P in (16, 32):
                base = (1 * 2 + 1) * P * d  # block 1, head 1 of 2
                for fn in (o.k_index, o.v_index):
                    pos = [fn(1, 1, t, x, 2, P, d, dtype) - base
                           for t in range(P) for x in range(d)]
                    assert sorted(pos) == list(range(P * d)), (fn.__name__, dtype, d, P)


def pin_append_roundtrip(o):
    """Appended rows read back at their slots; every other slot keeps its NaN canary."""
    for dtype, d, P in (("bf16", 128, 16), ("f16", 128, 32), ("f32", 64, 16)):
        pr = build(o, 11, B=2, Hq=2, Hkv=2, d=d, dtype=dtype, P=P, lens=[37, 16], spare=2)
        K, V = synth.raw_numpy(pr.K), synth.raw_numpy(pr.V)
        written = np.zeros(pr.kpool.size, bool)
        for b, L in enumerate(pr.lens):
            for t in range(L):
                blk = int(pr.bt[b, t // P])
                for h in range(pr.Hkv):
                    for x in range(0, d, 7):
                        ki = o.k_index(blk, h, t % P, x, pr.Hkv, P, d, dtype)
                        vi = o.v_index(blk, h, t % P, x, pr.Hkv, P, d, dtype)
                        assert pr.kpool[ki].tobytes() == K[b, t, h, x].tobytes()
                        assert pr.vpool[vi].tobytes() == V[b, t, h, x].tobytes()
                    for x in range(d):
                        written[o.k_index(blk, h, t % P, x, pr.Hkv, P, d, dtype)] = True
        canary = NAN_BITS[dtype].tobytes()
        untouched = pr.kpool[~written]
        assert untouched.size > 0
        assert all(u.tobytes() == canary for u in untouched[:: max(1, untouched.size // 97)])
        # a skipped slot (negative) writes nothing
        before = pr.kpool.copy()
        o.kv_append(dtype, pr.kpool, pr.vpool, synth.raw_numpy(pr.K[0, :1]),
                    synth.raw_numpy(pr.V[0, :1]), np.array([-1], np.int32), P=P, Hkv=pr.Hkv, d=d)
        assert np.array_equal(before.view(np.uint8), pr.kpool.view(np.uint8))


def pin_bruteforce(o):
    """Main oracle == long-double brute force on a contiguous cache, all modes, tiny shapes."""
    rng = np.random.default_rng(5)
    for case in range(18):
        dtype = ("f32", "f16", "bf16")[case % 3]
        d = (64, 128)[(case // 3) % 2]
        P = (16, 32)[case % 2]
        G = (1, 2, 3)[case % 3]
        Hkv = 1 + case % 2
        B = 1 + case % 3
        lens = [int(x) for x in rng.integers(1, 41, size=B)]
        pr = build(o, 100 + case, B=B, Hq=G * Hkv, Hkv=Hkv, d=d, dtype=dtype, P=P, lens=lens)
        modes = [dict(), dict(window=int(rng.integers(1, 20)), sinks=int(rng.integers(0, 6)))]
        pl = np.full((B, 3), -1, np.int32)
        for b, L in enumerate(lens):
            npg = (L + P - 1) // P
            pick = sorted(rng.choice(npg, size=min(2, npg), replace=False).tolist())
            pl[b, :len(pick)] = pick
        modes.append(dict(page_list=pl))
        for kw in modes:
            out, lse = attend(o, pr, **kw)
            bo, bl = brute(o, pr, **kw)
            assert np.abs(out - bo.astype(np.float64)).max() <= TOL, (case, kw)
            assert np.abs(lse - bl.astype(np.float64)).max() <= TOL, (case, kw)


def pin_permutation(o):
    """Placing the same logical pages in other physical blocks changes nothing (bitwise)."""
    for dtype in ("bf16", "f32"):
        kw = dict(B=2, Hq=4, Hkv=2, d=64, dtype=dtype, P=16, lens=[256, 77])
        a = build(o, 7, table_seed=1, **kw)
        b = build(o, 7, table_seed=2, spare=5, **kw)
        assert not np.array_equal(a.bt.numpy(), b.bt.numpy())
        for mode in (dict(), dict(window=40, sinks=3)):
            oa, la = attend(o, a, **mode)
            ob, lb = attend(o, b, **mode)
            assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def pin_window_reductions(o):
    """W >= L and W + S >= L are full attention (bitwise); W = 1, S = s attends {0..s-1, L-1}."""
    pr = build(o, 21, B=2, Hq=2, Hkv=1, d=64, dtype="bf16", P=16, lens=[40, 19])
    full, fl = attend(o, pr)
    for w, s in ((40, 0), (100, 2), (30, 10), (21, 19), (1, 40)):
        out, lse = attend(o, pr, window=w, sinks=s)
        assert np.array_equal(out, full) and np.array_equal(lse, fl), (w, s)
    # W = 1, S = 3 on L = 40: exactly tokens 0, 1, 2 and 39
    keep = [0, 1, 2, 39]
    sub = build(o, 0, B=1, Hq=2, Hkv=1, d=64, dtype="bf16", P=16, lens=[4],
                q=pr.q[:1], K=pr.K[:1, keep], V=pr.V[:1, keep])
    so, sl = attend(o, sub)
    out, lse = attend(o, pr, window=1, sinks=3)
    assert np.abs(out[0] - so[0]).max() <= TOL and np.abs(lse[0] - sl[0]).max() <= TOL
    # and W = 8, S = 0 on L = 40 is tokens 32..39
    sub = build(o, 0, B=1, Hq=2, Hkv=1, d=64, dtype="bf16", P=16, lens=[8],
                q=pr.q[:1], K=pr.K[:1, 32:40], V=pr.V[:1, 32:40])
    so, _ = attend(o, sub)
    out, _ = attend(o, pr, window=8, sinks=0)
    assert np.abs(out[0] - so[0]).max() <= TOL


def pin_identical_keys(o):
    """All keys equal -> every weight equal -> the output is the mean of V over the attended set."""
    B, Hkv, d, L = 1, 1, 64, 45
    K = synth.normal((1, 1, Hkv, d), 3, "k", dtype="bf16").expand(B, L, Hkv, d).contiguous()
    V = synth.normal((B, L, Hkv, d), 3, "v", dtype="bf16")
    pr = build(o, 3, B=B, Hq=2, Hkv=Hkv, d=d, dtype="bf16", P=16, lens=[L], K=K, V=V)
    Vd = to_f64(V)[0, :, 0]
    for kw, toks in ((dict(), range(L)),
                     (dict(window=10, sinks=2), [0, 1] + list(range(35, 45))),
                     (dict(page_list=np.array([[0, 2]], np.int32)), list(range(16)) + list(range(32, 45)))):
        out, _ = attend(o, pr, **kw)
        ref = Vd[list(toks)].mean(axis=0)
        assert np.abs(out[0, 0] - ref).max() <= TOL and np.abs(out[0, 1] - ref).max() <= TOL, kw


def pin_identical_values(o):
    """All value rows equal to v -> the output is v whatever the weights."""
    B, Hkv, d, L = 2, 2, 128, 33
    V = synth.normal((1, 1, Hkv, d), 4, "v", dtype="f16").expand(B, L, Hkv, d).contiguous()
    pr = build(o, 4, B=B, Hq=4, Hkv=Hkv, d=d, dtype="f16", P=32, lens=[L, 5], V=V)
    out, _ = attend(o, pr)
    Vd = to_f64(V)[0, 0]
    for b in range(B):
        for h in range(4):
            assert np.abs(out[b, h] - Vd[h // 2]).max() <= TOL


def pin_small_closed_forms(o):
    """L = 1: out = v0, lse = s0. L = 2: out = v0 + sigmoid(s1 - s0)(v1 - v0), lse = logaddexp."""
    for dtype in ("f32", "f16", "bf16"):
        d = 64
        pr = build(o, 9, B=2, Hq=1, Hkv=1, d=d, dtype=dtype, P=16, lens=[1, 2])
        out, lse = attend(o, pr)
        q = to_f64(pr.q)
        K, V = to_f64(pr.K), to_f64(pr.V)
        s0 = q[0, 0] @ K[0, 0, 0] / np.sqrt(d)
        assert np.array_equal(out[0, 0], V[0, 0, 0]), dtype
        assert abs(lse[0, 0] - s0) <= TOL
        s = [q[1, 0] @ K[1, t, 0] / np.sqrt(d) for t in range(2)]
        sig = 1.0 / (1.0 + np.exp(-(s[1] - s[0])))
        ref = V[1, 0, 0] + sig * (V[1, 1, 0] - V[1, 0, 0])
        assert np.abs(out[1, 0] - ref).max() <= TOL, dtype
        assert abs(lse[1, 0] - np.logaddexp(s[0], s[1])) <= TOL
        # an explicit scale is used as given; 0 selects 1/sqrt(d)
        o2, _ = attend(o, pr, scale=1.0 / np.sqrt(d))
        assert np.array_equal(o2, out)
        o3, l3 = attend(o, pr, scale=0.5)
        s = [q[1, 0] @ K[1, t, 0] * 0.5 for t in range(2)]
        assert abs(l3[1, 0] - np.logaddexp(s[0], s[1])) <= TOL


def pin_peaked(o):
    """Logits hundreds apart: the result is the top key's value, finite (max-shifted softmax)."""
    d, L = 64, 20
    K = synth.normal((1, L, 1, d), 8, "k", dtype="f32")
    q = (K[0, 13, 0] * 200.0).reshape(1, 1, d).contiguous()  # s_13 ~ 1600, the rest ~ +-200
    pr = build(o, 8, B=1, Hq=1, Hkv=1, d=d, dtype="f32", P=16, lens=[L], q=q, K=K)
    out, lse = attend(o, pr)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert np.abs(out[0, 0] - to_f64(pr.V)[0, 13, 0]).max() <= TOL


def pin_key_shift(o):
    """Adding one vector u to every key shifts all logits equally: the output is unchanged."""
    d, L = 64, 30
    g = torch.Generator().manual_seed(1)
    K = (torch.randint(-64, 64, (1, L, 1, d), generator=g).float() / 32.0)
    u = (torch.randint(-64, 64, (1, 1, 1, d), generator=g).float() / 32.0)
    q = (torch.randint(-64, 64, (1, 2, d), generator=g).float() / 64.0)
    a = build(o, 2, B=1, Hq=2, Hkv=1, d=d, dtype="f32", P=16, lens=[L], q=q, K=K)
    b = build(o, 2, B=1, Hq=2, Hkv=1, d=d, dtype="f32", P=16, lens=[L], q=q, K=K + u)
    oa, la = attend(o, a)
    ob, lb = attend(o, b)
    assert np.abs(oa - ob).max() <= TOL
    shift = to_f64(q[0]) @ to_f64(u)[0, 0, 0] / np.sqrt(d)
    assert np.abs((lb - la)[0] - shift).max() <= TOL


def pin_gqa_grouping(o):
    """Query head h reads kv head h // G (contiguous groups): V of kv head g is constant g+1."""
    Hkv, G, d, L = 3, 2, 64, 18
    V = torch.stack([torch.full((L, d), float(g + 1)) for g in range(Hkv)], dim=1)[None]
    pr = build(o, 6, B=1, Hq=Hkv * G, Hkv=Hkv, d=d, dtype="f32", P=16, lens=[L], V=V)
    out, _ = attend(o, pr)
    for h in range(Hkv * G):
        assert np.abs(out[0, h] - (h // G + 1)).max() <= TOL, h


def pin_page_list_reductions(o):
    """All pages == full (bitwise); the last k pages with L % P == 0 == window k*P, no sinks."""
    for P in (16, 32):
        L = 4 * P
        pr = build(o, 12, B=1, Hq=2, Hkv=1, d=128, dtype="bf16", P=P, lens=[L])
        full, fl = attend(o, pr)
        pa, la = attend(o, pr, page_list=np.array([[0, 1, 2, 3]], np.int32))
        assert np.array_equal(pa, full) and np.array_equal(la, fl)
        pa, _ = attend(o, pr, page_list=np.array([[-1, 2, 3, -1]], np.int32))
        wa, _ = attend(o, pr, window=2 * P, sinks=0)
        assert np.array_equal(pa, wa)
        # pages at or beyond the context contribute nothing
        pb, _ = attend(o, pr, page_list=np.array([[2, 3, 7, 9]], np.int32))
        assert np.array_equal(pb, wa)


def pin_split_combine(o):
    """Split partials merged by log-sum-exp equal the direct result; partials are consistent."""
    pr = build(o, 13, B=3, Hq=4, Hkv=2, d=64, dtype="bf16", P=16, lens=[130, 1, 64])
    for kw in (dict(), dict(window=50, sinks=4),
               dict(page_list=np.array([[0, 3, 8], [0, -1, -1], [1, 2, -1]], np.int32))):
        direct, dl = attend(o, pr, **kw)
        for units in (1, 2, 3, 16):
            op, mp, lp, out, lse = o.decode_attention_split(
                pr.dtype, pr.kpool, pr.vpool, synth.raw_numpy(pr.q), pr.bt.numpy(),
                np.array(pr.lens, np.int32), P=16, Hkv=2, d=64, units=units, max_splits=9, **kw)
            assert np.abs(out - direct).max() <= TOL and np.abs(lse - dl).max() <= TOL
            # each partition's own softmax mass, weighted back by the global lse, sums to 1
            live = lp > 0
            mass = np.where(live, lp * np.exp(np.where(live, mp, 0.0) - dl[..., None]), 0.0)
            assert np.abs(mass.sum(-1) - 1.0).max() <= 1e-12
            assert np.all(np.isneginf(mp[~live]))



def pin_split_page_partitions(o):
    """Page-list partitions follow the list: entry k owns enumerated units k*P/16 ..
    (k+1)*P/16 - 1, padding and pages past L included, so some partitions are empty. With
    q = 0 every logit is 0, so a partition's l is its token count, m is 0 and o[0] sums the
    token ids the V rows carry (V[t][0] = t, V[t][1] = 1). Hand-worked, P = 32:
      row 0, list [-1, 0, 3], L = 100: entry 0 (padding) -> units 0, 1; page 0 -> units 2
      (tokens 0..15), 3 (16..31); page 3 -> unit 4 (96..99, the rest is past L), 5 (empty);
      row 1, list [1, 5, -1], L = 40: page 1 -> unit 0 (32..39), 1 (48..63, past L); page 5
      (past L) -> units 2, 3; padding -> 4, 5."""
    B, P, d, Lmax = 2, 32, 64, 100
    V = torch.zeros((B, Lmax, 1, d), dtype=torch.float32)
    V[:, :, 0, 0] = torch.arange(Lmax, dtype=torch.float32)
    V[:, :, 0, 1] = 1.0
    pr = build(o, 15, B=B, Hq=1, Hkv=1, d=d, dtype="f32", P=P, lens=[100, 40],
               q=torch.zeros((B, 1, d), dtype=torch.float32), V=V)
    pl = np.array([[-1, 0, 3], [1, 5, -1]], np.int32)
    # units per partition -> per row, per partition: (token count, sum of token ids)
    expect = {
        1: [[(0, 0), (0, 0), (16, 120), (16, 376), (4, 390), (0, 0)],
            [(8, 284), (0, 0), (0, 0), (0, 0), (0, 0), (0, 0)]],
        2: [[(0, 0), (32, 496), (4, 390)], [(8, 284), (0, 0), (0, 0)]],
        3: [[(16, 120), (20, 766)], [(8, 284), (0, 0)]],
    }
    for units, rows in expect.items():
        S = len(rows[0])
        op, mp, lp, out, lse = o.decode_attention_split(
            pr.dtype, pr.kpool, pr.vpool, synth.raw_numpy(pr.q), pr.bt.numpy(), np.array(pr.lens, np.int32),
            P=P, Hkv=1, d=d, units=units, max_splits=S, page_list=pl)
        for b in range(B):
            for s_, (n, tsum) in enumerate(rows[b]):
                assert lp[b, 0, s_] == n, (units, b, s_, lp[b, 0, s_], n)
                if n:
                    assert mp[b, 0, s_] == 0.0 and op[b, 0, s_, 0] == tsum and op[b, 0, s_, 1] == n
                else:
                    assert np.isneginf(mp[b, 0, s_])

def scores(o, pr, stride, score=None, block=1, **kw):
    return o.decode_scores(pr.dtype, pr.kpool, synth.raw_numpy(pr.q), pr.bt.numpy(),
                           np.array(pr.lens, np.int32), P=pr.P, Hkv=pr.Hkv, d=pr.d, stride=stride,
                           score=score, block=block, **kw)


def pin_scores(o):
    """Decode-time KV scores: per (sequence, kv head) they sum to G (one softmax per query
    head); weighting V by them reproduces the sum of the group's attention outputs (with
    linearly independent V rows this fixes every score); tokens that are not attended keep
    the value they had, and attended ones are added to it."""
    rng = np.random.default_rng(21)
    for case in range(9):
        dtype = ("f32", "f16", "bf16")[case % 3]
        G = (1, 2, 3)[(case // 3) % 3]
        Hkv = 1 + case % 2
        d, P = 64, (16, 32)[case % 2]
        B = 2
        lens = [int(x) for x in rng.integers(1, 41, size=B)]
        if case == 4:
            lens[1] = 0
        pr = build(o, 300 + case, B=B, Hq=G * Hkv, Hkv=Hkv, d=d, dtype=dtype, P=P, lens=lens)
        stride = max(lens) + 3
        pl = np.full((B, 2), -1, np.int32)
        for b, L in enumerate(lens):
            npg = (L + P - 1) // P
            if npg:
                pl[b, 0] = int(rng.integers(0, npg))
        for kw in (dict(), dict(window=7, sinks=2), dict(page_list=pl)):
            init = rng.standard_normal((B, Hkv, stride))
            got = scores(o, pr, stride, score=init.copy(), **kw)
            new = got - init
            out, _ = attend(o, pr, **kw)
            Vd = to_f64(pr.V)
            for b, L in enumerate(lens):
                for h in range(Hkv):
                    sb = new[b, h]
                    if L == 0:
                        assert np.abs(sb).max() <= TOL
                        continue
                    assert abs(sb.sum() - G) <= 1e-12, (case, kw, b, h)
                    mix = (sb[:L, None] * Vd[b, :L, h]).sum(0)
                    ref = out[b, h * G:(h + 1) * G].sum(0)
                    assert np.abs(mix - ref).max() <= 1e-11, (case, kw, b, h)
                    att = scores(o, pr, stride, score=np.zeros((B, Hkv, stride)), **kw)[b, h] != 0
                    assert np.abs(sb[~att]).max(initial=0.0) <= TOL, (case, kw)
    # closed forms: one token gets all of every head's mass; identical keys share it equally
    pr = build(o, 310, B=1, Hq=3, Hkv=1, d=64, dtype="bf16", P=16, lens=[1])
    s1 = scores(o, pr, 4)
    assert abs(s1[0, 0, 0] - 3.0) <= TOL and np.abs(s1[0, 0, 1:]).max() <= TOL
    L = 45
    K = synth.normal((1, 1, 1, 64), 3, "k", dtype="bf16").expand(1, L, 1, 64).contiguous()
    pr = build(o, 311, B=1, Hq=2, Hkv=1, d=64, dtype="bf16", P=16, lens=[L], K=K)
    s2 = scores(o, pr, L, window=10, sinks=2)[0, 0]
    toks = [0, 1] + list(range(35, 45))
    assert np.abs(s2[toks] - 2.0 / len(toks)).max() <= TOL
    assert np.abs(np.delete(s2, toks)).max() <= TOL


def pin_scores_block(o):
    """Score entries of `block` consecutive tokens hold the sums of the (pinned) per-token
    scores of their tokens, in every mode and for blocks that do and do not divide P."""
    pr = build(o, 320, B=2, Hq=6, Hkv=2, d=64, dtype="bf16", P=16, lens=[70, 33])
    pl = np.array([[0, 3, -1], [1, -1, -1]], np.int32)
    for kw in (dict(), dict(window=20, sinks=3), dict(page_list=pl)):
        tok = scores(o, pr, 70, **kw)
        for block in (16, 5, 1000):
            n = (70 + block - 1) // block
            got = scores(o, pr, n, block=block, **kw)
            ref = np.zeros_like(got)
            for t in range(70):
                ref[:, :, t // block] += tok[:, :, t]
            assert np.abs(got - ref).max() <= 1e-12, (kw, block)


def _f32_weights(sc):
    """Page weights in float32, heads added in index order."""
    B, H, n = sc.shape
    w = np.zeros((B, n), np.float32)
    for h in range(H):
        w = (w + sc[:, h]).astype(np.float32)
    return w


def pin_select_pages(o):
    """Page selection: the hand-worked cases of tests/golden/page_select.json ([OVAL] §3.3),
    and on random inputs with many ties the properties that define the result: ids ascending
    and distinct; the newest pages present; min(k, n) ids; every older page taken weighs at
    least as much as every older page left out, and where they weigh the same the taken id is
    the lower."""
    with open(os.path.join(GOLDEN, "page_select.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = o.select_pages(np.array(c["scores"], np.float32), np.array(c["lens"], np.int32), P=c["P"],
                             k=c["k"], recent=c["recent"])
        assert got.tolist() == c["expect"], (c["what"], got.tolist())
    rng = np.random.default_rng(33)
    for case in range(40):
        B, H, P = 3, int(rng.integers(1, 4)), int(rng.choice([16, 32]))
        k, recent = int(rng.integers(1, 9)), 0
        recent = int(rng.integers(0, k + 1))
        lens = rng.integers(0, 20 * P, size=B)
        stride = int((lens.max() + P - 1) // P) + 2
        sc = rng.integers(0, 4, size=(B, H, stride)).astype(np.float32) * 0.5  # small integers: many ties
        got = o.select_pages(sc, lens, P=P, k=k, recent=recent)
        w = _f32_weights(sc)
        for b in range(B):
            n = int((lens[b] + P - 1) // P)
            row = [int(x) for x in got[b] if x >= 0]
            assert all(x == -1 for x in got[b][len(row):]), (case, got[b])
            assert row == sorted(set(row)) and len(row) == min(k, n), (case, row)
            newest = list(range(max(0, n - recent), n))
            assert set(newest) <= set(row), (case, row, newest)
            older = [x for x in row if x < n - recent]
            rest = [x for x in range(max(0, n - recent)) if x not in older]
            for a in older:
                for r in rest:
                    assert w[b, a] > w[b, r] or (w[b, a] == w[b, r] and a < r), (case, a, r)


def pin_int8_quantise(o):
    """INT8 rows: the hand-worked cases of tests/golden/int8_rows.json, and on random rows the
    properties of symmetric rounding quantisation: |q| <= 127, the largest |x| maps to +-127,
    and every x is within half a step of q * scale."""
    with open(os.path.join(GOLDEN, "int8_rows.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        q, sc = o.quantise_rows(np.array([c["x"]], np.float32))
        assert q[0].tolist() == c["q"], (c["what"], q[0].tolist())
        if "scale" in c:
            assert float(sc[0]) == c["scale"], c["what"]
        else:
            assert abs(float(sc[0]) - c["scale_approx"]) <= c["scale_approx"] * 2.0 ** -23, c["what"]
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((64, 128)) * rng.uniform(0.01, 30, size=(64, 1))).astype(np.float32)
    q, sc = o.quantise_rows(x)
    assert np.abs(q.astype(np.int32)).max() <= 127
    amax_pos = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(64), amax_pos]) == 127)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * sc[:, None].astype(np.float64))
    assert np.all(err <= sc[:, None] * (0.5 + 1e-5)), err.max()


def _int8_problem(o, seed, B, Hq, Hkv, d, P, lens):
    """K/V rows whose largest |value| is 127 * 2^-k (k per row, 5..7) and the rest smaller
    bf16 values: every scale is 2^-k and every dequantised value rint(x * 2^k) * 2^-k is exact
    in fp32. Returns the INT8 problem and the fp32 problem holding the dequantised values."""
    rng = np.random.default_rng(seed)
    Lmax = max(lens + [1])

    def rows(tag):
        k = rng.integers(5, 8, size=(B, Lmax, Hkv, 1)).astype(np.float64)
        amax = 127.0 * 2.0 ** -k
        x = rng.uniform(-0.95, 0.95, size=(B, Lmax, Hkv, d)) * amax
        x[..., 0] = amax[..., 0] * np.where(rng.random((B, Lmax, Hkv)) < 0.5, -1.0, 1.0)
        xb = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
        deq = np.rint(xb.to(torch.float64).numpy() * 2.0 ** k) * 2.0 ** -k
        return xb, torch.tensor(deq, dtype=torch.float32)

    K, Kd = rows("k")
    V, Vd = rows("v")
    q = synth.normal((B, Hq, d), seed, "q", dtype="bf16")
    lens = [int(x) for x in lens]
    bt, nb = synth.block_tables(lens, P, seed, spare_blocks=1)
    slots = synth.token_slots(bt, lens, P)
    out = []
    for dtype, KK, VV, qq in (("i8bf16", K, V, q), ("f32", Kd, Vd, q.to(torch.float32))):
        if dtype == "i8bf16":
            kpool = np.zeros(nb * Hkv * P * (d + 4), np.uint8)
            vpool = np.zeros_like(kpool)
        else:
            kpool = np.full(nb * Hkv * P * d, np.float32(np.nan), np.float32)
            vpool = np.full_like(kpool, np.float32(np.nan))
        kn = torch.cat([KK[b, :L] for b, L in enumerate(lens)])
        vn = torch.cat([VV[b, :L] for b, L in enumerate(lens)])
        o.kv_append(dtype, kpool, vpool, synth.raw_numpy(kn), synth.raw_numpy(vn), slots.numpy(), P=P, Hkv=Hkv, d=d)
        out.append(SimpleNamespace(q=qq, bt=bt, nb=nb, lens=lens, kpool=kpool, vpool=vpool, P=P, Hkv=Hkv, Hq=Hq,
                                   d=d, dtype=dtype, B=B))
    return out


def pin_int8_attention(o):
    """Attention (and scores) over an INT8 cache equal attention over an fp32 cache holding
    the same dequantised values (rows built so that they are exact): int8 plane layout, scale
    plane and dequantisation, in every mode."""
    pr8, pr32 = _int8_problem(o, 500, B=3, Hq=4, Hkv=2, d=64, P=16, lens=[70, 33, 1])
    pl = np.array([[0, 3, -1], [1, 2, -1], [0, -1, -1]], np.int32)
    for kw in (dict(), dict(window=20, sinks=3), dict(page_list=pl)):
        a8 = attend(o, pr8, **kw)
        a32 = attend(o, pr32, **kw)
        assert np.abs(a8[0] - a32[0]).max() <= 1e-12 and np.abs(a8[1] - a32[1]).max() <= 1e-12, kw
        s8 = scores(o, pr8, 70, **kw)
        s32 = scores(o, pr32, 70, **kw)
        assert np.abs(s8 - s32).max() <= 1e-12, kw


def pin_ring_golden(o):
    """Ring sizes, ring columns and blocks held, worked out by hand in
    tests/golden/ring_policy.json; pool bytes against the primer's KV formula."""
    with open(os.path.join(GOLDEN, "ring_policy.json")) as f:
        g = json.load(f)
    for c in g["ring_pages"]:
        assert o.ring_pages(c["W"], c["P"]) == c["R"], c["what"]
    for c in g["columns"]:
        got = [o.ring_column(j, sinks=c["S"], P=c["P"], ring_pages=c["R"]) for j in c["pages"]]
        assert got == c["cols"], (c["what"], got)
    for c in g["blocks"]:
        assert o.policy_blocks(c["L"], P=c["P"], window=c["W"], sinks=c["S"]) == c["n"], c["what"]
    for c in g["bytes"]:
        n = o.policy_blocks(c["L"], P=c["P"], window=c["W"], sinks=c["S"])
        assert n * c["P"] * 2 * c["Hkv"] * c["d"] * c["es"] == c["bytes"], c["what"]
        if c["W"] <= 0:
            assert o.kv_cache_bytes(1, 1, c["Hkv"], c["d"], c["L"], c["es"], c["P"]) == c["bytes"], c["what"]


def pin_ring_pages_bruteforce(o):
    """The ring size is the most pages any W consecutive tokens touch (enumerated over window
    positions), and the blocks a sequence holds follow min(ceil(L/P), ceil(S/P) + R)."""
    for P in (16, 32):
        for W in range(1, 3 * P + 3):
            most = max(len({t // P for t in range(L - W, L)}) for L in range(W, W + 2 * P + 1))
            assert o.ring_pages(W, P) == most, (W, P)
    rng = np.random.default_rng(77)
    for _ in range(300):
        P = int(rng.choice([16, 32, 64]))
        W = int(rng.integers(0, 700))
        S = int(rng.integers(0, 70))
        L = int(rng.integers(0, 5000))
        R = 0 if W <= 0 else o.ring_pages(W, P) + int(rng.integers(0, 3))
        pages = -(-L // P)
        want = pages if W <= 0 else min(pages, -(-S // P) + R)
        assert o.policy_blocks(L, P=P, window=W, sinks=S, ring_pages=R) == want, (L, P, W, S, R)


def _ring_problem(o, seed, *, B, Hq, Hkv, d, dtype, P, lens, W, S, R):
    """A window layer over a ring table: every token of every sequence appended in order
    through the ring (later pages write over the blocks of dead ones), into NaN pools holding
    only ceil(S/P) + R blocks per sequence."""
    Lmax = max(lens + [1])
    q = synth.normal((B, Hq, d), seed, "q", dtype=dtype)
    K = synth.normal((B, Lmax, Hkv, d), seed, "k", dtype=dtype)
    V = synth.normal((B, Lmax, Hkv, d), seed, "v", dtype=dtype)
    cols = -(-S // P) + R
    ring, nb = synth.block_tables([cols * P] * B, P, seed, spare_blocks=1)
    plain = o.ring_expand(ring.numpy(), sinks=S, P=P, ring_pages=R, pages=max(1, -(-Lmax // P)))
    n_el = nb * Hkv * P * d
    kpool = np.full(n_el, NAN_BITS[dtype], dtype=_raw_dtype(dtype))
    vpool = np.full(n_el, NAN_BITS[dtype], dtype=_raw_dtype(dtype))
    slots = synth.token_slots(torch.from_numpy(plain), lens, P)
    k_new = torch.cat([K[b, :L] for b, L in enumerate(lens)])
    v_new = torch.cat([V[b, :L] for b, L in enumerate(lens)])
    o.kv_append(dtype, kpool, vpool, synth.raw_numpy(k_new), synth.raw_numpy(v_new), slots.numpy(), P=P,
                Hkv=Hkv, d=d)
    return SimpleNamespace(q=q, K=K, V=V, bt=ring, nb=nb, lens=lens, kpool=kpool, vpool=vpool, P=P, Hkv=Hkv,
                           Hq=Hq, d=d, dtype=dtype, B=B)


def pin_ring_attention(o):
    """Attention of a window layer through its ring table equals the brute force on the
    contiguous logical rows, over lengths that wrap the ring several times. A ring slot is
    shared by tokens R*P apart, so a ring of R pages with R*P < W drops window tokens: some
    result must then differ."""
    cases = [(16, 23, 0), (16, 23, 3), (16, 40, 16), (16, 16, 20), (32, 33, 5), (16, 1, 0), (16, 1, 2)]
    for i, (P, W, S) in enumerate(cases):
        Rmin = o.ring_pages(W, P)
        lens = [1, W, W + 1, 5 * P + 7, 11 * P, 9 * P + 1, 13 * P - 1]
        for R, must_match in ((Rmin, True), (Rmin + 2, True), (-(-W // P) - 1, False)):
            if R <= 0:
                continue
            pr = _ring_problem(o, 600 + i, B=len(lens), Hq=2, Hkv=1, d=64, dtype="bf16", P=P, lens=lens, W=W,
                               S=S, R=R)
            out, lse = attend(o, pr, window=W, sinks=S, ring_pages=R)
            bo, bl = brute(o, pr, window=W, sinks=S)
            same = (np.abs(out - bo.astype(np.float64)).max() <= TOL and
                    np.abs(lse - bl.astype(np.float64)).max() <= TOL)
            assert same == must_match, (P, W, S, R)


def pin_ring_reuse(o):
    """With the least ring size, a block is taken over by a new page only when none of its
    tokens is attended any more (the block lies wholly outside sinks and window); one page
    fewer breaks that. Checked by walking a sequence token by token."""
    def reuse_ok(P, W, S, R, Lmax):
        owner = {}  # column -> logical page it holds
        for L in range(1, Lmax + 1):
            j = (L - 1) // P
            c = o.ring_column(j, sinks=S, P=P, ring_pages=R)
            old = owner.get(c)
            if old is not None and old != j:
                live = [t for t in range(old * P, old * P + P) if t < S or t >= L - W]
                if live:
                    return False
            owner[c] = j
        return True

    for P, W, S in ((16, 23, 0), (16, 23, 3), (16, 32, 0), (16, 40, 16), (32, 33, 5), (16, 17, 0), (16, 64, 4)):
        R = o.ring_pages(W, P)
        assert reuse_ok(P, W, S, R, 14 * P + 5), (P, W, S)
        assert not reuse_ok(P, W, S, R - 1, 14 * P + 5), (P, W, S)


def pin_empty(o):
    pr = build(o, 14, B=2, Hq=2, Hkv=1, d=64, dtype="f16", P=16, lens=[0, 3])
    out, lse = attend(o, pr)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0])) and np.isfinite(lse[1]).all()


PINS = [pin_kv_bytes, pin_layout_golden, pin_layout_bijection, pin_append_roundtrip,
        pin_bruteforce, pin_permutation, pin_window_reductions, pin_identical_keys,
        pin_identical_values, pin_small_closed_forms, pin_peaked, pin_key_shift,
        pin_gqa_grouping, pin_page_list_reductions, pin_split_combine, pin_split_page_partitions, pin_scores, pin_scores_block, pin_select_pages,
        pin_int8_quantise, pin_int8_attention, pin_ring_golden, pin_ring_pages_bruteforce,
        pin_ring_attention, pin_ring_reuse, pin_empty]


if __name__ == "__main__":
    # Runs every pin against the oracle build given on the command line; prints the names
    # of the failing pins and exits 1 if any failed (used for planted-mistake builds).
    import sys

    import oracle as _oracle

    o = _oracle.Oracle(sys.argv[1])
    failed = []
    for pin in PINS:
        try:
            pin(o)
        except (AssertionError, _oracle.OracleError):
            failed.append(pin.__name__)
    print(" ".join(failed))
    sys.exit(1 if failed else 0)
