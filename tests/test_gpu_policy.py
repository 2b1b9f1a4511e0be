"""Per-layer memory policy on the GPU ([Novita] §關鍵技術 1: each layer keeps a full cache or a
sliding window, and window layers hold fewer blocks): the library's block manager drives a
prefill and decode steps for a full group and window groups whose block tables are rings; the
HIP kernels read the rings through the C ABI. Every output is compared with the oracle's
attention over the logical rows (its own plain table, its own pools), so nothing on the
expected side depends on the manager's block choices.

Tolerances as for plain tables (2e-3 for 2-byte and INT8 caches, 1e-5 for fp32). Pools start
NaN-filled (0xFF bytes for INT8) and ring blocks are reused while the test runs, so a read of
a token outside the attended set, or of a page the ring has dropped, shows up."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import NAN_BITS, assert_close, log, max_err, oracle_sequence, window_tokens

pytestmark = pytest.mark.gpu
IN = {"i8bf16": "bf16", "i8f16": "f16"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import paged_kv_cache_16_amd  # noqa: F401  (fails loudly if the library is missing)


def _tol_case(dtype):
    return SimpleNamespace(dtype=IN.get(dtype, dtype))


def _new_pool(pkv, dtype, nb, Hkv, P, d):
    if dtype in IN:
        t = pkv.new_cache(nb, Hkv, P, d, torch.int8, device="cuda")
        t.fill_(-1)
        return t
    return torch.full((nb, Hkv, P, d), float("nan"), dtype=synth.TORCH_DTYPE[dtype], device="cuda")


def oracle_logical(dtype, q, K, V, lens, *, P, Hkv, d, seed, **kw):
    """The oracle on the logical rows [0, L_b) of every sequence, through its own plain table
    and pools."""
    lens = [int(x) for x in lens]
    bt, nb = synth.block_tables(lens, P, seed, "oracle", spare_blocks=1)
    n = oracle.pool_elems(nb, Hkv, P, d, dtype)
    if dtype in IN:
        kpool = np.full(n, 0xFF, np.uint8)
    else:
        kpool = np.full(n, NAN_BITS[dtype], np.float32 if dtype == "f32" else np.uint16)
    vpool = kpool.copy()
    kn = torch.cat([K[b, :L] for b, L in enumerate(lens)])
    vn = torch.cat([V[b, :L] for b, L in enumerate(lens)])
    oracle.kv_append(dtype, kpool, vpool, synth.raw_numpy(kn), synth.raw_numpy(vn),
                     synth.token_slots(bt, lens, P).numpy(), P=P, Hkv=Hkv, d=d)
    return SimpleNamespace(kpool=kpool, vpool=vpool, bt=bt.numpy(), lens=np.array(lens, np.int32))


def run_policy(seed, *, dtype, B, Hq, Hkv, d, P, prefill, steps, groups, path="fused", scores=False,
               check=None):
    """Prefill, then `steps` decode steps; every step checks each group's output (and scores)
    against the oracle on the steps listed in `check` (default: all)."""
    import paged_kv_cache_16_amd as pkv
    ind = IN.get(dtype, dtype)
    Lmax = max(prefill) + steps
    K = synth.normal((B, Lmax, Hkv, d), seed, "k", dtype=ind)
    V = synth.normal((B, Lmax, Hkv, d), seed, "v", dtype=ind)
    qs = synth.normal((steps, B, Hq, d), seed, "q", dtype=ind)
    bm = pkv.BlockManager(P, B, -(-Lmax // P), groups)
    pools = [(_new_pool(pkv, dtype, g["num_blocks"], Hkv, P, d), _new_pool(pkv, dtype, g["num_blocks"], Hkv, P, d))
             for g in groups]
    ids = np.arange(B, dtype=np.int32)
    slots, lens = bm.append(ids, prefill)
    if slots.shape[1]:
        kp = torch.cat([K[b, :prefill[b]] for b in range(B)]).cuda()
        vp = torch.cat([V[b, :prefill[b]] for b in range(B)]).cuda()
        for g, (gk, gv) in enumerate(pools):
            pkv.kv_cache_append(gk, gv, kp, vp, torch.from_numpy(slots[g]).cuda())
    stride = -(-Lmax // 1)
    acc = [torch.zeros((B, Hkv, stride), dtype=torch.float32, device="cuda") for _ in groups] if scores else None
    ref_acc = [np.zeros((B, Hkv, stride)) for _ in groups] if scores else None
    worst = 0.0
    for s in range(steps):
        slots, lens = bm.append(ids)
        cl = torch.from_numpy(lens).cuda()
        kn = torch.stack([K[b, lens[b] - 1] for b in range(B)]).cuda()
        vn = torch.stack([V[b, lens[b] - 1] for b in range(B)]).cuda()
        q = qs[s].cuda()
        do_check = check is None or s in check
        ref_prob = oracle_logical(dtype, qs[s], K, V, lens, P=P, Hkv=Hkv, d=d, seed=seed) if do_check or scores else None
        for g, spec in enumerate(groups):
            gk, gv = pools[g]
            W, S = spec.get("window", 0), spec.get("num_sinks", 0)
            bt = torch.from_numpy(bm.block_table(g, ids)).cuda()
            kw = dict(window=W, num_sinks=S, ring_pages=bm.ring_pages(g)) if W else {}
            sl = torch.from_numpy(slots[g].copy()).cuda()
            sc = dict(scores=acc[g]) if scores else {}
            if path == "fused":
                out, lse = pkv.paged_decode_append_attention(q, gk, gv, kn, vn, sl, bt, cl, max_context_len=int(lens.max()),
                                                             **kw, **sc)
            else:
                pkv.kv_cache_append(gk, gv, kn, vn, sl)
                split = dict(split_tokens=64) if path == "split" else {}
                out, lse = pkv.paged_decode_attention(q, gk, gv, bt, cl, max_context_len=int(lens.max()), **kw, **split,
                                                      **sc)
            if scores:
                ref_acc[g] = oracle.decode_scores(dtype, ref_prob.kpool, synth.raw_numpy(qs[s]), ref_prob.bt,
                                                  ref_prob.lens, P=P, Hkv=Hkv, d=d, stride=stride, window=W, sinks=S,
                                                  score=ref_acc[g])
            if not do_check:
                continue
            torch.cuda.synchronize()
            ref = oracle.decode_attention(dtype, ref_prob.kpool, ref_prob.vpool, synth.raw_numpy(qs[s]), ref_prob.bt,
                                          ref_prob.lens, P=P, Hkv=Hkv, d=d, window=W, sinks=S)
            got = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
            assert_close(_tol_case(dtype), got, ref, f"step {s} group {g} (W={W}, S={S}) L={lens.tolist()}")
            worst = max(worst, max_err(got[0], ref[0]))
            if scores:
                e = max_err(acc[g].cpu().numpy(), ref_acc[g])
                assert e <= 1e-5, f"step {s} group {g}: score error {e:.3e}"
    for g, spec in enumerate(groups):
        want = sum(oracle.policy_blocks(int(L), P=P, window=spec.get("window", 0), sinks=spec.get("num_sinks", 0),
                                        ring_pages=spec.get("ring_pages", 0)) for L in lens)
        assert bm.blocks_in_use(g) == want
    bm.close()
    return worst


GROUPS_16 = [dict(num_blocks=80), dict(window=40, num_sinks=3, num_blocks=3 * 5 + 2),
             dict(window=23, num_sinks=20, num_blocks=3 * 5 + 1)]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f32", 64), ("i8bf16", 128)])
def test_ring_decode_steps_fused(dtype, d):
    """Full group and two window groups (one with sinks spanning two pages): prefill of
    uneven lengths, then 40 fused decode steps that cross pages and wrap the rings."""
    log(f"ring fused {dtype} d={d}")
    run_policy(70, dtype=dtype, B=3, Hq=4, Hkv=2, d=d, P=16, prefill=[5, 150, 333], steps=40, groups=GROUPS_16,
               check=set(range(0, 40, 3)) | {39})


@pytest.mark.parametrize("path", ["append", "split"])
def test_ring_decode_steps_unfused(path):
    """The same through kv_cache_append + paged_decode_attention, on the work-split path and on
    fixed 64-token partitions (the partial/combine kernels)."""
    log(f"ring {path}")
    run_policy(71, dtype="bf16", B=3, Hq=8, Hkv=1, d=128, P=16, prefill=[0, 64, 200], steps=24,
               groups=GROUPS_16, path=path, check=set(range(0, 24, 4)) | {23})


def test_ring_larger_than_least_and_page_32():
    """32-token pages, a ring two pages above the least size, and a window of 100 tokens."""
    log("ring P=32 R=least+2")
    groups = [dict(num_blocks=40), dict(window=100, num_sinks=0, ring_pages=6, num_blocks=4 * 6),
              dict(window=33, num_sinks=5, num_blocks=4 * 4)]
    run_policy(72, dtype="f16", B=4, Hq=6, Hkv=1, d=128, P=32, prefill=[1, 31, 100, 400], steps=36,
               groups=groups, check=set(range(0, 36, 5)) | {35})


def test_ring_score_export():
    """Score export through ring tables accumulates the oracle's per-token scores."""
    log("ring scores")
    run_policy(73, dtype="bf16", B=2, Hq=4, Hkv=2, d=128, P=16, prefill=[90, 200], steps=20, groups=GROUPS_16[:2],
               scores=True, check=set(range(0, 20, 4)) | {19})


def test_full_size_kvsparse_ring_window_layer():
    """The KV-sparse Llama-3-8B shape's window layer (B=8, 32 q / 8 kv heads, d=128, bf16,
    L ~ U[7000, 30000], window 512 + 4 sinks) on a ring pool of 8 x 34 blocks: prefill of
    L-1 tokens through the manager, one fused decode step, every sequence against the
    oracle."""
    import paged_kv_cache_16_amd as pkv
    name = "llama3_8b_kvsparse_bf16"
    w = synth.WORKLOADS[name]
    B, P, d, Hkv, Hq, seed = w.batch, w.block_size, w.head_dim, w.kv_heads, w.q_heads, 7
    lens = synth.uniform_lengths(B, w.ctx_lo, w.ctx_hi, seed, name).tolist()
    R = pkv.ring_pages(512, P)
    nb = B * (1 + R)
    log(f"{name} ring window layer B={B} lens={lens} pool={nb} blocks")
    bm = pkv.BlockManager(P, B, -(-max(lens) // P), [dict(window=512, num_sinks=4, num_blocks=nb)])
    gk = torch.full((nb, Hkv, P, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    gv = torch.full_like(gk, float("nan"))

    def rows(b, tag):  # drawn on the GPU; the oracle gets a copy of the same values
        return synth.normal((lens[b], Hkv, d), seed, name, b, tag, dtype="bf16", device="cuda")

    ids = np.arange(B, dtype=np.int32)
    slots, _ = bm.append(ids, [L - 1 for L in lens])
    k0 = 0
    for b, L in enumerate(lens):
        sl = torch.from_numpy(slots[0, k0:k0 + L - 1].copy()).cuda()
        pkv.kv_cache_append(gk, gv, rows(b, "k")[:L - 1], rows(b, "v")[:L - 1], sl)
        k0 += L - 1
    assert bm.blocks_in_use(0) == nb
    slots, new_lens = bm.append(ids)
    assert new_lens.tolist() == lens
    qs = synth.normal((B, Hq, d), seed, name, "q", dtype="bf16")
    kn = torch.stack([rows(b, "k")[L - 1] for b, L in enumerate(lens)])
    vn = torch.stack([rows(b, "v")[L - 1] for b, L in enumerate(lens)])
    bt = torch.from_numpy(bm.block_table(0, ids)).cuda()
    out, lse = pkv.paged_decode_append_attention(qs.cuda(), gk, gv, kn, vn, torch.from_numpy(slots[0].copy()).cuda(),
                                                 bt, torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                                 max_context_len=max(lens), window=512, num_sinks=4, ring_pages=R)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    for b, L in enumerate(lens):  # every sequence; the oracle holds only the attended tokens
        toks = window_tokens(L, 512, 4)
        idx = torch.as_tensor(toks, device="cuda")
        ref = oracle_sequence("bf16", rows(b, "k")[idx].cpu(), rows(b, "v")[idx].cpu(),
                              [(qs[b:b + 1], L, dict(window=512, sinks=4))], n_tokens=L, P=P, Hkv=Hkv, d=d,
                              seed=seed, tokens=toks)[0]
        assert_close(_tol_case("bf16"), (out[b:b + 1], lse[b:b + 1]), ref, f"{name} ring seq {b}")
    bm.close()
