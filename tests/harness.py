"""Shared set-up for the GPU parity tests: one seeded problem, two caches.

The logical K/V rows come from ``synth``; the oracle appends them into NaN-filled
numpy pools on the CPU, the HIP library appends the same rows into NaN-filled
device pools, and every comparison runs the two sides on those inputs.
"""
from __future__ import annotations

import os
from types import SimpleNamespace

import numpy as np
import torch

import oracle
import synth

NAN_BITS = {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
LSE_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def log(msg: str) -> None:
    print(msg, flush=True)


def make_case(seed, *, B, Hq, Hkv, d, dtype, P, lens, spare=1, q_std=1.0, q=None, K=None, V=None,
              table_seed=None, oracle_side=True, gpu_side=True, pad_value=None):
    """Builds both caches. pad_value: what unused block-table entries hold (default: a spare,
    NaN-filled block, so a read past the context shows up as NaN)."""
    import paged_kv_cache_16_amd as pkv

    lens = [int(x) for x in lens]
    Lmax = max(lens + [1])
    tdt = synth.TORCH_DTYPE[dtype]
    q = synth.normal((B, Hq, d), seed, "q", dtype=dtype, std=q_std) if q is None else q
    K = synth.normal((B, Lmax, Hkv, d), seed, "k", dtype=dtype) if K is None else K
    V = synth.normal((B, Lmax, Hkv, d), seed, "v", dtype=dtype) if V is None else V
    bt, nb = synth.block_tables(lens, P, seed if table_seed is None else table_seed,
                                spare_blocks=spare if pad_value is not None else max(spare, 1))
    if pad_value is None:
        used = set(bt[bt >= 0].tolist())
        free = [x for x in range(nb) if x not in used]
        pad_value = free[0]
    bt = torch.where(bt >= 0, bt, torch.full_like(bt, pad_value))
    slots = synth.token_slots(bt, lens, P)
    k_new = torch.cat([K[b, :L] for b, L in enumerate(lens)]) if sum(lens) else K.reshape(-1, Hkv, d)[:0]
    v_new = torch.cat([V[b, :L] for b, L in enumerate(lens)]) if sum(lens) else V.reshape(-1, Hkv, d)[:0]
    c = SimpleNamespace(q=q, K=K, V=V, bt=bt, nb=nb, lens=lens, P=P, Hkv=Hkv, Hq=Hq, d=d, dtype=dtype,
                        B=B, slots=slots, k_new=k_new, v_new=v_new, seed=seed)
    if oracle_side:
        n_el = nb * Hkv * P * d
        raw_t = np.float32 if dtype == "f32" else np.uint16
        c.kpool = np.full(n_el, NAN_BITS[dtype], dtype=raw_t)
        c.vpool = np.full(n_el, NAN_BITS[dtype], dtype=raw_t)
        oracle.kv_append(dtype, c.kpool, c.vpool, synth.raw_numpy(k_new), synth.raw_numpy(v_new),
                         slots.numpy(), P=P, Hkv=Hkv, d=d)
    if gpu_side:
        dev = torch.device("cuda")
        c.gk = torch.full((nb, Hkv, P, d), float("nan"), dtype=tdt, device=dev)
        c.gv = torch.full((nb, Hkv, P, d), float("nan"), dtype=tdt, device=dev)
        c.gq = q.to(dev)
        c.gbt = bt.to(dev)
        c.gcl = torch.tensor(lens, dtype=torch.int32, device=dev)
        if k_new.shape[0]:
            pkv.kv_cache_append(c.gk, c.gv, k_new.to(dev), v_new.to(dev), slots.to(dev))
    return c


def oracle_attend(c, **kw):
    return oracle.decode_attention(c.dtype, c.kpool, c.vpool, synth.raw_numpy(c.q), c.bt.numpy(),
                                   np.array(c.lens, np.int32), P=c.P, Hkv=c.Hkv, d=c.d, **kw)


def gpu_attend(c, *, max_context_len=None, page_list=None, **kw):
    import paged_kv_cache_16_amd as pkv

    mcl = max(c.lens + [0]) if max_context_len is None else max_context_len
    gpl = None if page_list is None else torch.as_tensor(page_list, dtype=torch.int32).cuda()
    out, lse = pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=mcl,
                                          page_list=gpl, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def raw_bytes(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy().reshape(-1)


def max_err(a, b):
    """Max abs difference; -inf == -inf counts as 0, any other non-finite value counts as inf."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_ninf = np.isneginf(a) & np.isneginf(b)
    with np.errstate(invalid="ignore"):  # -inf - -inf is NaN; those entries are replaced by 0 here
        diff = np.where(both_ninf, 0.0, np.abs(a - b))
    diff = np.where(np.isnan(diff), np.inf, diff)
    return float(diff.max()) if diff.size else 0.0


def assert_close(c, got, ref, what=""):
    out, lse = got
    rout, rlse = ref
    e_out = max_err(out, rout)
    e_lse = max_err(lse, rlse)
    log(f"    {what} max|out err| = {e_out:.3e}  max|lse err| = {e_lse:.3e}")
    assert e_out <= TOL[c.dtype], f"{what}: output error {e_out:.3e} > {TOL[c.dtype]}"
    assert e_lse <= LSE_TOL[c.dtype] * max(1.0, float(np.nanmax(np.abs(np.where(np.isfinite(rlse), rlse, 0))))), \
        f"{what}: lse error {e_lse:.3e}"


# ---------------------------------------------------------------------------------------------
# Full-size parity: the oracle per sequence, on a pool of host threads (the C oracle runs
# outside the interpreter lock). One GPU's share of the host is 16 threads.
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def oracle_pool(dtype, K_rows, V_rows, *, n_tokens, P, Hkv, d, seed, tokens=None):
    """One sequence of n_tokens logical tokens in an oracle pool. K_rows / V_rows ([m, Hkv, d],
    CPU, the input dtype) are the rows of the tokens `tokens` (default: tokens 0 .. m-1); they
    are appended through the oracle into a fresh pool (NaN-filled; 0xFF bytes for INT8) under a
    seeded random block table, and every other token stays NaN, so it must never be read.
    Returns (kpool, vpool, block_table [1, pages] numpy)."""
    bt, nb = synth.block_tables([n_tokens], P, seed, "oracle-sequence", spare_blocks=1)
    if dtype in oracle.INPUT_DTYPE:
        kp = np.full(nb * Hkv * P * (d + 4), 0xFF, np.uint8)
    else:
        kp = np.full(nb * Hkv * P * d, NAN_BITS[dtype], dtype=np.float32 if dtype == "f32" else np.uint16)
    vp = kp.copy()
    t = np.arange(K_rows.shape[0]) if tokens is None else np.asarray(tokens, np.int64)
    assert t.size == K_rows.shape[0] == V_rows.shape[0] and (t.size == 0 or int(t.max()) < n_tokens)
    if t.size:
        slots = (bt[0].numpy().astype(np.int64)[t // P] * P + t % P).astype(np.int32)
        oracle.kv_append(dtype, kp, vp, synth.raw_numpy(K_rows), synth.raw_numpy(V_rows), slots,
                         P=P, Hkv=Hkv, d=d)
    return kp, vp, bt.numpy()


def oracle_sequence(dtype, K_rows, V_rows, evals, *, n_tokens, P, Hkv, d, seed, tokens=None):
    """Attention of one sequence (rows and pool as in oracle_pool). evals: (q [1, Hq, d], L,
    oracle kwargs) triples; returns one (out, lse) pair per triple."""
    kp, vp, bt = oracle_pool(dtype, K_rows, V_rows, n_tokens=n_tokens, P=P, Hkv=Hkv, d=d, seed=seed, tokens=tokens)
    return [oracle.decode_attention(dtype, kp, vp, synth.raw_numpy(q), bt, np.array([L], np.int32),
                                    P=P, Hkv=Hkv, d=d, **okw) for q, L, okw in evals]


def run_threads(fns):
    """Runs the callables on ORACLE_THREADS host threads; results in order."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=ORACLE_THREADS) as ex:
        return list(ex.map(lambda f: f(), fns))


def window_tokens(L, window, sinks):
    """Token indices a window layer attends at context length L (sinks, then the window)."""
    if window <= 0 or window >= L:
        return np.arange(L)
    e0 = min(sinks, L)
    return np.concatenate([np.arange(e0), np.arange(max(e0, L - window), L)])


def page_tokens(L, P, pages):
    """Token indices of the listed pages below L, ascending."""
    parts = [np.arange(p * P, min((p + 1) * P, L)) for p in sorted(int(x) for x in pages if x >= 0) if p * P < L]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)
