"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars: kv_cache_append is bit-exact; attention outputs are within max abs error 2e-3
for bf16/fp16 caches (fp32 accumulation) and 1e-5 for fp32 caches. Pools start
NaN-filled and unused block-table entries point at a NaN-filled block, so any read
of memory outside the attended set shows up as NaN.
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import (NAN_BITS, TOL, assert_close, gpu_attend, log, make_case, max_err,
                     oracle_attend, raw_bytes)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_16_amd  # noqa: F401  (fails loudly if the library is missing)


# ---------------------------------------------------------------------------- append
@pytest.mark.parametrize("dtype,P,d", [("bf16", 16, 128), ("f16", 32, 128), ("f32", 16, 64),
                                       ("bf16", 32, 64), ("f16", 16, 64), ("f32", 32, 128)])
def test_append_bit_exact(dtype, P, d):
    log(f"append {dtype} P={P} d={d}")
    c = make_case(31, B=3, Hq=4, Hkv=2, d=d, dtype=dtype, P=P, lens=[45, 16, 100], spare=3)
    assert np.array_equal(raw_bytes(c.gk), c.kpool.view(np.uint8))
    assert np.array_equal(raw_bytes(c.gv), c.vpool.view(np.uint8))


@pytest.mark.parametrize("P,dtype,d", [(48, "bf16", 128), (64, "f16", 64), (128, "f32", 128), (256, "bf16", 64),
                                       (256, "f16", 128)])
def test_block_sizes_up_to_256(P, dtype, d):
    """Block sizes past 32, up to the largest the library takes (any multiple of 16 to 256):
    append bit-exact, attention in every mode and on the partition path, and the fused step,
    against the oracle."""
    import paged_kv_cache_16_amd as pkv
    lens = [3 * P + 5, P, 1, 0, 700]
    log(f"block size {P} {dtype} d={d}")
    c = make_case(33 + P, B=5, Hq=8, Hkv=2, d=d, dtype=dtype, P=P, lens=lens, spare=2)
    assert np.array_equal(raw_bytes(c.gk), c.kpool.view(np.uint8))
    assert np.array_equal(raw_bytes(c.gv), c.vpool.view(np.uint8))
    assert_close(c, gpu_attend(c), oracle_attend(c), f"P={P} full")
    assert_close(c, gpu_attend(c, split_tokens=P), oracle_attend(c), f"P={P} partitions")
    W, S = P + 7, 3
    assert_close(c, gpu_attend(c, window=W, num_sinks=S), oracle_attend(c, window=W, sinks=S), f"P={P} window")
    pl = synth.page_lists(lens, P, 2, 33 + P).numpy()
    assert_close(c, gpu_attend(c, page_list=pl), oracle_attend(c, page_list=pl), f"P={P} pages")
    # fused step: the cache already holds every row, and row L-1 comes again from k_new/v_new
    slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, P) if L else -1 for b, L in enumerate(lens)],
                         dtype=torch.int32).cuda()
    kn = torch.stack([c.K[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
    vn = torch.stack([c.V[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
    out, lse = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl,
                                                 max_context_len=max(lens))
    torch.cuda.synchronize()
    assert_close(c, (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)),
                 oracle_attend(c), f"P={P} fused")
    assert np.array_equal(raw_bytes(c.gk), c.kpool.view(np.uint8))


def test_append_skips_negative_and_out_of_range_slots():
    import paged_kv_cache_16_amd as pkv
    c = make_case(32, B=1, Hq=2, Hkv=2, d=128, dtype="bf16", P=16, lens=[20], spare=2)
    before_k, before_v = raw_bytes(c.gk).copy(), raw_bytes(c.gv).copy()
    n_slots = c.nb * c.P
    slots = torch.tensor([-1, n_slots, n_slots + 7, -5], dtype=torch.int32, device="cuda")
    kn = synth.normal((4, 2, 128), 9, "kn", dtype="bf16").cuda()
    pkv.kv_cache_append(c.gk, c.gv, kn, kn, slots)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bytes(c.gk), before_k)
    assert np.array_equal(raw_bytes(c.gv), before_v)


@pytest.mark.parametrize("dtype,P,d", [("bf16", 16, 128), ("f16", 32, 64), ("f32", 32, 128)])
def test_append_long_runs_whole_and_partial_sub_tiles(dtype, P, d):
    """Appends of 64 tokens or more go 16 tokens at a time: a group whose slots fill one 16-token
    sub-tile in order is written as whole chunks, every other group chunk by chunk. Groups here:
    whole sub-tiles (a block's first or second half), consecutive but unaligned slots, a -1 inside
    an aligned run, an aligned run in reverse order, a slot past the pool, scattered slots and a
    partial last group. Both pools must equal the oracle's append bit for bit (the slot past the
    pool skipped and reported)."""
    import paged_kv_cache_16_amd as pkv
    Hkv, nb = 2, 24
    n_slots = nb * P
    rng = np.random.default_rng(77 + P + d)
    groups = [
        list(range(3 * P, 3 * P + 16)),                          # whole sub-tile (a block's first)
        list(range(5 * P + P - 16, 5 * P + P)),                  # a block's last sub-tile
        list(range(7 * P + 4, 7 * P + 20)),                      # consecutive, not aligned
        [9 * P + k if k != 6 else -1 for k in range(16)],        # aligned run with a hole
        list(range(11 * P + 15, 11 * P - 1, -1)),                # aligned slots in reverse
        [13 * P + k if k != 9 else n_slots + 3 for k in range(16)],  # one slot past the pool
        [int(x) for x in rng.choice(np.arange(15 * P, 19 * P), 16, replace=False)],  # scattered
        list(range(0, 16)),                                      # whole sub-tile of block 0
        list(range((nb - 1) * P, (nb - 1) * P + 16)),            # the pool's last block
        list(range(21 * P, 21 * P + 5)),                         # partial last group
    ]
    slots = [x for g in groups for x in g]
    N = len(slots)
    assert N >= 64 and len({x for x in slots if x >= 0}) == sum(1 for x in slots if x >= 0)
    log(f"append long run {dtype} P={P} d={d} N={N}")
    kn = synth.normal((N, Hkv, d), 70, "kn-long", dtype=dtype)
    vn = synth.normal((N, Hkv, d), 70, "vn-long", dtype=dtype)
    n_el = nb * Hkv * P * d
    raw_t = np.float32 if dtype == "f32" else np.uint16
    kpool = np.full(n_el, NAN_BITS[dtype], dtype=raw_t)
    vpool = np.full(n_el, NAN_BITS[dtype], dtype=raw_t)
    oracle.kv_append(dtype, kpool, vpool, synth.raw_numpy(kn), synth.raw_numpy(vn),
                     np.array([x if x < n_slots else -1 for x in slots], np.int32), P=P, Hkv=Hkv, d=d)
    tdt = synth.TORCH_DTYPE[dtype]
    gk = torch.full((nb, Hkv, P, d), float("nan"), dtype=tdt, device="cuda")
    gv = torch.full((nb, Hkv, P, d), float("nan"), dtype=tdt, device="cuda")
    pkv.device_errors(clear=True)
    pkv.kv_cache_append(gk, gv, kn.cuda(), vn.cuda(), torch.tensor(slots, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(raw_bytes(gk), kpool.view(np.uint8))
    assert np.array_equal(raw_bytes(gv), vpool.view(np.uint8))
    assert pkv.device_errors() == pkv.DEV_SLOT


def test_decode_step_append_then_attend():
    """One decode step: prefill L-1 tokens, append the new token, attend over L ([primer] §2.2)."""
    import paged_kv_cache_16_amd as pkv
    lens = [300, 129, 17]
    c = make_case(33, B=3, Hq=8, Hkv=2, d=128, dtype="bf16", P=16, lens=lens)
    ref = oracle_attend(c)
    # rebuild the GPU cache as prefill of L-1 tokens plus one appended token per sequence
    c.gk.fill_(float("nan"))
    c.gv.fill_(float("nan"))
    pre = synth.token_slots(c.bt, lens, c.P, last=[L - 1 for L in lens])
    kp = torch.cat([c.K[b, :L - 1] for b, L in enumerate(lens)]).cuda()
    vp = torch.cat([c.V[b, :L - 1] for b, L in enumerate(lens)]).cuda()
    pkv.kv_cache_append(c.gk, c.gv, kp, vp, pre.cuda())
    new_slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, c.P) for b, L in enumerate(lens)],
                             dtype=torch.int32).cuda()
    kn = torch.stack([c.K[b, L - 1] for b, L in enumerate(lens)]).cuda()
    vn = torch.stack([c.V[b, L - 1] for b, L in enumerate(lens)]).cuda()
    pkv.kv_cache_append(c.gk, c.gv, kn, vn, new_slots)
    assert_close(c, gpu_attend(c), ref, "decode step")


# ---------------------------------------------------------------------------- parity per workload shape
def _case_for(name, seed=1, B=None):
    w = synth.WORKLOADS[name]
    B = w.batch if B is None else B
    if name == "tiny_mha_f32":
        lens = [256] * B
    else:
        lens = synth.uniform_lengths(B, w.ctx_lo, w.ctx_hi, seed, name).tolist()
    return w, lens


def test_parity_tiny_mha_f32_exact_config():
    """1 seq, 8 heads (q = kv), d=64, L=256, P=16, fp32; the pool is exactly 16 blocks, the
    table a seeded permutation of them."""
    w, lens = _case_for("tiny_mha_f32")
    log("tiny_mha_f32 full size")
    c = make_case(1, B=1, Hq=8, Hkv=8, d=64, dtype="f32", P=16, lens=lens, spare=0,
                  pad_value=0)
    assert c.nb == 16 and sorted(c.bt[0].tolist()) == list(range(16))
    assert_close(c, gpu_attend(c), oracle_attend(c), "tiny_mha_f32")


@pytest.mark.parametrize("split_tokens", [0, 256, 1024])
def test_parity_llama3_layer_shape(split_tokens):
    """Llama-3-8B layer shape (32 q / 8 kv heads, d=128, bf16, P=16, L ~ U[1024, 4096]), 4 seqs."""
    w, lens = _case_for("llama3_8b_layer_bf16", B=4)
    log(f"llama3 layer B=4 lens={lens} split_tokens={split_tokens}")
    c = make_case(2, B=4, Hq=32, Hkv=8, d=128, dtype="bf16", P=16, lens=lens)
    assert_close(c, gpu_attend(c, split_tokens=split_tokens), oracle_attend(c), "llama3 layer")


def test_parity_qwen_g6_shape():
    """Qwen2.5-1.5B layer shape (12 q / 2 kv heads, G=6), contexts 4097..4128."""
    lens = [4097, 4110, 4128]
    log(f"qwen G=6 lens={lens}")
    c = make_case(3, B=3, Hq=12, Hkv=2, d=128, dtype="bf16", P=16, lens=lens)
    assert_close(c, gpu_attend(c), oracle_attend(c), "qwen g6")


@pytest.mark.parametrize("mode", ["full", "window"])
def test_parity_kvsparse_shape(mode):
    """Per-layer KV sparsity shape: 32 q / 8 kv, d=128, bf16, L in [7000, 30000];
    window layers attend to the last 512 tokens plus 4 sinks."""
    lens = [7000, 29999]
    kw = dict(window=512, sinks=4) if mode == "window" else {}
    log(f"kvsparse {mode} lens={lens}")
    c = make_case(4, B=2, Hq=32, Hkv=8, d=128, dtype="bf16", P=16, lens=lens)
    gkw = dict(window=512, num_sinks=4) if mode == "window" else {}
    assert_close(c, gpu_attend(c, **gkw), oracle_attend(c, **kw), f"kvsparse {mode}")


def test_parity_page_selected_f16_shape():
    """7B MHA page selection: 32 heads (q = kv), d=128, fp16, P=32, 16 selected pages (the last
    page always, 15 earlier ones sorted), here over L = 4096 so the oracle's pool stays small."""
    lens = [4096, 3001]
    log("page select f16")
    c = make_case(5, B=2, Hq=32, Hkv=32, d=128, dtype="f16", P=32, lens=lens)
    pl = synth.page_lists(lens, 32, 16, 5).numpy()
    assert_close(c, gpu_attend(c, page_list=pl), oracle_attend(c, page_list=pl), "pages f16")


# ---------------------------------------------------------------------------- fuzz
FUZZ = []
_rng = np.random.default_rng(2024)
for _i in range(36):
    FUZZ.append(dict(
        seed=1000 + _i,
        dtype=("bf16", "f16", "f32")[_i % 3],
        d=(64, 128)[(_i // 3) % 2],
        P=(16, 32)[(_i // 6) % 2],
        G=(1, 2, 4, 6, 8)[_i % 5],
        Hkv=(1, 2)[_i % 2],
        B=int(_rng.integers(1, 5)),
        Lmax=int(_rng.integers(0, 301)),
        mode=("full", "window", "pages")[_i % 3],
        split=(0, 16, 64, 256)[_i % 4],
    ))


@pytest.mark.parametrize("f", FUZZ, ids=[f"s{f['seed']}-{f['dtype']}-d{f['d']}-P{f['P']}-G{f['G']}-{f['mode']}"
                                         for f in FUZZ])
def test_fuzz(f):
    rng = np.random.default_rng(f["seed"])
    lens = [int(x) for x in rng.integers(0, f["Lmax"] + 1, size=f["B"])]
    log(f"fuzz {f} lens={lens}")
    c = make_case(f["seed"], B=f["B"], Hq=f["G"] * f["Hkv"], Hkv=f["Hkv"], d=f["d"], dtype=f["dtype"],
                  P=f["P"], lens=lens)
    okw, gkw = {}, dict(split_tokens=f["split"])
    if f["mode"] == "window":
        W, S = int(rng.integers(1, 120)), int(rng.integers(0, 20))
        okw = dict(window=W, sinks=S)
        gkw.update(window=W, num_sinks=S)
    elif f["mode"] == "pages":
        k = 4
        pl = np.full((f["B"], k), -1, np.int32)
        for b, L in enumerate(lens):
            npg = (L + f["P"] - 1) // f["P"]
            if npg:
                pick = sorted(rng.choice(npg, size=min(k, npg), replace=False).tolist())
                pl[b, :len(pick)] = pick
        okw = dict(page_list=pl)
        gkw.update(page_list=pl)
    assert_close(c, gpu_attend(c, **gkw), oracle_attend(c, **okw), "fuzz")


# ---------------------------------------------------------------------------- persistent-path fuzz
# Longer contexts than the fuzz above, so the persistent kernel runs and cuts segments into many
# pieces: random batch, group, kv heads, dtype, head dim, mode and ragged lengths up to 6000.
STREAM_FUZZ = []
_srng = np.random.default_rng(2027)
for _i in range(12):
    STREAM_FUZZ.append(dict(
        seed=3000 + _i,
        dtype=("bf16", "f16", "f32")[_i % 3],
        d=(128, 64)[(_i // 3) % 2],
        G=(1, 2, 4, 6, 8)[_i % 5],
        Hkv=int(_srng.integers(1, 4)),
        B=int(_srng.integers(1, 9)),
        Lmax=int(_srng.integers(600, 6001)),
        mode=("full", "window", "pages")[_i % 3],
    ))


@pytest.mark.parametrize("f", STREAM_FUZZ, ids=[f"s{f['seed']}-{f['dtype']}-d{f['d']}-G{f['G']}-H{f['Hkv']}-B{f['B']}-{f['mode']}"
                                                for f in STREAM_FUZZ])
def test_stream_fuzz(f):
    rng = np.random.default_rng(f["seed"])
    lens = [int(x) for x in rng.integers(1, f["Lmax"] + 1, size=f["B"])]
    lens[int(rng.integers(0, f["B"]))] = f["Lmax"]  # one sequence at the bound: the persistent path
    log(f"stream fuzz {f} lens={lens}")
    c = make_case(f["seed"], B=f["B"], Hq=f["G"] * f["Hkv"], Hkv=f["Hkv"], d=f["d"], dtype=f["dtype"],
                  P=16, lens=lens)
    okw, gkw = {}, {}
    if f["mode"] == "window":
        W, S = int(rng.integers(300, 2000)), int(rng.integers(0, 40))
        okw = dict(window=W, sinks=S)
        gkw = dict(window=W, num_sinks=S)
    elif f["mode"] == "pages":
        k = 24
        pl = np.full((f["B"], k), -1, np.int32)
        for b, L in enumerate(lens):
            npg = (L + 15) // 16
            pick = sorted(rng.choice(npg, size=min(k, npg), replace=False).tolist())
            pl[b, :len(pick)] = pick
        okw = dict(page_list=pl)
        gkw = dict(page_list=pl)
    assert_close(c, gpu_attend(c, **gkw), oracle_attend(c, **okw), "stream fuzz")


# ---------------------------------------------------------------------------- batches past 64
@pytest.mark.parametrize("B,mode,fused", [(65, "full", False), (129, "full", True), (130, "window", True),
                                          (200, "pages", False), (200, "full", True)])
def test_batches_beyond_64(B, mode, fused):
    """More than 64 sequences: the persistent kernel holds the first 64 lengths in lanes and
    reads the rest from memory, scanning them per 64-sequence chunk; empty sequences sit on
    both sides of the chunk boundary and one long sequence past it takes many waves."""
    import paged_kv_cache_16_amd as pkv
    rng = np.random.default_rng(B)
    lens = [int(x) for x in rng.integers(0, 160, size=B)]
    lens[63] = 0
    lens[64] = 0
    lens[B - 2] = 1500
    log(f"batch {B} {mode} fused={fused} sum(L)={sum(lens)}")
    c = make_case(60 + B, B=B, Hq=8, Hkv=2, d=128, dtype="bf16", P=16, lens=lens)
    okw, gkw = {}, {}
    if mode == "window":
        okw, gkw = dict(window=100, sinks=3), dict(window=100, num_sinks=3)
    elif mode == "pages":
        pl = np.full((B, 3), -1, np.int32)
        for b, L in enumerate(lens):
            npg = (L + 15) // 16
            if npg:
                pick = sorted(rng.choice(npg, size=min(3, npg), replace=False).tolist())
                pl[b, :len(pick)] = pick
        okw = dict(page_list=pl)
        gkw = dict(page_list=torch.as_tensor(pl).cuda())
    ref = oracle_attend(c, **okw)
    if not fused:
        got = gpu_attend(c, **{k: v for k, v in gkw.items() if k != "page_list"},
                         page_list=okw.get("page_list"))
    else:
        # the cache already holds every row; the step appends row L-1 again from k_new/v_new
        slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, c.P) if L else -1 for b, L in enumerate(lens)],
                             dtype=torch.int32).cuda()
        kn = torch.stack([c.K[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
        vn = torch.stack([c.V[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
        out, lse = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl,
                                                     max_context_len=max(lens), **gkw)
        torch.cuda.synchronize()
        got = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    assert_close(c, got, ref, f"batch {B} {mode}")


def test_max_batch_65535():
    """The largest batch the library takes: 65535 sequences, almost all short and three long
    (the longest puts the call on the persistent path), so every wave's prologue scans 1024
    chunks of 64 lengths from memory. Attention and the fused step, every sequence against
    the oracle."""
    import paged_kv_cache_16_amd as pkv
    from harness import NAN_BITS
    B, Hq, Hkv, d, P, dt = 65535, 2, 1, 64, 16, "bf16"
    rng = np.random.default_rng(65535)
    lens = rng.integers(0, 24, size=B)
    lens[[5, 40000, B - 1]] = [700, 650, 333]
    T = int(lens.sum())
    log(f"max batch {B}: {T} tokens")
    K = synth.normal((T, Hkv, d), 91, "k", dtype=dt)
    V = synth.normal((T, Hkv, d), 91, "v", dtype=dt)
    q = synth.normal((B, Hq, d), 91, "q", dtype=dt)
    bt, nb = synth.block_tables(lens.tolist(), P, 91, spare_blocks=1)
    free = torch.ones(nb, dtype=torch.bool)
    free[bt[bt >= 0].long()] = False
    bt = torch.where(bt >= 0, bt, torch.full_like(bt, int(free.nonzero()[0])))
    slots = synth.token_slots(bt, lens.tolist(), P)
    n_el = nb * Hkv * P * d
    kpool = np.full(n_el, NAN_BITS[dt], dtype=np.uint16)
    vpool = np.full(n_el, NAN_BITS[dt], dtype=np.uint16)
    oracle.kv_append(dt, kpool, vpool, synth.raw_numpy(K), synth.raw_numpy(V), slots.numpy(), P=P, Hkv=Hkv, d=d)
    ref = oracle.decode_attention(dt, kpool, vpool, synth.raw_numpy(q), bt.numpy(), lens.astype(np.int32),
                                  P=P, Hkv=Hkv, d=d)
    dev = torch.device("cuda")
    pkv.device_errors()  # start from a clear error word
    gk = torch.full((nb, Hkv, P, d), float("nan"), dtype=torch.bfloat16, device=dev)
    gv = torch.full_like(gk, float("nan"))
    pkv.kv_cache_append(gk, gv, K.to(dev), V.to(dev), slots.to(dev))
    gq, gbt = q.to(dev), bt.to(dev)
    gcl = torch.as_tensor(lens.astype(np.int32)).to(dev)
    assert pkv.workspace_size(gk, B, Hq, int(lens.max())) > 0  # the persistent path
    out, lse = pkv.paged_decode_attention(gq, gk, gv, gbt, gcl, max_context_len=int(lens.max()))
    torch.cuda.synchronize()
    c = SimpleNamespace(dtype=dt)
    assert_close(c, (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)), ref,
                 "max batch")
    # fused step: row L-1 of every sequence again from k_new/v_new
    last = np.cumsum(lens) - 1
    take = torch.as_tensor(np.where(lens > 0, last, 0))
    kn, vn = K[take].to(dev), V[take].to(dev)
    sl = torch.as_tensor(np.where(lens > 0, slots.numpy()[np.maximum(last, 0)], -1).astype(np.int32)).to(dev)
    out, lse = pkv.paged_decode_append_attention(gq, gk, gv, kn, vn, sl, gbt, gcl, max_context_len=int(lens.max()))
    torch.cuda.synchronize()
    assert_close(c, (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)), ref,
                 "max batch fused")
    assert pkv.device_errors() == 0


# ---------------------------------------------------------------------------- one-kernel path, many segments
@pytest.mark.parametrize("mode,fused", [("full", False), ("window", True), ("pages", False), ("full", True)])
def test_direct_path_many_segments(mode, fused):
    """256 (sequence, kv head) segments of at most 40 units take the one-kernel path (no workspace):
    every sequence against the oracle, lengths 0..640 (up to 40 units)."""
    import paged_kv_cache_16_amd as pkv
    B, Hkv, G = 64, 4, 2
    rng = np.random.default_rng(77 + len(mode))
    lens = [int(x) for x in rng.integers(0, 641, size=B)]
    lens[5] = 0
    lens[9] = 640
    log(f"direct path {mode} fused={fused} sum(L)={sum(lens)}")
    c = make_case(77, B=B, Hq=G * Hkv, Hkv=Hkv, d=128, dtype="bf16", P=32, lens=lens)
    okw, gkw = {}, {}
    if mode == "window":
        okw, gkw = dict(window=200, sinks=5), dict(window=200, num_sinks=5)
    elif mode == "pages":
        pl = np.full((B, 6), -1, np.int32)
        for b, L in enumerate(lens):
            npg = (L + 31) // 32
            if npg:
                pick = sorted(rng.choice(npg, size=min(6, npg), replace=False).tolist())
                pl[b, :len(pick)] = pick
        okw = dict(page_list=pl)
        gkw = dict(page_list=torch.as_tensor(pl).cuda())
    assert pkv.workspace_size(c.gk, B, G * Hkv, max(lens), window=gkw.get("window", 0),
                              num_sinks=gkw.get("num_sinks", 0), page_list=gkw.get("page_list")) == 0
    ref = oracle_attend(c, **okw)
    if not fused:
        got = gpu_attend(c, **{k: v for k, v in gkw.items() if k != "page_list"}, page_list=okw.get("page_list"))
    else:
        slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, c.P) if L else -1 for b, L in enumerate(lens)],
                             dtype=torch.int32).cuda()
        kn = torch.stack([c.K[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
        vn = torch.stack([c.V[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
        out, lse = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl,
                                                     max_context_len=max(lens), **gkw)
        torch.cuda.synchronize()
        got = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    assert_close(c, got, ref, f"direct {mode}")


# ---------------------------------------------------------------------------- special cases
def test_empty_and_single_token():
    c = make_case(40, B=3, Hq=4, Hkv=1, d=128, dtype="bf16", P=16, lens=[0, 1, 0])
    out, lse = gpu_attend(c)
    ref = oracle_attend(c)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    # L = 1: the output is v_0 exactly (weight exp(0) = 1, normaliser 1)
    v0 = c.V[1, 0].float().numpy()
    for h in range(4):
        assert np.array_equal(out[1, h], v0[0].astype(np.float64))
    assert_close(c, (out, lse), ref, "empty/single")


def test_peaked_logits():
    """q scaled x4 and one planted key aligned with q: running-max rescaling under stress."""
    d, L = 128, 700
    K = synth.normal((2, L, 2, d), 41, "k", dtype="bf16")
    q = synth.normal((2, 8, d), 41, "q", dtype="bf16", std=4.0)
    K[0, 333, 0] = (q[0, 0].float() * 0.5).to(torch.bfloat16)
    K[1, 5, 1] = (q[1, 6].float() * 0.5).to(torch.bfloat16)
    c = make_case(41, B=2, Hq=8, Hkv=2, d=d, dtype="bf16", P=16, lens=[L, 611], q=q, K=K)
    assert_close(c, gpu_attend(c), oracle_attend(c), "peaked")
    assert_close(c, gpu_attend(c, split_tokens=64), oracle_attend(c), "peaked split64")


def test_window_edge_cases():
    c = make_case(42, B=4, Hq=8, Hkv=2, d=64, dtype="f16", P=16, lens=[40, 17, 300, 1])
    for W, S in [(1, 0), (1, 3), (16, 16), (20, 30), (299, 1), (1000, 4), (33, 0), (15, 17)]:
        assert_close(c, gpu_attend(c, window=W, num_sinks=S), oracle_attend(c, window=W, sinks=S),
                     f"window W={W} S={S}")


def test_page_list_padding_and_beyond_context():
    c = make_case(43, B=2, Hq=4, Hkv=1, d=128, dtype="bf16", P=32, lens=[100, 64])
    pl = np.array([[-1, 0, 3, -1, 7], [1, 2, 5, -1, -1]], np.int32)  # 7, 2 and 5 are past L
    assert_close(c, gpu_attend(c, page_list=pl), oracle_attend(c, page_list=pl), "pages padding")


def test_block_table_permutation_is_bitwise_invariant():
    lens = [555, 1024]
    a = make_case(44, B=2, Hq=8, Hkv=2, d=128, dtype="bf16", P=16, lens=lens, table_seed=1, spare=3)
    b = make_case(44, B=2, Hq=8, Hkv=2, d=128, dtype="bf16", P=16, lens=lens, table_seed=2, spare=9)
    assert not torch.equal(a.bt, b.bt)
    for kw in (dict(), dict(window=300, num_sinks=4), dict(split_tokens=128)):
        oa, la = gpu_attend(a, **kw)
        ob, lb = gpu_attend(b, **kw)
        assert np.array_equal(oa, ob) and np.array_equal(la, lb), kw
    # and repeated runs are identical
    o1, _ = gpu_attend(a)
    o2, _ = gpu_attend(a)
    assert np.array_equal(o1, o2)


def test_out_dtype_and_explicit_scale():
    import paged_kv_cache_16_amd as pkv
    c = make_case(45, B=2, Hq=4, Hkv=2, d=128, dtype="bf16", P=16, lens=[200, 77])
    ref_out, _ = oracle_attend(c, scale=0.05)
    out, _ = pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=200,
                                        scale=0.05, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    # bound: fp32 tolerance plus half an ulp of bf16 at the reference magnitude
    bound = TOL["bf16"] + np.abs(ref_out) * 2.0 ** -8
    assert np.all(np.abs(got - ref_out) <= bound)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_stream_combine_piece_counts(dtype, d):
    """Persistent path over few, short segments, so that the flat split cuts them into about
    (units + lead) / 2 pieces each (two units per wave once the whole batch is under two units per
    wave): counts around the combine's first batch (8, 12 or 16 own slots, by the segment count),
    the rest of the 16 own slots, and the overflow slots (up to 24 per round trip, then the rest)."""
    units = [13, 14, 15, 29, 30, 60, 61, 62, 77, 140]
    lens = [16 * u for u in units[:-2]] + [16 * units[-2] - 5, 16 * units[-1] - 15]
    log(f"stream combine piece counts {dtype} d={d} lens={lens}")
    c = make_case(77, B=len(lens), Hq=4, Hkv=1, d=d, dtype=dtype, P=16, lens=lens)
    assert_close(c, gpu_attend(c), oracle_attend(c), "pieces")
    c2 = make_case(78, B=3, Hq=12, Hkv=2, d=d, dtype=dtype, P=16, lens=[16 * 33, 16 * 33 + 1, 16 * 64])
    assert_close(c2, gpu_attend(c2), oracle_attend(c2), "pieces G=6")
    # many segments (the combine's first batch is 8 wide), a few of them long enough for the
    # rest of their own slots and the overflow slots
    lens3 = [16] * 150 + [16 * 12, 16 * 20, 16 * 40, 2000]
    c3 = make_case(79, B=len(lens3), Hq=2, Hkv=1, d=d, dtype=dtype, P=16, lens=lens3)
    assert_close(c3, gpu_attend(c3), oracle_attend(c3), "pieces, 154 segments")
    # 96 and 80 segments: first batches of 12 and 16 own slots, each with a long sequence whose
    # pieces run past the own slots
    lens4 = [200] * 30 + [1200, 1201]
    c4 = make_case(80, B=len(lens4), Hq=6, Hkv=3, d=d, dtype=dtype, P=16, lens=lens4)
    assert_close(c4, gpu_attend(c4), oracle_attend(c4), "pieces, 96 segments")
    lens5 = [300] * 18 + [3000, 2900]
    c5 = make_case(81, B=len(lens5), Hq=8, Hkv=4, d=d, dtype=dtype, P=16, lens=lens5)
    assert_close(c5, gpu_attend(c5), oracle_attend(c5), "pieces, 80 segments")


def test_partial_and_combine_match_oracle_partitions():
    """Partials of the partition path against the oracle's partitions, in full, window and
    page-list mode. Page lists are cut by list entry (every 16-token quarter of every entry,
    padding and pages past the context included), so the lists here hold padding, pages past
    L and, with 32-token pages and 16-token partitions, pages split over two partitions."""
    import paged_kv_cache_16_amd as pkv
    lens = [333, 64, 0, 129]
    c = make_case(46, B=4, Hq=6, Hkv=1, d=128, dtype="bf16", P=16, lens=lens)
    pl16 = np.array([[-1, 2, 7, 20, 25], [0, -1, 3, -1, -1], [0, 1, -1, -1, -1], [1, 4, 8, 9, -1]], np.int32)
    lens32 = [333, 70, 129]
    c32 = make_case(56, B=3, Hq=6, Hkv=1, d=128, dtype="bf16", P=32, lens=lens32)
    pl32 = np.array([[-1, 0, 3, 10, 11], [1, -1, 2, 5, -1], [0, 4, -1, -1, -1]], np.int32)
    cases = [(c, 64, dict(), dict()), (c, 64, dict(window=100, num_sinks=3), dict(window=100, sinks=3)),
             (c, 64, dict(page_list=torch.as_tensor(pl16).cuda()), dict(page_list=pl16)),
             (c32, 16, dict(page_list=torch.as_tensor(pl32).cuda()), dict(page_list=pl32)),
             (c32, 48, dict(page_list=torch.as_tensor(pl32).cuda()), dict(page_list=pl32))]
    for c, st, kw, okw in cases:
        lens = c.lens
        op, mp, lp = pkv.paged_decode_attention_partial(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens),
                                                        split_tokens=st, **kw)
        torch.cuda.synchronize()
        S = op.shape[2]
        ro, rm, rl, rout, rlse = oracle.decode_attention_split(
            c.dtype, c.kpool, c.vpool, synth.raw_numpy(c.q), c.bt.numpy(), np.array(lens, np.int32),
            P=c.P, Hkv=1, d=128, units=st // 16, max_splits=S, **okw)
        log(f"    partitions P={c.P} split={st} S={S} {sorted(okw)}: live {int((rl > 0).sum())} of {rl.size}")
        mp_, lp_ = mp.cpu().numpy(), lp.cpu().numpy()
        live = rl > 0
        assert np.array_equal(live, lp_ > 0)
        assert max_err(mp_[live], rm[live]) <= 1e-4
        assert max_err(np.log(lp_[live]), np.log(rl[live])) <= 1e-4
        o_ = op.cpu().numpy()
        # compare the normalised partition outputs (scale-free)
        assert max_err((o_[live] / lp_[live][:, None]), ro[live] / rl[live][:, None]) <= 2e-3
        out, lse = pkv.paged_decode_combine(op, mp, lp)
        torch.cuda.synchronize()
        assert_close(c, (out.cpu().numpy(), lse.cpu().numpy()), (rout, rlse), f"combine P={c.P} split={st} {sorted(okw)}")


def test_status_codes():
    import paged_kv_cache_16_amd as pkv
    c = make_case(47, B=1, Hq=4, Hkv=2, d=128, dtype="bf16", P=16, lens=[20])
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=20, window=8,
                                   page_list=torch.zeros((1, 1), dtype=torch.int32, device="cuda"))
    assert e.value.status == 4
    bad_q = torch.zeros((1, 3, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_decode_attention(bad_q, c.gk, c.gv, c.gbt, c.gcl, max_context_len=20)
    assert e.value.status == 2
    big_g = torch.zeros((1, 2 * 9, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_decode_attention(big_g, c.gk, c.gv, c.gbt, c.gcl, max_context_len=20)
    assert e.value.status == 3


@pytest.mark.parametrize("fill", [0xA5, 0xFF])
def test_workspace_reuse(fill):
    """One workspace serves any number of calls, which all give the same result: its
    contents on entry are ignored, also between calls whose plans differ (full and window
    attention sharing one workspace, as the layers of one model do). 0xFF bytes are NaN as
    floats: partial slots past a segment's piece count must be dropped, not weighted by 0."""
    import paged_kv_cache_16_amd as pkv
    lens = [1500, 333, 4000, 2, 0, 129]
    c = make_case(48, B=6, Hq=16, Hkv=4, d=128, dtype="bf16", P=16, lens=lens)
    n = pkv.workspace_size(c.gk, 6, 16, max(lens))
    n_w = pkv.workspace_size(c.gk, 6, 16, max(lens), window=1000, num_sinks=4)
    assert n > 0 and n_w > 0
    ws = torch.full((max(n, n_w),), fill, dtype=torch.uint8, device="cuda")  # garbage on entry
    ref = oracle_attend(c)
    ref_w = oracle_attend(c, window=1000, sinks=4)
    outs = []
    for _ in range(3):
        out, lse = pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens),
                                              workspace=ws)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)))
        out, lse = pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens),
                                              window=1000, num_sinks=4, workspace=ws)
        torch.cuda.synchronize()
        assert_close(c, (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)), ref_w,
                     "workspace reuse, window")
    for got in outs:
        assert_close(c, got, ref, "workspace reuse")
        assert np.array_equal(got[0], outs[0][0])


FUSED_CASES = [
    dict(name="llama3-shape", B=4, Hq=32, Hkv=8, d=128, dtype="bf16", P=16, lens=[1500, 4096, 17, 2049], kw={}),
    dict(name="g6-window", B=3, Hq=12, Hkv=2, d=128, dtype="bf16", P=16, lens=[4100, 600, 31],
         kw=dict(window=512, num_sinks=4)),
    dict(name="f16-pages", B=2, Hq=8, Hkv=8, d=128, dtype="f16", P=32, lens=[1000, 64], kw="pages"),
    dict(name="f32-d64", B=2, Hq=4, Hkv=4, d=64, dtype="f32", P=16, lens=[300, 45], kw={}),
    dict(name="tiny-direct", B=2, Hq=4, Hkv=2, d=128, dtype="bf16", P=16, lens=[100, 7], kw={}, direct=True),
    dict(name="partitions", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", P=16, lens=[900, 333], kw=dict(split_tokens=128)),
    # one-kernel path: the workgroup of each (sequence, kv head) patches the new token in and writes it
    dict(name="direct-window", B=3, Hq=8, Hkv=2, d=128, dtype="bf16", P=16, lens=[300, 50, 1],
         kw=dict(window=64, num_sinks=4), direct=True),
    dict(name="direct-pages", B=2, Hq=8, Hkv=8, d=128, dtype="f16", P=32, lens=[1000, 64], kw=dict(pages=2),
         direct=True),
    dict(name="direct-pages-no-newest", B=2, Hq=8, Hkv=8, d=128, dtype="f16", P=32, lens=[1000, 70],
         kw=dict(pages=2, newest=False), direct=True),
    dict(name="direct-wide-pages", B=64, Hq=8, Hkv=4, d=128, dtype="f16", P=32,
         lens=[int(x) for x in np.random.default_rng(61).integers(1, 900, size=64)], kw=dict(pages=6), direct=True),
    dict(name="direct-wide-f32-d64", B=64, Hq=4, Hkv=4, d=64, dtype="f32", P=16,
         lens=[int(x) for x in np.random.default_rng(62).integers(1, 640, size=64)], kw={}, direct=True),
]


@pytest.mark.parametrize("fc", FUSED_CASES, ids=[f["name"] for f in FUSED_CASES])
def test_fused_append_attention(fc):
    """paged_decode_append_attention == kv_cache_append + paged_decode_attention: the cache
    bytes match the oracle's append bit for bit and the outputs match the oracle."""
    import paged_kv_cache_16_amd as pkv
    lens = fc["lens"]
    log(f"fused {fc['name']}")
    c = make_case(60, B=fc["B"], Hq=fc["Hq"], Hkv=fc["Hkv"], d=fc["d"], dtype=fc["dtype"], P=fc["P"], lens=lens)
    # GPU cache: prefill all but each sequence's last token; the fused call appends it
    c.gk.fill_(float("nan"))
    c.gv.fill_(float("nan"))
    pre = synth.token_slots(c.bt, lens, c.P, last=[L - 1 for L in lens])
    kp = torch.cat([c.K[b, :L - 1] for b, L in enumerate(lens)]).cuda()
    vp = torch.cat([c.V[b, :L - 1] for b, L in enumerate(lens)]).cuda()
    pkv.kv_cache_append(c.gk, c.gv, kp, vp, pre.cuda())
    slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, c.P) for b, L in enumerate(lens)], dtype=torch.int32).cuda()
    kn = torch.stack([c.K[b, L - 1] for b, L in enumerate(lens)]).cuda()
    vn = torch.stack([c.V[b, L - 1] for b, L in enumerate(lens)]).cuda()
    kw, okw = fc["kw"], {}
    if kw == "pages" or "pages" in kw:
        npages = 6 if kw == "pages" else kw["pages"]
        if kw == "pages" or kw.get("newest", True):
            pl = synth.page_lists(lens, c.P, npages, 60).numpy()
        else:  # earlier pages only: the new token is written but not attended
            pl = synth.page_lists([max(L - c.P, 1) for L in lens], c.P, npages, 60).numpy()
            assert all((pl[b] < (L - 1) // c.P).all() for b, L in enumerate(lens))
        kw = dict(page_list=torch.as_tensor(pl).cuda())
        okw = dict(page_list=pl)
    elif "window" in kw:
        okw = dict(window=kw["window"], sinks=kw["num_sinks"])
    if "direct" in fc:  # the path this case is meant to take (the one-kernel path needs no workspace)
        n_ws = pkv.workspace_size(c.gk, fc["B"], fc["Hq"], max(lens), window=kw.get("window", 0),
                                  num_sinks=kw.get("num_sinks", 0), page_list=kw.get("page_list"))
        assert (n_ws == 0) == fc["direct"], n_ws
    out, lse = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl,
                                                 max_context_len=max(lens), **kw)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bytes(c.gk), c.kpool.view(np.uint8))
    assert np.array_equal(raw_bytes(c.gv), c.vpool.view(np.uint8))
    got = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    assert_close(c, got, oracle_attend(c, **okw), f"fused {fc['name']}")


@pytest.mark.parametrize("mode", ["full", "pages"])
def test_graph_replay_one_kernel_fused_step(mode):
    """The one-kernel fused step (64 segments of at most 40 units: no workspace, the append
    inside the attention kernel) captured in a HIP graph: every replay, with eager calls in
    between, gives the eager result bit for bit, and the eager result matches the oracle."""
    import paged_kv_cache_16_amd as pkv
    B, Hq, Hkv = 16, 8, 4
    rng = np.random.default_rng(52)
    lens = [int(x) for x in rng.integers(1, 600, size=B)]
    c = make_case(52, B=B, Hq=Hq, Hkv=Hkv, d=128, dtype="f16", P=32, lens=lens)
    kw, okw = {}, {}
    if mode == "pages":
        pl = synth.page_lists(lens, c.P, 5, 52).numpy()
        kw, okw = dict(page_list=torch.as_tensor(pl).cuda()), dict(page_list=pl)
    assert pkv.workspace_size(c.gk, B, Hq, max(lens), page_list=kw.get("page_list")) == 0  # one kernel
    slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, c.P) for b, L in enumerate(lens)], dtype=torch.int32).cuda()
    kn = torch.stack([c.K[b, L - 1] for b, L in enumerate(lens)]).cuda()
    vn = torch.stack([c.V[b, L - 1] for b, L in enumerate(lens)]).cuda()
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    def step():
        pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl, max_context_len=max(lens),
                                          out=out, lse=lse, **kw)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    assert_close(c, (ref[0].cpu().numpy().astype(np.float64), ref[1].cpu().numpy().astype(np.float64)),
                 oracle_attend(c, **okw), f"graph one-kernel {mode}: eager step")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {i} differs from the eager step"
        pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens), window=100)
        torch.cuda.synchronize()
    assert np.array_equal(raw_bytes(c.gk), c.kpool.view(np.uint8))


def test_graph_replay_fused_step():
    """The fused decode step captured in a HIP graph: every replay, with eager calls and
    synchronisations in between, reproduces the eager result bit for bit (the work split
    and the merge order are fixed by the arguments, not by timing), and the eager result
    matches the oracle."""
    import paged_kv_cache_16_amd as pkv
    lens = [1500, 333, 4000, 2, 0, 129]
    B, Hq, Hkv = 6, 16, 4
    c = make_case(49, B=B, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16", P=16, lens=lens)
    # the new row of each sequence is its last token, already in the cache: rewriting it is a no-op
    slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, c.P) if L > 0 else -1 for b, L in enumerate(lens)],
                         dtype=torch.int32).cuda()
    kn = torch.stack([c.K[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
    vn = torch.stack([c.V[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
    ws = torch.empty(pkv.workspace_size(c.gk, B, Hq, max(lens)), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    def step():
        pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl, max_context_len=max(lens),
                                          out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    assert_close(c, (ref[0].cpu().numpy().astype(np.float64), ref[1].cpu().numpy().astype(np.float64)),
                 oracle_attend(c), "graph: eager step")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    ws2 = torch.empty(pkv.workspace_size(c.gk, B, Hq, max(lens), window=1000, num_sinks=4), dtype=torch.uint8,
                      device="cuda")
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {i} differs from the eager step"
        # eager work between replays, on another workspace and with another plan
        pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens), window=1000,
                                   num_sinks=4, workspace=ws2)
        torch.cuda.synchronize()


def test_prepared_call_equals_wrapper():
    """prepare_decode_append_attention (checked and marshalled once, one library call per step)
    gives the wrapper's result bit for bit, call after call, and follows the tensors' contents."""
    import paged_kv_cache_16_amd as pkv
    lens = [1500, 333, 4000, 2, 0, 129]
    B, Hq, Hkv = 6, 16, 4
    c = make_case(57, B=B, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16", P=16, lens=lens)
    slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, c.P) if L > 0 else -1 for b, L in enumerate(lens)],
                         dtype=torch.int32).cuda()
    kn = torch.stack([c.K[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
    vn = torch.stack([c.V[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
    ref = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl, max_context_len=4000)
    call = pkv.prepare_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl, max_context_len=4000)
    for _ in range(3):
        out, lse = call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
    assert_close(c, (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)), oracle_attend(c),
                 "prepared call")
    c.gq.mul_(0.5)  # new contents of the same tensor: the prepared call sees them
    ref2 = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl, max_context_len=4000)
    out2, lse2 = call()
    torch.cuda.synchronize()
    assert torch.equal(out2, ref2[0]) and torch.equal(lse2, ref2[1]) and not torch.equal(out2, ref[0])
