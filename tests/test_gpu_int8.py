"""INT8 KV cache ([primer] §4.2, §5.2: an int8 cache dtype halves the bytes per token) on the
GPU, through the C ABI, against the oracle's INT8 path: the quantising append bit for bit
(data plane, scale plane and untouched bytes), attention within the 2-byte tolerance, the
fused decode step, score export and the full Llama-3-8B-shaped layer.

Attention tolerance: as for bf16 / fp16 caches (2e-3). The int8 values widen to bf16 / fp16
exactly, products with q are exact in fp32, a row's scale enters the logit as one fp32
multiply and V's scale enters through P before P's two-part split, so the error is that of
the 2-byte path. Pools start as 0xFF bytes (int8 -1, scales NaN) so that reading a token
that was never appended, or a masked token's scale, shows up."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import assert_close, log, raw_bytes

pytestmark = pytest.mark.gpu
TDT = {"i8bf16": torch.bfloat16, "i8f16": torch.float16}
IN = {"i8bf16": "bf16", "i8f16": "f16"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def make_case8(seed, *, B, Hq, Hkv, d, dtype, P, lens, gpu_append=True, drop_last=False):
    import paged_kv_cache_16_amd as pkv
    lens = [int(x) for x in lens]
    Lmax = max(lens + [1])
    ind = IN[dtype]
    q = synth.normal((B, Hq, d), seed, "q", dtype=ind)
    K = synth.normal((B, Lmax, Hkv, d), seed, "k", dtype=ind)
    V = synth.normal((B, Lmax, Hkv, d), seed, "v", dtype=ind)
    bt, nb = synth.block_tables(lens, P, seed, spare_blocks=1)
    used = set(bt[bt >= 0].tolist())
    pad = [x for x in range(nb) if x not in used][0]
    bt = torch.where(bt >= 0, bt, torch.full_like(bt, pad))
    slots = synth.token_slots(bt, lens, P)
    kn = torch.cat([K[b, :L] for b, L in enumerate(lens)])
    vn = torch.cat([V[b, :L] for b, L in enumerate(lens)])
    kpool = np.full(nb * Hkv * P * (d + 4), 0xFF, np.uint8)
    vpool = kpool.copy()
    oracle.kv_append(dtype, kpool, vpool, synth.raw_numpy(kn), synth.raw_numpy(vn), slots.numpy(), P=P, Hkv=Hkv, d=d)
    c = SimpleNamespace(q=q, K=K, V=V, bt=bt, nb=nb, lens=lens, P=P, Hkv=Hkv, Hq=Hq, d=d, dtype=dtype, B=B,
                        kpool=kpool, vpool=vpool, slots=slots)
    c.gk = pkv.new_cache(nb, Hkv, P, d, torch.int8)
    c.gv = pkv.new_cache(nb, Hkv, P, d, torch.int8)
    c.gk.fill_(-1)
    c.gv.fill_(-1)
    if drop_last:  # all but each sequence's last token: a fused step appends it
        pre = synth.token_slots(bt, lens, P, last=[max(L - 1, 0) for L in lens])
        kp = torch.cat([K[b, :max(L - 1, 0)] for b, L in enumerate(lens)])
        vp = torch.cat([V[b, :max(L - 1, 0)] for b, L in enumerate(lens)])
        if kp.shape[0]:
            pkv.kv_cache_append(c.gk, c.gv, kp.cuda(), vp.cuda(), pre.cuda())
    elif gpu_append:
        pkv.kv_cache_append(c.gk, c.gv, kn.cuda(), vn.cuda(), slots.cuda())
    c.gq, c.gbt = q.cuda(), bt.cuda()
    c.gcl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return c


def oracle_attend8(c, **kw):
    return oracle.decode_attention(c.dtype, c.kpool, c.vpool, synth.raw_numpy(c.q), c.bt.numpy(),
                                   np.array(c.lens, np.int32), P=c.P, Hkv=c.Hkv, d=c.d, **kw)


def tol_case(c):
    return SimpleNamespace(dtype=IN[c.dtype])


@pytest.mark.parametrize("dtype,d,P", [("i8bf16", 128, 16), ("i8f16", 64, 32), ("i8bf16", 64, 16)])
def test_int8_append_bit_exact(dtype, d, P):
    c = make_case8(80, B=3, Hq=4, Hkv=2, d=d, dtype=dtype, P=P, lens=[70, 1, 33])
    torch.cuda.synchronize()
    assert np.array_equal(raw_bytes(c.gk), c.kpool)
    assert np.array_equal(raw_bytes(c.gv), c.vpool)


def test_int8_append_zero_row_and_skipped_slots():
    import paged_kv_cache_16_amd as pkv
    nb, Hkv, P, d = 4, 2, 16, 128
    g = pkv.new_cache(nb, Hkv, P, d, torch.int8)
    g.fill_(-1)
    gv = g.clone()
    k = synth.normal((3, Hkv, d), 81, "k", dtype="bf16")
    k[1] = 0.0  # a zero row: scale 0, all int8 0
    v = synth.normal((3, Hkv, d), 81, "v", dtype="bf16")
    slots = torch.tensor([5, 17, -1], dtype=torch.int32)
    pkv.kv_cache_append(g, gv, k.cuda(), v.cuda(), slots.cuda())
    torch.cuda.synchronize()
    kp = np.full(nb * Hkv * P * (d + 4), 0xFF, np.uint8)
    vp = kp.copy()
    oracle.kv_append("i8bf16", kp, vp, synth.raw_numpy(k), synth.raw_numpy(v), slots.numpy(), P=P, Hkv=Hkv, d=d)
    assert np.array_equal(raw_bytes(g), kp) and np.array_equal(raw_bytes(gv), vp)


INT8_CASES = [
    dict(name="llama3-shape", B=4, Hq=32, Hkv=8, d=128, dtype="i8bf16", P=16, lens=[1500, 4096, 17, 2049], kw={}),
    dict(name="g6-window", B=3, Hq=12, Hkv=2, d=128, dtype="i8bf16", P=16, lens=[4100, 600, 31],
         kw=dict(window=512, num_sinks=4)),
    dict(name="f16-pages", B=2, Hq=8, Hkv=8, d=128, dtype="i8f16", P=32, lens=[1000, 64], kw="pages"),
    dict(name="d64-g1-tiny", B=3, Hq=4, Hkv=4, d=64, dtype="i8f16", P=16, lens=[100, 0, 7], kw={}),
    dict(name="d64-g8", B=2, Hq=16, Hkv=2, d=64, dtype="i8bf16", P=16, lens=[333, 70], kw={}),
]


def _kw(c, kw):
    if kw == "pages":
        pl = synth.page_lists(c.lens, c.P, 6, 82).numpy()
        return dict(page_list=torch.as_tensor(pl).cuda()), dict(page_list=pl)
    if "window" in kw:
        return kw, dict(window=kw["window"], sinks=kw["num_sinks"])
    return kw, {}


@pytest.mark.parametrize("ic", INT8_CASES, ids=[x["name"] for x in INT8_CASES])
def test_int8_attention(ic):
    import paged_kv_cache_16_amd as pkv
    log(f"int8 {ic['name']}")
    c = make_case8(82, B=ic["B"], Hq=ic["Hq"], Hkv=ic["Hkv"], d=ic["d"], dtype=ic["dtype"], P=ic["P"], lens=ic["lens"])
    gkw, okw = _kw(c, ic["kw"])
    out, lse = pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(c.lens), **gkw)
    torch.cuda.synchronize()
    got = (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    assert_close(tol_case(c), got, oracle_attend8(c, **okw), f"int8 {ic['name']}")


@pytest.mark.parametrize("with_scores", [False, True], ids=["plain", "scores"])
@pytest.mark.parametrize("ic", INT8_CASES, ids=[x["name"] for x in INT8_CASES])
def test_int8_fused_step_and_scores(ic, with_scores):
    """paged_decode_append_attention on an INT8 cache (the new row quantised inside the attention
    kernel, stored by the combine): the cache bytes equal the oracle's append, the outputs and the
    exported scores match the oracle."""
    import paged_kv_cache_16_amd as pkv
    c = make_case8(83, B=ic["B"], Hq=ic["Hq"], Hkv=ic["Hkv"], d=ic["d"], dtype=ic["dtype"], P=ic["P"],
                   lens=ic["lens"], drop_last=True)
    lens = c.lens
    slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, c.P) if L > 0 else -1 for b, L in enumerate(lens)],
                         dtype=torch.int32).cuda()
    kn = torch.stack([c.K[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
    vn = torch.stack([c.V[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
    gkw, okw = _kw(c, ic["kw"])
    stride = max(lens)
    gs = torch.zeros((c.B, c.Hkv, stride), dtype=torch.float32, device="cuda")
    log(f"int8 fused {ic['name']} scores={with_scores}")
    out, lse = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl,
                                                 max_context_len=max(lens), scores=gs if with_scores else None,
                                                 **gkw)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bytes(c.gk), c.kpool) and np.array_equal(raw_bytes(c.gv), c.vpool)
    got = (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    assert_close(tol_case(c), got, oracle_attend8(c, **okw), f"int8 fused {ic['name']}")
    if not with_scores:
        return
    ref = oracle.decode_scores(c.dtype, c.kpool, synth.raw_numpy(c.q), c.bt.numpy(), np.array(lens, np.int32),
                               P=c.P, Hkv=c.Hkv, d=c.d, stride=stride, **okw)
    err = float(np.abs(gs.cpu().double().numpy() - ref).max())
    log(f"    max|score err| = {err:.3e}")
    assert err <= 1e-5


def test_int8_fused_step_edge_rows():
    """The fused step's in-kernel quantisation at its edges: an all-zero K and V row (scale 0,
    codes 0), rows with one large element (every other code rounds to 0 or +-1), a sequence of
    length 1 (the new token alone) and a skipped store (slot -1: the token is still attended,
    quantised, and the cache keeps what it held)."""
    import paged_kv_cache_16_amd as pkv
    lens = [300, 17, 1, 70]
    B, Hq, Hkv, d, P, dt = 4, 8, 2, 128, 16, "i8bf16"
    c = make_case8(85, B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dt, P=P, lens=lens, drop_last=True)
    c.K[0, lens[0] - 1] = 0.0
    c.V[0, lens[0] - 1] = 0.0
    c.K[1, lens[1] - 1] = 0.01
    c.K[1, lens[1] - 1, :, 5] = 50.0
    c.V[1, lens[1] - 1] = -0.02
    c.V[1, lens[1] - 1, :, 77] = -3.0
    kn = torch.stack([c.K[b, L - 1] for b, L in enumerate(lens)])
    vn = torch.stack([c.V[b, L - 1] for b, L in enumerate(lens)])
    true_slots = [synth.slot_of(c.bt, b, L - 1, P) for b, L in enumerate(lens)]
    store_slots = true_slots[:3] + [-1]
    # oracle pools: the prefixes, then the new rows (all of them for attention, the stored ones
    # for the cache bytes)
    pre = synth.token_slots(c.bt, lens, P, last=[L - 1 for L in lens])
    kp = torch.cat([c.K[b, :L - 1] for b, L in enumerate(lens)])
    vp = torch.cat([c.V[b, :L - 1] for b, L in enumerate(lens)])
    base_k = np.full(c.nb * Hkv * P * (d + 4), 0xFF, np.uint8)
    base_v = base_k.copy()
    oracle.kv_append(dt, base_k, base_v, synth.raw_numpy(kp), synth.raw_numpy(vp), pre.numpy(), P=P, Hkv=Hkv, d=d)
    att_k, att_v, st_k, st_v = base_k.copy(), base_v.copy(), base_k.copy(), base_v.copy()
    oracle.kv_append(dt, att_k, att_v, synth.raw_numpy(kn), synth.raw_numpy(vn), np.array(true_slots, np.int32),
                     P=P, Hkv=Hkv, d=d)
    oracle.kv_append(dt, st_k, st_v, synth.raw_numpy(kn), synth.raw_numpy(vn), np.array(store_slots, np.int32),
                     P=P, Hkv=Hkv, d=d)
    log(f"int8 fused edge rows lens={lens}")
    out, lse = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn.cuda(), vn.cuda(),
                                                 torch.tensor(store_slots, dtype=torch.int32).cuda(), c.gbt, c.gcl,
                                                 max_context_len=max(lens))
    torch.cuda.synchronize()
    assert np.array_equal(raw_bytes(c.gk), st_k) and np.array_equal(raw_bytes(c.gv), st_v)
    ref = oracle.decode_attention(dt, att_k, att_v, synth.raw_numpy(c.q), c.bt.numpy(), np.array(lens, np.int32),
                                  P=P, Hkv=Hkv, d=d)
    got = (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    assert_close(tol_case(c), got, ref, "int8 fused edge rows")


def test_int8_status_codes():
    import paged_kv_cache_16_amd as pkv
    c = make_case8(84, B=1, Hq=4, Hkv=2, d=128, dtype="i8bf16", P=16, lens=[300])
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=300, split_tokens=64)
    assert e.value.status == 3
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_decode_attention_partial(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=300, split_tokens=64)
    assert e.value.status == 3
