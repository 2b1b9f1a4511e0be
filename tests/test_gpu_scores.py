"""GPU parity of the decode-time KV score export ([Novita] §關鍵技術 2: a token's score is its
softmax probability, summed over the query heads of its kv head and accumulated over steps),
through the C ABI, against the oracle's decode_scores.

Tolerance: a score is a sum of at most G = 8 probabilities p = 2^(x - lse2) <= 1 computed in
fp32 from fp32 logits (MFMA accumulation of exact products) and an fp32 normaliser; each
term's relative error is at most a few 1e-7 (logit and normaliser rounding, the hardware
exp2), so 1e-5 absolute per token bounds the sum for every dtype with a wide margin. The random initial values the scores are added to are carried exactly by both sides
(fp32 on the GPU, the same values as doubles in the oracle)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import assert_close, log, make_case, oracle_attend, oracle_pool, run_threads

pytestmark = pytest.mark.gpu
SCORE_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


SCORE_CASES = [
    dict(name="llama3-shape", B=4, Hq=32, Hkv=8, d=128, dtype="bf16", P=16, lens=[1500, 4096, 17, 2049], kw={}),
    dict(name="g6-window", B=3, Hq=12, Hkv=2, d=128, dtype="bf16", P=16, lens=[4100, 600, 31],
         kw=dict(window=512, num_sinks=4)),
    dict(name="f16-pages", B=2, Hq=8, Hkv=8, d=128, dtype="f16", P=32, lens=[1000, 64], kw="pages"),
    dict(name="f32-d64-tiny", B=3, Hq=4, Hkv=4, d=64, dtype="f32", P=16, lens=[100, 0, 7], kw={}),
    dict(name="g8-f16-d64", B=2, Hq=16, Hkv=2, d=64, dtype="f16", P=16, lens=[333, 70], kw={}),
]


def _oracle_scores(c, stride, init, okw):
    return oracle.decode_scores(c.dtype, c.kpool, synth.raw_numpy(c.q), c.bt.numpy(), np.array(c.lens, np.int32),
                                P=c.P, Hkv=c.Hkv, d=c.d, stride=stride, score=init.double().numpy(), **okw)


@pytest.mark.parametrize("fused", [False, True], ids=["attention", "fused-step"])
@pytest.mark.parametrize("sc", SCORE_CASES, ids=[s["name"] for s in SCORE_CASES])
def test_score_export(sc, fused):
    import paged_kv_cache_16_amd as pkv
    lens = sc["lens"]
    log(f"scores {sc['name']} fused={fused}")
    c = make_case(70, B=sc["B"], Hq=sc["Hq"], Hkv=sc["Hkv"], d=sc["d"], dtype=sc["dtype"], P=sc["P"], lens=lens)
    kw, okw = sc["kw"], {}
    if kw == "pages":
        pl = synth.page_lists(lens, c.P, 6, 70).numpy()
        kw = dict(page_list=torch.as_tensor(pl).cuda())
        okw = dict(page_list=pl)
    elif "window" in kw:
        okw = dict(window=kw["window"], sinks=kw["num_sinks"])
    stride = max(lens) + 5
    init = synth.normal((c.B, c.Hkv, stride), 70, "score-init", dtype="f32")
    gs = init.clone().cuda()
    if fused:
        # GPU cache without each sequence's last token: the fused call appends it
        c.gk.fill_(float("nan"))
        c.gv.fill_(float("nan"))
        pre = synth.token_slots(c.bt, lens, c.P, last=[max(L - 1, 0) for L in lens])
        kp = torch.cat([c.K[b, :max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
        vp = torch.cat([c.V[b, :max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
        if kp.shape[0]:
            pkv.kv_cache_append(c.gk, c.gv, kp, vp, pre.cuda())
        slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, c.P) if L > 0 else -1 for b, L in enumerate(lens)],
                             dtype=torch.int32).cuda()
        kn = torch.stack([c.K[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
        vn = torch.stack([c.V[b, max(L - 1, 0)] for b, L in enumerate(lens)]).cuda()
        out, lse = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl,
                                                     max_context_len=max(lens), scores=gs, **kw)
    else:
        out, lse = pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens),
                                              scores=gs, **kw)
    torch.cuda.synchronize()
    ref = _oracle_scores(c, stride, init, okw)
    err = float(np.abs(gs.cpu().double().numpy() - ref).max())
    log(f"    max|score err| = {err:.3e}")
    assert err <= SCORE_TOL
    got = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    assert_close(c, got, oracle_attend(c, **okw), f"scores {sc['name']} outputs")


ONE_KERNEL_CASES = [("full", 1), ("full", 32), ("window", 1), ("window", 5), ("pages", 32), ("pages", 1)]


@pytest.mark.parametrize("fused", [False, True], ids=["attention", "fused-step"])
@pytest.mark.parametrize("mode,block", ONE_KERNEL_CASES, ids=[f"{m}-B{b}" for m, b in ONE_KERNEL_CASES])
def test_score_export_one_kernel(mode, block, fused):
    """Score export on the one-kernel path (64 segments of at most 40 units: no workspace), per
    token, per page and per odd-sized entry, against the oracle; the cache is NaN-filled past
    every context and, in the fused step, holds no copy of the new token."""
    import paged_kv_cache_16_amd as pkv
    B, Hq, Hkv, P = 16, 8, 4, 32
    rng = np.random.default_rng(75 + block)
    lens = [int(x) for x in rng.integers(1, 620, size=B)]
    lens[3] = 1
    log(f"one-kernel scores {mode} B={block} fused={fused}")
    c = make_case(75, B=B, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16", P=P, lens=lens)
    kw, okw = {}, {}
    if mode == "window":
        kw, okw = dict(window=150, num_sinks=5), dict(window=150, sinks=5)
    elif mode == "pages":
        pl = synth.page_lists(lens, P, 5, 75).numpy()
        kw, okw = dict(page_list=torch.as_tensor(pl).cuda()), dict(page_list=pl)
    stride = (max(lens) + block - 1) // block + 3
    assert pkv.workspace_size(c.gk, B, Hq, max(lens), scores=True, window=kw.get("window", 0),
                              num_sinks=kw.get("num_sinks", 0), page_list=kw.get("page_list")) == 0
    init = synth.normal((B, Hkv, stride), 75, "score-init", block, dtype="f32")
    gs = init.clone().cuda()
    if fused:
        c.gk.fill_(float("nan"))
        c.gv.fill_(float("nan"))
        pre = synth.token_slots(c.bt, lens, P, last=[L - 1 for L in lens])
        kp = torch.cat([c.K[b, :L - 1] for b, L in enumerate(lens)]).cuda()
        vp = torch.cat([c.V[b, :L - 1] for b, L in enumerate(lens)]).cuda()
        pkv.kv_cache_append(c.gk, c.gv, kp, vp, pre.cuda())
        slots = torch.tensor([synth.slot_of(c.bt, b, L - 1, P) for b, L in enumerate(lens)], dtype=torch.int32).cuda()
        kn = torch.stack([c.K[b, L - 1] for b, L in enumerate(lens)]).cuda()
        vn = torch.stack([c.V[b, L - 1] for b, L in enumerate(lens)]).cuda()
        out, lse = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn, vn, slots, c.gbt, c.gcl,
                                                     max_context_len=max(lens), scores=gs, score_block=block, **kw)
    else:
        out, lse = pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens),
                                              scores=gs, score_block=block, **kw)
    torch.cuda.synchronize()
    ref = oracle.decode_scores(c.dtype, c.kpool, synth.raw_numpy(c.q), c.bt.numpy(), np.array(lens, np.int32),
                               P=P, Hkv=Hkv, d=128, stride=stride, score=init.double().numpy(), block=block, **okw)
    err = float(np.abs(gs.cpu().double().numpy() - ref).max())
    log(f"    max|score err| = {err:.3e}")
    assert err <= SCORE_TOL
    got = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    assert_close(c, got, oracle_attend(c, **okw), f"one-kernel scores {mode} outputs")


def test_score_accumulates_over_steps():
    """Two calls on one array add two steps' scores; tokens outside the window keep theirs."""
    import paged_kv_cache_16_amd as pkv
    lens = [700, 50]
    c = make_case(71, B=2, Hq=8, Hkv=2, d=128, dtype="bf16", P=16, lens=lens)
    stride = 704
    gs = torch.zeros((2, 2, stride), dtype=torch.float32, device="cuda")
    for _ in range(2):
        pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens), window=100,
                                   num_sinks=3, scores=gs)
    torch.cuda.synchronize()
    one = _oracle_scores(c, stride, torch.zeros((2, 2, stride)), dict(window=100, sinks=3))
    got = gs.cpu().double().numpy()
    assert np.abs(got - 2 * one).max() <= 2 * SCORE_TOL
    assert np.all(got[0, :, 3:600] == 0.0)  # outside sinks and window: untouched


def test_score_export_full_size_llama3_layer():
    """Full Llama-3-8B-shaped layer (the benchmark's shape and launch configuration): every
    (sequence, kv head) row of scores sums to G, and every sequence matches the oracle."""
    import paged_kv_cache_16_amd as pkv
    name, seed = "llama3_8b_layer_bf16", 7
    w = synth.WORKLOADS[name]
    B, P, d, Hkv, Hq = w.batch, w.block_size, w.head_dim, w.kv_heads, w.q_heads
    G = Hq // Hkv
    lens = synth.uniform_lengths(B, w.ctx_lo, w.ctx_hi, seed, name).tolist()
    dev = torch.device("cuda")
    bt, nb = synth.block_tables(lens, P, seed, name)
    gk = torch.empty((nb, Hkv, P, d), dtype=torch.bfloat16, device=dev)
    gv = torch.empty_like(gk)
    qs = synth.normal((B, Hq, d), seed, name, "q", dtype=w.dtype)

    def rows(b, tag):
        return synth.normal((lens[b], Hkv, d), seed, name, b, tag, dtype=w.dtype, device=dev)

    for b, L in enumerate(lens):
        pkv.kv_cache_append(gk, gv, rows(b, "k"), rows(b, "v"), synth.token_slots(bt[b:b + 1], [L], P).to(dev))
    stride = max(lens)
    gs = torch.zeros((B, Hkv, stride), dtype=torch.float32, device=dev)
    pkv.paged_decode_attention(qs.to(dev), gk, gv, bt.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev),
                               max_context_len=max(lens), scores=gs)
    torch.cuda.synchronize()
    sums = gs.double().sum(-1).cpu().numpy()
    log(f"    max|row sum - G| = {np.abs(sums - G).max():.3e}")
    assert np.abs(sums - G).max() <= 1e-4
    got = gs.cpu().double().numpy()
    del gk, gv

    def one(b, kb, vb):  # the oracle's scores of sequence b, from zero
        kp, _, bt1 = oracle_pool(w.dtype, kb, vb, n_tokens=lens[b], P=P, Hkv=Hkv, d=d, seed=seed)
        return oracle.decode_scores(w.dtype, kp, synth.raw_numpy(qs[b:b + 1]), bt1, np.array([lens[b]], np.int32),
                                    P=P, Hkv=Hkv, d=d, stride=stride)

    tasks = [lambda b=b, kb=rows(b, "k").cpu(), vb=rows(b, "v").cpu(): one(b, kb, vb) for b in range(B)]
    worst = 0.0
    for b, ref in enumerate(run_threads(tasks)):  # every sequence
        err = float(np.abs(got[b:b + 1] - ref).max())
        worst = max(worst, err)
        assert err <= SCORE_TOL, f"seq {b}: max|score err| = {err:.3e}"
    log(f"    every sequence: max|score err| = {worst:.3e}")
