"""Full-size GPU parity: every sequence, at the benchmarked workload sizes, in the launch
configuration the benchmark times, against the oracle.

Single layers: the Llama-3-8B-shaped layer (bf16 and INT8 caches), the page-selected MHA-7B
step and the KV-sparse window layer, each as a plain attention call and as the fused decode
step. Whole models: the Qwen2.5-1.5B-shaped 28-layer decode (4096 cached tokens, then 32
steps of append + attention on every layer, the context advanced once per step after the last
layer; every layer checked at steps 1 and 32) and the KV-sparse Llama-3-8B-shaped 32-layer step
(16 full layers, 16 window layers; every layer checked).

The GPU side draws every row on the device from per-(layer, sequence) seeds; the oracle side
draws the same rows again, appends them into its own pool per sequence (only the attended
tokens for window and page-list attention, so any other token is NaN there) and runs on host
threads. Tolerance: 2e-3 absolute on the outputs (bf16 / fp16), as everywhere."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import pytest
import torch

import synth
from harness import (ORACLE_THREADS, assert_close, log, oracle_sequence, page_tokens, run_threads,
                     window_tokens)

pytestmark = pytest.mark.gpu
SEED = 7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _lens(w, seed):
    if w.ctx_lo == w.ctx_hi:
        return [w.ctx_lo] * w.batch
    return synth.uniform_lengths(w.batch, w.ctx_lo, w.ctx_hi, seed, w.name).tolist()


def _check_all(tasks, got, dtype, what):
    """tasks: (label, callable returning [(out, lse), ...]); got: label -> [(out, lse), ...] of
    the GPU. Runs the oracle on host threads in chunks (bounded host memory) and compares."""
    worst = 0.0
    tol = SimpleNamespace(dtype=dtype)
    chunk = 2 * ORACLE_THREADS
    for i in range(0, len(tasks), chunk):
        part = tasks[i:i + chunk]
        refs = run_threads([fn for _, fn in part])
        for (label, _), ref_list in zip(part, refs):
            for k, ref in enumerate(ref_list):
                g = got[label][k]
                assert_close(tol, g, ref, f"{what} {label} eval {k}")
                worst = max(worst, float(np.abs(g[0] - ref[0]).max()))
        log(f"  {what}: {min(i + chunk, len(tasks))}/{len(tasks)} sequences checked, worst |out err| {worst:.3e}")
    return worst


# ------------------------------------------------------------------------------ single layers
def _single_layer(name, *, fused, window=0, sinks=0, pages=0, int8=False, seed=SEED):
    import paged_kv_cache_16_amd as pkv
    w = synth.WORKLOADS[name]
    B, P, d, Hkv, Hq = w.batch, w.block_size, w.head_dim, w.kv_heads, w.q_heads
    lens = _lens(w, seed)
    log(f"{name} full size B={B} sum(L)={sum(lens)} fused={fused} int8={int8} window={window} pages={pages}")
    dev = torch.device("cuda")
    bt, nb = synth.block_tables(lens, P, seed, name)
    gk = pkv.new_cache(nb, Hkv, P, d, torch.int8 if int8 else synth.TORCH_DTYPE[w.dtype], device=dev)
    gv = torch.empty_like(gk)
    qs = synth.normal((B, Hq, d), seed, name, "q", dtype=w.dtype)
    page_list = synth.page_lists(lens, P, pages, seed, name) if pages else None

    def rows(b, tag):
        return synth.normal((lens[b], Hkv, d), seed, name, b, tag, dtype=w.dtype, device=dev)

    gcl = torch.tensor(lens, dtype=torch.int32, device=dev)
    kw = dict(max_context_len=max(lens), window=window, num_sinks=sinks,
              page_list=None if page_list is None else page_list.to(dev))
    if not fused:
        for b, L in enumerate(lens):
            pkv.kv_cache_append(gk, gv, rows(b, "k"), rows(b, "v"), synth.token_slots(bt[b:b + 1], [L], P).to(dev))
        out, lse = pkv.paged_decode_attention(qs.to(dev), gk, gv, bt.to(dev), gcl, **kw)
    else:
        kn, vn = [], []
        for b, L in enumerate(lens):
            kb, vb = rows(b, "k"), rows(b, "v")
            pkv.kv_cache_append(gk, gv, kb[:L - 1].contiguous(), vb[:L - 1].contiguous(),
                                synth.token_slots(bt[b:b + 1], [L - 1], P).to(dev))
            kn.append(kb[L - 1])
            vn.append(vb[L - 1])
        slots = torch.tensor([synth.slot_of(bt, b, L - 1, P) for b, L in enumerate(lens)], dtype=torch.int32,
                             device=dev)
        out, lse = pkv.paged_decode_append_attention(qs.to(dev), gk, gv, torch.stack(kn), torch.stack(vn), slots,
                                                     bt.to(dev), gcl, **kw)
        # a plain attention call afterwards reads the stored new rows back: the same bits
        out2, lse2 = pkv.paged_decode_attention(qs.to(dev), gk, gv, bt.to(dev), gcl, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(lse, lse2), "stored new rows read back differ"
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    del gk, gv
    torch.cuda.empty_cache()

    odt = "i8bf16" if int8 else w.dtype
    tasks, got = [], {}
    for b, L in enumerate(lens):
        if page_list is not None:
            toks, okw = page_tokens(L, P, page_list[b].tolist()), dict(page_list=page_list[b:b + 1].numpy())
        elif window:
            toks, okw = window_tokens(L, window, sinks), dict(window=window, sinks=sinks)
        else:
            toks, okw = None, {}
        idx = None if toks is None else torch.as_tensor(toks, device=dev)
        kb, vb = rows(b, "k"), rows(b, "v")
        kb, vb = (kb, vb) if idx is None else (kb[idx], vb[idx])
        kb, vb = kb.cpu(), vb.cpu()
        label = f"seq {b} (L={L})"
        got[label] = [(out[b:b + 1], lse[b:b + 1])]
        tasks.append((label, lambda kb=kb, vb=vb, q=qs[b:b + 1], L=L, okw=okw, toks=toks: oracle_sequence(
            odt, kb, vb, [(q, L, okw)], n_tokens=L, P=P, Hkv=Hkv, d=d, seed=seed, tokens=toks)))
    _check_all(tasks, got, w.dtype, name)


@pytest.mark.parametrize("fused", [False, True], ids=["attention", "fused-step"])
def test_llama3_layer_every_sequence(fused):
    _single_layer("llama3_8b_layer_bf16", fused=fused)


@pytest.mark.parametrize("fused", [False, True], ids=["attention", "fused-step"])
def test_llama3_layer_int8_every_sequence(fused):
    _single_layer("llama3_8b_layer_bf16", fused=fused, int8=True)


@pytest.mark.parametrize("fused", [False, True], ids=["attention", "fused-step"])
def test_page_selected_every_sequence(fused):
    _single_layer("mha7b_pagesel_f16", fused=fused, pages=16)


@pytest.mark.parametrize("fused", [False, True], ids=["attention", "fused-step"])
def test_kvsparse_window_layer_every_sequence(fused):
    w = synth.WORKLOADS["llama3_8b_kvsparse_bf16"]
    _single_layer(w.name, fused=fused, window=w.window, sinks=w.sinks)


# -------------------------------------------------------------------------------- whole models
def _model_steps(name, *, checked_steps, seed=SEED):
    """Runs every decode step of the workload on the GPU (per layer: the fused append +
    attention; window layers with their window and sinks), keeps every layer's output at the
    checked steps, then checks each (layer, sequence, checked step) against the oracle."""
    import paged_kv_cache_16_amd as pkv
    w = synth.WORKLOADS[name]
    B, P, d, Hkv, Hq = w.batch, w.block_size, w.head_dim, w.kv_heads, w.q_heads
    steps = w.steps
    if w.ctx_lo == w.ctx_hi:
        first = [w.ctx_lo + 1] * B  # context cached before step 1, plus the step's token
    else:
        first = synth.uniform_lengths(B, w.ctx_lo, w.ctx_hi, seed, w.name).tolist()
    cap = [L + steps - 1 for L in first]  # length at the last step
    log(f"{name}: B={B}, {w.layers} layers ({len(w.window_layers)} window), {steps} steps, "
        f"L {min(first)}..{max(cap)}")
    dev = torch.device("cuda")
    bt, nb = synth.block_tables(cap, P, seed, name)  # one table for every layer
    gbt = bt.to(dev)
    tdt = synth.TORCH_DTYPE[w.dtype]

    def rows(layer, b, tag):  # logical rows of every token up to the last step
        return synth.normal((cap[b], Hkv, d), seed, name, layer, b, tag, dtype=w.dtype, device=dev)

    def q_of(layer, s):
        return synth.normal((B, Hq, d), seed, name, layer, s, "q", dtype=w.dtype, device=dev)

    layers = []
    for layer in range(w.layers):
        gk = torch.empty((nb, Hkv, P, d), dtype=tdt, device=dev)
        gv = torch.empty_like(gk)
        kn = torch.empty((steps, B, Hkv, d), dtype=tdt, device=dev)
        vn = torch.empty_like(kn)
        for b, L in enumerate(first):  # cache tokens [0, L-1); tokens L-1 .. are the steps' new rows
            kb, vb = rows(layer, b, "k"), rows(layer, b, "v")
            pkv.kv_cache_append(gk, gv, kb[:L - 1].contiguous(), vb[:L - 1].contiguous(),
                                synth.token_slots(bt[b:b + 1], [L - 1], P).to(dev))
            kn[:, b] = kb[L - 1:]
            vn[:, b] = vb[L - 1:]
        layers.append(dict(k=gk, v=gv, kn=kn, vn=vn, window=w.window if layer in w.window_layers else 0))
    got = {}
    for s in range(steps):
        lens_s = [L + s for L in first]
        gcl = torch.tensor(lens_s, dtype=torch.int32, device=dev)
        slots = torch.tensor([synth.slot_of(bt, b, L - 1, P) for b, L in enumerate(lens_s)], dtype=torch.int32,
                             device=dev)
        for li, ly in enumerate(layers):
            out, lse = pkv.paged_decode_append_attention(
                q_of(li, s), ly["k"], ly["v"], ly["kn"][s], ly["vn"][s], slots, gbt, gcl,
                max_context_len=max(cap), window=ly["window"], num_sinks=w.sinks if ly["window"] else 0)
            if s in checked_steps:
                got[(li, s)] = (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
        # the context advances once per step, after the last layer
    torch.cuda.synchronize()
    log(f"  GPU: {steps} steps x {w.layers} layers done")
    del layers
    torch.cuda.empty_cache()

    tasks, got_seq = [], {}
    for li in range(w.layers):
        win = w.window if li in w.window_layers else 0
        qs = {s: q_of(li, s).cpu() for s in checked_steps}
        for b in range(B):
            Lmax = first[b] + max(checked_steps)  # the longest context checked
            if win:  # only the tokens some checked step attends
                toks = np.unique(np.concatenate([window_tokens(first[b] + s, win, w.sinks) for s in checked_steps]))
            else:
                toks = np.arange(Lmax)
            idx = torch.as_tensor(toks, device=dev)
            kb, vb = rows(li, b, "k")[idx].cpu(), rows(li, b, "v")[idx].cpu()
            okw = dict(window=win, sinks=w.sinks) if win else {}
            evals = [(qs[s][b:b + 1], first[b] + s, okw) for s in checked_steps]
            label = f"layer {li} seq {b}"
            got_seq[label] = [(got[(li, s)][0][b:b + 1], got[(li, s)][1][b:b + 1]) for s in checked_steps]
            tasks.append((label, lambda kb=kb, vb=vb, evals=evals, Lmax=Lmax, toks=toks: oracle_sequence(
                w.dtype, kb, vb, evals, n_tokens=Lmax, P=P, Hkv=Hkv, d=d, seed=seed, tokens=toks)))
    _check_all(tasks, got_seq, w.dtype, name)


def test_qwen_28_layers_32_steps():
    """4096 cached tokens, then 32 decode steps of every layer; each layer's output at steps 1
    (L = 4097) and 32 (L = 4128) against the oracle, every sequence."""
    _model_steps("qwen25_1p5b_28l_bf16", checked_steps=(0, 31))


def test_kvsparse_32_layer_step():
    """The whole 32-layer step (layers 0-7 and 24-31 full, 8-23 window 512 + 4 sinks), every
    layer and every sequence against the oracle."""
    _model_steps("llama3_8b_kvsparse_bf16", checked_steps=(0,))
