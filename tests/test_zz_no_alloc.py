"""paged_decode_attention_noalloc, the entry point for callers that cannot allocate device
memory, through the C ABI: its outputs equal those of paged_decode_attention given a caller
workspace (same kernels, same plan: bit for bit) and the oracle's (2e-3 for bf16), on calls in a
row whose sizes differ, the later ones smaller, so each call runs over what the previous one
left in the library's scratch. A call needing more than the scratch holds is refused before
anything is enqueued."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import assert_close, log, make_case, oracle_attend

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _both(c, **kw):
    """(workspace entry point, no-allocation entry point) outputs for case c."""
    import paged_kv_cache_16_amd as pkv
    B, Hq, d = c.gq.shape
    mcl = max(c.lens)
    n_ws = pkv.workspace_size(c.gk, B, Hq, mcl, window=kw.get("window", 0), num_sinks=kw.get("num_sinks", 0),
                              split_tokens=kw.get("split_tokens", 0), scores=kw.get("scores"))
    assert n_ws > 0, "the case is meant to need a workspace"
    ws = torch.full((n_ws,), 0x5A, dtype=torch.uint8, device="cuda")
    out_w, lse_w = pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=mcl, workspace=ws,
                                              **{k: v for k, v in kw.items() if k != "scores_na"})
    out_n = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse_n = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    kw_n = dict(kw)
    if "scores" in kw:
        kw_n["scores"] = kw_n.pop("scores_na")
    pkv.paged_decode_attention_noalloc(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=mcl, out=out_n, lse=lse_n,
                                       **kw_n)
    torch.cuda.synchronize()
    return (out_w, lse_w), (out_n, lse_n), n_ws


def _np(t):
    return t.cpu().numpy().astype(np.float64)


def test_noalloc_equals_workspace_entry_point():
    cases = [
        # the persistent path (Llama-3-8B-shaped heads), then smaller problems over the same scratch
        dict(seed=101, B=6, Hq=32, Hkv=8, lens=[1500, 333, 4000, 2, 0, 129], kw={}),
        dict(seed=102, B=3, Hq=16, Hkv=4, lens=[900, 300, 50], kw={}),
        dict(seed=103, B=2, Hq=12, Hkv=2, lens=[2700, 20], kw=dict(window=1000, num_sinks=4)),
        dict(seed=104, B=2, Hq=8, Hkv=2, lens=[500, 64], kw=dict(split_tokens=64)),
    ]
    for cs in cases:
        log(f"noalloc case seed={cs['seed']} B={cs['B']} lens={cs['lens']} {cs['kw']}")
        c = make_case(cs["seed"], B=cs["B"], Hq=cs["Hq"], Hkv=cs["Hkv"], d=128, dtype="bf16", P=16, lens=cs["lens"])
        (ow, lw), (on, ln), n_ws = _both(c, **cs["kw"])
        log(f"    workspace {n_ws} bytes")
        assert torch.equal(ow, on) and torch.equal(lw, ln), "no-allocation result differs from the workspace call"
        okw = dict(window=cs["kw"]["window"], sinks=cs["kw"]["num_sinks"]) if "window" in cs["kw"] else {}
        assert_close(c, (_np(on), _np(ln)), oracle_attend(c, **okw), f"noalloc seed {cs['seed']}")


def test_noalloc_score_export():
    """Score export through the scratch (the logits live there too), twice in a row, the second
    call smaller."""
    for seed, B, lens in ((111, 4, [3000, 1200, 17, 2049]), (112, 2, [900, 90])):
        c = make_case(seed, B=B, Hq=32, Hkv=8, d=128, dtype="bf16", P=16, lens=lens)
        stride = max(lens)
        init = synth.normal((B, 8, stride), seed, "score-init", dtype="f32").cuda()
        s_w, s_n = init.clone(), init.clone()
        (ow, lw), (on, ln), _ = _both(c, scores=s_w, scores_na=s_n)
        assert torch.equal(ow, on) and torch.equal(lw, ln)
        assert torch.equal(s_w, s_n), "scores differ between the two entry points"
        ref = oracle.decode_scores(c.dtype, c.kpool, synth.raw_numpy(c.q), c.bt.numpy(), np.array(lens, np.int32),
                                   P=16, Hkv=8, d=128, stride=stride, score=init.cpu().double().numpy())
        err = float(np.abs(s_n.cpu().double().numpy() - ref).max())
        log(f"    noalloc scores seed {seed}: max|score err| = {err:.3e}")
        assert err <= 1e-5


def test_noalloc_refuses_beyond_scratch():
    """Score export over 64 sequences of 30000 tokens needs 245 MB of logits: refused with
    PKV_ERR_SCRATCH before anything is enqueued (outputs untouched)."""
    import paged_kv_cache_16_amd as pkv
    B, Hq, Hkv, d = 64, 32, 8, 128
    k = torch.zeros((1, Hkv, 16, d), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    cl = torch.zeros((B,), dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, Hkv, 30000), dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, d), 7.0, dtype=torch.float32, device="cuda")
    need = pkv.workspace_size(k, B, Hq, 30000, scores=True)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_decode_attention_noalloc(q, k, k, bt, cl, max_context_len=30000, out=out, scores=sc)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
