"""GPU parity of page selection ([OVAL] §3.3: the next step keeps the k pages of largest
weight, the newest pages always) and of page-granular score export, through the C ABI.

Selection decides integers from fp32 weights, so both sides sum the weights in the same
precision and order (fp32, heads in index order) and the page lists must match exactly.
Page-granular scores are compared like token scores (1e-5 absolute per entry: an entry sums
at most 8 heads x 32 tokens of probabilities whose sum is at most 8, each term with a
relative error of a few 1e-7)."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from harness import assert_close, log, make_case, oracle_attend

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
SCORE_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _gpu_select(sc, lens, P, k, recent):
    import paged_kv_cache_16_amd as pkv
    out = pkv.select_pages(torch.as_tensor(sc, dtype=torch.float32).cuda().contiguous(),
                           torch.as_tensor(np.asarray(lens), dtype=torch.int32).cuda(), block_size=P, k=k,
                           recent=recent)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_select_golden_cases():
    with open(os.path.join(GOLDEN, "page_select.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = _gpu_select(np.array(c["scores"], np.float32), c["lens"], c["P"], c["k"], c["recent"])
        assert got.tolist() == c["expect"], (c["what"], got.tolist())


@pytest.mark.parametrize("seed", range(6))
def test_select_random_with_ties(seed):
    rng = np.random.default_rng(400 + seed)
    B, H, P = 7, int(rng.integers(1, 9)), int(rng.choice([16, 32]))
    k = int(rng.integers(1, 65))
    recent = int(rng.integers(0, min(k, 4) + 1))
    lens = rng.integers(0, 300 * P, size=B)
    lens[0] = 0
    stride = int((lens.max() + P - 1) // P) + 3
    coarse = seed % 2 == 0  # half the cases: few distinct values, so many ties
    sc = (rng.integers(0, 5, size=(B, H, stride)) * 0.25 if coarse else rng.random((B, H, stride))).astype(np.float32)
    got = _gpu_select(sc, lens, P, k, recent)
    ref = oracle.select_pages(sc, lens, P=P, k=k, recent=recent)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("shape", [dict(B=16, H=32, P=32, L=32768, k=16), dict(B=8, H=8, P=16, L=30000, k=64),
                                   dict(B=2, H=2, P=16, L=15360 * 16, k=32)], ids=["pagesel", "kvsparse", "max-pages"])
def test_select_full_size(shape):
    """The page-selected workload's shape (1024 pages, 32 heads), a 30k context, and the
    largest page count the kernel takes."""
    B, H, P, L, k = shape["B"], shape["H"], shape["P"], shape["L"], shape["k"]
    n = (L + P - 1) // P
    sc = synth.normal((B, H, n), 401, "page-scores", dtype="f32").abs().numpy()
    lens = np.full(B, L, np.int32)
    got = _gpu_select(sc, lens, P, k, 1)
    ref = oracle.select_pages(sc, lens, P=P, k=k, recent=1)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("case", ["stride-not-multiple-of-4", "staged-in-chunks", "unaligned-base", "one-head"])
def test_select_load_paths(case):
    """Both ways of reading the weights give the oracle's lists: rows staged in LDS with
    16-byte loads (stride a multiple of 4, 16-byte aligned array; in several chunks when the
    heads' rows exceed the LDS), and 4-byte loads otherwise."""
    import paged_kv_cache_16_amd as pkv
    rng = np.random.default_rng(410 + len(case))
    B, P, k = 5, 16, 24
    H = {"staged-in-chunks": 64, "one-head": 1}.get(case, 8)
    lens = rng.integers(1, 1500 * P, size=B)
    n = int((lens.max() + P - 1) // P)
    stride = n + (-n) % 4 + (1 if case == "stride-not-multiple-of-4" else 0)
    assert (stride % 4 != 0) == (case == "stride-not-multiple-of-4")
    sc = (rng.integers(0, 7, size=(B, H, stride)) * 0.5).astype(np.float32)  # many ties
    ref = oracle.select_pages(sc, lens, P=P, k=k, recent=2)
    if case == "unaligned-base":
        flat = torch.zeros(B * H * stride + 1, dtype=torch.float32, device="cuda")
        flat[1:] = torch.as_tensor(sc).reshape(-1).cuda()
        g = flat[1:].view(B, H, stride)
        assert g.data_ptr() % 16 != 0
    else:
        g = torch.as_tensor(sc).cuda().contiguous()
    out = pkv.select_pages(g, torch.as_tensor(lens.astype(np.int32)).cuda(), block_size=P, k=k, recent=2)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("block", [16, 32, 5])
def test_score_export_per_page(block):
    import paged_kv_cache_16_amd as pkv
    lens = [1000, 333, 0, 47]
    c = make_case(72, B=4, Hq=8, Hkv=4, d=128, dtype="bf16", P=16, lens=lens)
    pl = synth.page_lists(lens, c.P, 5, 72).numpy()
    for kw, okw in ((dict(), dict()), (dict(window=200, num_sinks=4), dict(window=200, sinks=4)),
                    (dict(page_list=torch.as_tensor(pl).cuda()), dict(page_list=pl))):
        n = (max(lens) + block - 1) // block
        init = synth.normal((4, 4, n), 72, "init", block, dtype="f32")
        gs = init.clone().cuda()
        pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens), scores=gs,
                                   score_block=block, **kw)
        torch.cuda.synchronize()
        ref = oracle.decode_scores(c.dtype, c.kpool, synth.raw_numpy(c.q), c.bt.numpy(), np.array(lens, np.int32),
                                   P=c.P, Hkv=c.Hkv, d=c.d, stride=n, score=init.double().numpy(), block=block, **okw)
        err = float(np.abs(gs.cpu().double().numpy() - ref).max())
        log(f"    block {block} {okw.keys()}: max|score err| = {err:.3e}")
        assert err <= SCORE_TOL


def test_select_loop_closes():
    """Scores of one decode step (per page) choose the next step's pages; that list drives
    attention. The GPU's selection equals the oracle's on the same score array, and the
    attention over the chosen pages matches the oracle."""
    import paged_kv_cache_16_amd as pkv
    lens = [2000, 700, 64]
    P, k = 32, 6
    c = make_case(73, B=3, Hq=8, Hkv=8, d=128, dtype="f16", P=P, lens=lens)
    n = (max(lens) + P - 1) // P
    gs = torch.zeros((3, 8, n), dtype=torch.float32, device="cuda")
    pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens), scores=gs, score_block=P)
    pl = pkv.select_pages(gs, c.gcl, block_size=P, k=k, recent=1)
    out, lse = pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens), page_list=pl)
    torch.cuda.synchronize()
    ref_pl = oracle.select_pages(gs.cpu().numpy(), lens, P=P, k=k, recent=1)
    assert np.array_equal(pl.cpu().numpy(), ref_pl)
    got = (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    assert_close(c, got, oracle_attend(c, page_list=ref_pl), "selected pages")
