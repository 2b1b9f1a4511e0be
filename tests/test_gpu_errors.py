"""The device error word: inputs whose device-side preconditions do not hold are skipped by the
kernels' own bounds checks (no access leaves the caller's buffers) and raise a PKV_DEV_* bit;
the other sequences' results stay exact; a clean run leaves the word at 0."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from harness import assert_close, gpu_attend, log, make_case, oracle_attend, raw_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import paged_kv_cache_16_amd as pkv
    pkv.device_errors(clear=True)


def _case():
    return make_case(90, B=3, Hq=8, Hkv=2, d=128, dtype="bf16", P=16, lens=[300, 200, 90])


def test_clean_run_sets_nothing():
    import paged_kv_cache_16_amd as pkv
    pkv.device_errors(clear=True)
    c = _case()
    for kw in (dict(), dict(split_tokens=64), dict(window=40, num_sinks=3)):
        gpu_attend(c, **kw)
    assert pkv.device_errors() == 0


@pytest.mark.parametrize("split", [0, 64])
def test_block_id_out_of_range(split):
    """An attended page of sequence 1 maps outside the pool: its unit is skipped and the bit is
    set; sequences 0 and 2 are exact."""
    import paged_kv_cache_16_amd as pkv
    log(f"bad block id, split_tokens={split}")
    c = _case()
    ref = oracle_attend(c)
    bt = c.bt.clone()
    bt[1, 3] = c.nb + 7
    c.gbt = bt.cuda()
    pkv.device_errors(clear=True)
    out, lse = gpu_attend(c, split_tokens=split)
    assert pkv.device_errors() & pkv.DEV_BLOCK_ID
    assert pkv.device_errors() == 0  # cleared by the read before
    keep = [0, 2]
    assert_close(c, (out[keep], lse[keep]), (ref[0][keep], ref[1][keep]), "untouched sequences")


@pytest.mark.parametrize("block", [1, 16], ids=["per-token", "per-page"])
@pytest.mark.parametrize("lens", [[300, 200, 90], [120, 100, 90]], ids=["work-split", "one-kernel"])
def test_block_id_out_of_range_with_scores(lens, block):
    """Score export while a unit of sequence 1 is skipped for an invalid block id (on the
    work-split path and on the one-kernel path): the skipped unit adds nothing (its entries keep
    their initial values), every score stays finite, and sequences 0 and 2 match the oracle."""
    import oracle
    import paged_kv_cache_16_amd as pkv
    log(f"bad block id with score export, lens={lens}, score_block={block}")
    c = make_case(92, B=3, Hq=8, Hkv=2, d=128, dtype="bf16", P=16, lens=lens)
    stride = (max(lens) + block - 1) // block
    init = synth.normal((c.B, c.Hkv, stride), 92, "score-init", dtype="f32")
    ref = oracle.decode_scores(c.dtype, c.kpool, synth.raw_numpy(c.q), c.bt.numpy(), np.array(lens, np.int32),
                               P=c.P, Hkv=c.Hkv, d=c.d, stride=stride, score=init.double().numpy(), block=block)
    bt = c.bt.clone()
    bt[1, 3] = c.nb + 7  # tokens 48..63 of sequence 1
    c.gbt = bt.cuda()
    sc = init.clone().cuda()
    pkv.device_errors(clear=True)
    pkv.paged_decode_attention(c.gq, c.gk, c.gv, c.gbt, c.gcl, max_context_len=max(lens), scores=sc,
                               score_block=block)
    got = sc.cpu().numpy().astype(np.float64)
    assert pkv.device_errors() & pkv.DEV_BLOCK_ID
    assert np.isfinite(got).all()
    lo, hi = 48 // block, (63 // block) + 1
    assert np.array_equal(got[1, :, lo:hi], init.numpy()[1, :, lo:hi].astype(np.float64))
    err = float(np.abs(got[[0, 2]] - ref[[0, 2]]).max())
    log(f"    untouched sequences: max|score err| = {err:.3e}")
    assert err <= 1e-5


def test_slot_out_of_range():
    """Append slots past the pool: nothing is written and the bit is set, also in the fused step."""
    import paged_kv_cache_16_amd as pkv
    c = _case()
    n_slots = c.nb * c.P
    before_k, before_v = raw_bytes(c.gk).copy(), raw_bytes(c.gv).copy()
    kn = synth.normal((2, 2, 128), 91, "kn", dtype="bf16").cuda()
    pkv.device_errors(clear=True)
    pkv.kv_cache_append(c.gk, c.gv, kn, kn, torch.tensor([n_slots, -1], dtype=torch.int32, device="cuda"))
    assert pkv.device_errors() == pkv.DEV_SLOT
    assert np.array_equal(raw_bytes(c.gk), before_k) and np.array_equal(raw_bytes(c.gv), before_v)
    # fused step: sequence 2's slot is past the pool; its new token is still attended from k_new
    kn3 = torch.stack([c.K[b, L - 1] for b, L in enumerate(c.lens)]).cuda()
    vn3 = torch.stack([c.V[b, L - 1] for b, L in enumerate(c.lens)]).cuda()
    slots = torch.tensor([synth.slot_of(c.bt, 0, 299, 16), synth.slot_of(c.bt, 1, 199, 16), n_slots + 3],
                         dtype=torch.int32, device="cuda")
    out, lse = pkv.paged_decode_append_attention(c.gq, c.gk, c.gv, kn3, vn3, slots, c.gbt, c.gcl,
                                                 max_context_len=300)
    torch.cuda.synchronize()
    assert pkv.device_errors() == pkv.DEV_SLOT
    got = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    assert_close(c, got, oracle_attend(c), "fused step with a skipped write")


def test_context_beyond_bound():
    """A context length above max_context_len is clamped and reported."""
    import paged_kv_cache_16_amd as pkv
    c = _case()
    pkv.device_errors(clear=True)
    gpu_attend(c, max_context_len=250)  # sequence 0 holds 300 tokens
    assert pkv.device_errors() & pkv.DEV_CONTEXT


def test_select_pages_beyond_stride():
    import paged_kv_cache_16_amd as pkv
    pkv.device_errors(clear=True)
    scores = torch.rand((2, 3, 10), dtype=torch.float32, device="cuda")
    cl = torch.tensor([16 * 10, 16 * 12], dtype=torch.int32, device="cuda")  # sequence 1: 12 pages > 10
    pkv.select_pages(scores, cl, block_size=16, k=4)
    assert pkv.device_errors() == pkv.DEV_PAGES


def test_read_probe():
    """The read-rate probe reads whole 8 KiB steps per wave, never past the buffer, and rejects a
    short sink or too small a buffer before launching."""
    import paged_kv_cache_16_amd as pkv
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.zeros((64 << 20) + 4096, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(cus * 4 * 2, dtype=torch.int32, device="cuda")
    n = pkv.read_probe(buf, 2, sink)
    torch.cuda.synchronize()
    waves = cus * 4 * 2
    assert n == (buf.numel() // waves) // 8192 * 8192 * waves and 0 < n <= buf.numel()
    assert int(sink.abs().sum()) == 0  # zero data never matches the sink pattern
    with pytest.raises(pkv.PagedKVError):
        pkv.read_probe(buf, 4, sink)  # sink shorter than the waves
    with pytest.raises(pkv.PagedKVError):
        pkv.read_probe(buf[: waves * 8192 - 1], 2, sink)  # under 8 KiB per wave
    with pytest.raises(pkv.PagedKVError):
        pkv.read_probe(buf, 0, sink)
