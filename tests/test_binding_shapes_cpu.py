"""CPU tests: the Python binding checks every tensor it hands to the C ABI against the sizes
it passes with it, and raises ValueError before anything is enqueued. The C ABI only sees raw
pointers, so a tensor smaller than the call implies would otherwise be read or written past
its end by the kernels. These tests use CPU tensors: a check that passes leads on to the
device-tensor check ("must be a CUDA (HIP) tensor"), so a well-shaped call is told apart from a
mis-shaped one by the message, and no kernel can run."""
from __future__ import annotations

import pytest
import torch

import paged_kv_cache_16_amd as pkv

B, Hq, Hkv, d, P, NB = 3, 8, 2, 128, 16, 20
NOT_DEVICE = "must be a CUDA"


def _args(**over):
    a = dict(
        q=torch.zeros((B, Hq, d), dtype=torch.bfloat16),
        k_cache=torch.zeros((NB, Hkv, P, d), dtype=torch.bfloat16),
        v_cache=torch.zeros((NB, Hkv, P, d), dtype=torch.bfloat16),
        block_table=torch.zeros((B, 4), dtype=torch.int32),
        context_lens=torch.zeros((B,), dtype=torch.int32),
    )
    a.update(over)
    return a


def _decode(**over):
    a = _args(**{k: v for k, v in over.items() if k in ("q", "k_cache", "v_cache", "block_table", "context_lens")})
    kw = {k: v for k, v in over.items() if k not in a}
    return pkv.paged_decode_attention(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["context_lens"],
                                      max_context_len=64, **kw)


def _fused(**over):
    a = _args(**{k: v for k, v in over.items() if k in ("q", "k_cache", "v_cache", "block_table", "context_lens")})
    k_new = over.pop("k_new", torch.zeros((B, Hkv, d), dtype=torch.bfloat16))
    v_new = over.pop("v_new", torch.zeros((B, Hkv, d), dtype=torch.bfloat16))
    slots = over.pop("slot_mapping", torch.zeros((B,), dtype=torch.int32))
    kw = {k: v for k, v in over.items() if k not in a}
    return pkv.paged_decode_append_attention(a["q"], a["k_cache"], a["v_cache"], k_new, v_new, slots,
                                             a["block_table"], a["context_lens"], max_context_len=64, **kw)


def test_well_shaped_calls_reach_the_device_check():
    with pytest.raises(ValueError, match=NOT_DEVICE):
        _decode()
    with pytest.raises(ValueError, match=NOT_DEVICE):
        _fused()
    with pytest.raises(ValueError, match=NOT_DEVICE):
        _decode(page_list=torch.zeros((B, 2), dtype=torch.int32),
                out=torch.zeros((B, Hq, d)), lse=torch.zeros((B, Hq)),
                scores=torch.zeros((B, Hkv, 64)))
    with pytest.raises(ValueError, match=NOT_DEVICE):  # extra rows are allowed (never read)
        _decode(block_table=torch.zeros((B + 2, 4), dtype=torch.int32),
                context_lens=torch.zeros((B + 1,), dtype=torch.int32))


@pytest.mark.parametrize("over,what", [
    (dict(q=torch.zeros((B, Hq, 64), dtype=torch.bfloat16)), "head_dim"),
    (dict(q=torch.zeros((B, Hq * d), dtype=torch.bfloat16)), "q must be"),
    (dict(v_cache=torch.zeros((NB - 1, Hkv, P, d), dtype=torch.bfloat16)), "must match"),
    (dict(v_cache=torch.zeros((NB, Hkv, P, d), dtype=torch.float16)), "must match"),
    (dict(block_table=torch.zeros((B - 1, 4), dtype=torch.int32)), "block_table"),
    (dict(block_table=torch.zeros((B * 4,), dtype=torch.int32)), "block_table"),
    (dict(context_lens=torch.zeros((B - 1,), dtype=torch.int32)), "context_lens"),
    (dict(page_list=torch.zeros((B - 1, 2), dtype=torch.int32)), "page_list"),
    (dict(page_list=torch.zeros((B,), dtype=torch.int32)), "page_list"),
    (dict(out=torch.zeros((B, Hq, d - 1))), "out"),
    (dict(out=torch.zeros((B - 1, Hq, d))), "out"),
    (dict(lse=torch.zeros((B, Hq - 1))), "lse"),
    (dict(scores=torch.zeros((B, Hkv + 1, 64))), "scores"),
    (dict(scores=torch.zeros((B - 1, Hkv, 64))), "scores"),
])
def test_decode_rejects_mis_shaped_tensors(over, what):
    with pytest.raises(ValueError, match=what) as e:
        _decode(**over)
    assert NOT_DEVICE not in str(e.value)
    with pytest.raises(ValueError, match=what) as e:
        _fused(**over)
    assert NOT_DEVICE not in str(e.value)


@pytest.mark.parametrize("over,what", [
    (dict(k_new=torch.zeros((B - 1, Hkv, d), dtype=torch.bfloat16)), "k_new"),
    (dict(k_new=torch.zeros((B, Hkv + 1, d), dtype=torch.bfloat16)), "k_new"),
    (dict(v_new=torch.zeros((B, Hkv, d - 8), dtype=torch.bfloat16)), "v_new"),
    (dict(slot_mapping=torch.zeros((B + 1,), dtype=torch.int32)), "slot_mapping"),
    (dict(slot_mapping=torch.zeros((B, 1), dtype=torch.int32)), "slot_mapping"),
])
def test_fused_step_rejects_mis_shaped_new_rows(over, what):
    with pytest.raises(ValueError, match=what) as e:
        _fused(**over)
    assert NOT_DEVICE not in str(e.value)


def test_append_rejects_mis_shaped_rows():
    a = _args()
    slots = torch.zeros((5,), dtype=torch.int32)
    rows = torch.zeros((5, Hkv, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=NOT_DEVICE):
        pkv.kv_cache_append(a["k_cache"], a["v_cache"], rows, rows, slots)
    for k_new, v_new, what in ((rows[:4], rows, "k_new"), (rows, rows[:, :1], "v_new"),
                               (torch.zeros((5, Hkv, 64), dtype=torch.bfloat16), rows, "k_new")):
        with pytest.raises(ValueError, match=what):
            pkv.kv_cache_append(a["k_cache"], a["v_cache"], k_new, v_new, slots)
    with pytest.raises(ValueError, match="must match"):
        pkv.kv_cache_append(a["k_cache"], a["v_cache"][:1], rows, rows, slots)


def test_partial_and_combine_reject_mis_shaped_partials():
    a = _args()
    S = pkv.num_splits(a["k_cache"], B, 64, split_tokens=16)
    assert S == 4
    good = dict(o_part=torch.zeros((B, Hq, S, d)), m_part=torch.zeros((B, Hq, S)), l_part=torch.zeros((B, Hq, S)))
    with pytest.raises(ValueError, match=NOT_DEVICE):
        pkv.paged_decode_attention_partial(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["context_lens"],
                                           max_context_len=64, split_tokens=16, **good)
    for name, bad in (("o_part", torch.zeros((B, Hq, S - 1, d))), ("m_part", torch.zeros((B, Hq, S + 1))),
                      ("l_part", torch.zeros((B, Hq)))):
        with pytest.raises(ValueError, match=name):
            pkv.paged_decode_attention_partial(a["q"], a["k_cache"], a["v_cache"], a["block_table"],
                                               a["context_lens"], max_context_len=64, split_tokens=16,
                                               **dict(good, **{name: bad}))
    with pytest.raises(ValueError, match=NOT_DEVICE):
        pkv.paged_decode_combine(**good)
    for name, bad in (("m_part", torch.zeros((B, Hq, S - 1))), ("l_part", torch.zeros((B, Hq + 1, S)))):
        with pytest.raises(ValueError, match=name):
            pkv.paged_decode_combine(**dict(good, **{name: bad}))
    with pytest.raises(ValueError, match="out"):
        pkv.paged_decode_combine(**good, out=torch.zeros((B, Hq, d // 2)))
    with pytest.raises(ValueError, match="lse"):
        pkv.paged_decode_combine(**good, lse=torch.zeros((B * Hq,)))


def test_select_pages_rejects_mis_shaped_tensors():
    scores = torch.zeros((B, Hkv, 30))
    cl = torch.zeros((B,), dtype=torch.int32)
    with pytest.raises(ValueError, match=NOT_DEVICE):
        pkv.select_pages(scores, cl, block_size=16, k=4)
    with pytest.raises(ValueError, match="context_lens"):
        pkv.select_pages(scores, cl[:2], block_size=16, k=4)
    with pytest.raises(ValueError, match="page_list"):
        pkv.select_pages(scores, cl, block_size=16, k=4, page_list=torch.zeros((B, 3), dtype=torch.int32))
    with pytest.raises(ValueError, match="page_list"):
        pkv.select_pages(scores, cl, block_size=16, k=4, page_list=torch.zeros((B - 1, 4), dtype=torch.int32))
