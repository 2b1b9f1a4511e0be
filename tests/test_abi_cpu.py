"""CPU checks of the C ABI: the library loads, exports every function include/pagedkv.h
declares, and its host-only paths (validation, sizing, accounting) behave as documented.
Nothing here launches a kernel."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:pkv_status|size_t|int32_t|int64_t|uint64_t|void|const char\s*\*)\s+(\w+)\s*\(",
                       text, flags=re.M)
    return names


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_16_amd as m
    return m


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("kv_cache_append", "paged_decode_attention", "paged_decode_attention_workspace_size",
                 "paged_decode_attention_partial", "paged_decode_combine", "pkv_status_string",
                 "pkv_kv_cache_bytes", "paged_decode_attention_num_splits", "paged_select_pages",
                 "pkv_ring_pages", "pkv_policy_blocks", "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_append",
                 "pkv_bm_release", "pkv_bm_block_tables", "pkv_bm_blocks_in_use"):
        assert must in names


def test_library_exports_every_declared_symbol(pkv):
    lib = ctypes.CDLL(pkv.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(pkv):
    for s in range(8):
        assert pkv.status_string(s) and pkv.status_string(s) != "unknown status"
    assert pkv.status_string(99) == "unknown status"


def test_kv_cache_bytes_worked_values(pkv):
    with open(os.path.join(ROOT, "tests", "golden", "kv_cache_bytes.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert pkv.kv_cache_bytes(c["batch"], c["layers"], c["heads"], c["head_dim"], c["seq_len"],
                                  c["dtype_bytes"]) == c["bytes"]
    assert pkv.kv_cache_bytes(1, 1, 8, 128, 4001, 2, 16) == 2 * 8 * 128 * 4016 * 2


def _desc(pkv, nb=64, P=16, hkv=8, d=128, dt=2):
    return pkv.CacheDesc(nb, P, hkv, d, dt)


def test_workspace_and_split_queries(pkv):
    lib = pkv._lib
    d = _desc(pkv)
    o = pkv.DecodeOpts(0, 0, None, 0, 256)
    # 4096 tokens in 256-token partitions -> 16 partitions; workspace holds o, m, l for each
    assert lib.paged_decode_attention_num_splits(ctypes.byref(d), 32, 4096, ctypes.byref(o)) == 16
    ws = lib.paged_decode_attention_workspace_size(ctypes.byref(d), 32, 32, 4096, ctypes.byref(o))
    rows = 32 * 32 * 16
    assert ws >= rows * (128 + 2) * 4
    # a single partition needs no workspace
    o1 = pkv.DecodeOpts(0, 0, None, 0, 4096)
    assert lib.paged_decode_attention_workspace_size(ctypes.byref(d), 32, 32, 4096, ctypes.byref(o1)) == 0
    # window mode bounds the partitions by the window, not the context
    ow = pkv.DecodeOpts(512, 4, None, 0, 64)
    assert lib.paged_decode_attention_num_splits(ctypes.byref(d), 8, 30000, ctypes.byref(ow)) <= 9
    # rejected arguments give 0
    bad = _desc(pkv, d=96)
    assert lib.paged_decode_attention_workspace_size(ctypes.byref(bad), 1, 8, 10, None) == 0


def test_validation_precedes_any_launch(pkv):
    lib = pkv._lib
    d = _desc(pkv)
    # NULL descriptor
    assert lib.kv_cache_append(None, None, None, None, None, None, 1, None) == 1
    # zero tokens is a no-op even with NULL buffers
    assert lib.kv_cache_append(ctypes.byref(d), None, None, None, None, None, 0, None) == 0
    # missing buffers
    assert lib.kv_cache_append(ctypes.byref(d), None, None, None, None, None, 4, None) == 1
    # unsupported head_dim / block size
    assert lib.kv_cache_append(ctypes.byref(_desc(pkv, d=96)), None, None, None, None, None, 4, None) == 3
    assert lib.kv_cache_append(ctypes.byref(_desc(pkv, P=24)), None, None, None, None, None, 4, None) == 3
    call = lib.paged_decode_attention
    fake = ctypes.c_void_p(256)  # never dereferenced: every case below fails validation first
    args = lambda hq=32, opts=None, out=fake, mcl=100, batch=2, ws=None, wsn=0: (
        ctypes.byref(d), fake, fake, fake, fake, 8, fake, batch, hq, mcl, 0.0, opts, out, 2, None, ws, wsn, None)
    assert call(*args(hq=30)) == 2                      # Hq % Hkv != 0
    assert call(*args(hq=8 * 9)) == 3                   # group of 9 > 8
    both = pkv.DecodeOpts(16, 0, fake, 4, 0)
    assert call(*args(opts=ctypes.byref(both))) == 4    # window and page list together
    assert call(*args(out=None)) == 1                   # no output
    assert call(*args(batch=0)) == 0                    # empty batch: nothing to do
    many = pkv.DecodeOpts(0, 0, None, 0, 64)
    assert call(*args(opts=ctypes.byref(many), mcl=4096)) == 5   # needs a workspace, none given
    assert lib.paged_decode_combine(None, None, None, 2, 4, 3, 128, None, 0, None, None) == 1
    assert lib.paged_decode_combine(fake, fake, fake, 2, 4, 0, 128, fake, 0, None, None) == 2


def test_score_export_validation(pkv):
    """Score export: sizing grows by the logits buffer; invalid combinations are rejected on
    the host before anything is enqueued."""
    lib = pkv._lib
    d = _desc(pkv)
    fake = ctypes.c_void_p(256)  # never dereferenced
    plain = pkv.DecodeOpts(0, 0, None, 0, 0)
    scored = pkv.DecodeOpts(0, 0, None, 0, 0, fake, 4096)
    ws0 = lib.paged_decode_attention_workspace_size(ctypes.byref(d), 32, 32, 4096, ctypes.byref(plain))
    ws1 = lib.paged_decode_attention_workspace_size(ctypes.byref(d), 32, 32, 4096, ctypes.byref(scored))
    # logits of every unit and head: 32 seq x 8 kv heads x 256 units x 4 heads x 16 tokens x 4 B
    assert ws1 - ws0 >= 32 * 8 * 256 * 4 * 16 * 4
    # the one-kernel path exports scores itself, so a tiny problem still needs no workspace ...
    assert lib.paged_decode_attention_workspace_size(ctypes.byref(d), 2, 32, 20, ctypes.byref(plain)) == 0
    small = pkv.DecodeOpts(0, 0, None, 0, 0, fake, 20)
    assert lib.paged_decode_attention_workspace_size(ctypes.byref(d), 2, 32, 20, ctypes.byref(small)) == 0
    # ... except over a page list with entries other than single tokens or whole pages
    odd = pkv.DecodeOpts(0, 0, fake, 2, 0, fake, 20, 5)
    assert lib.paged_decode_attention_workspace_size(ctypes.byref(d), 2, 32, 20, ctypes.byref(odd)) > 0
    per_page = pkv.DecodeOpts(0, 0, fake, 2, 0, fake, 20, d.block_size)
    assert lib.paged_decode_attention_workspace_size(ctypes.byref(d), 2, 32, 20, ctypes.byref(per_page)) == 0
    call = lib.paged_decode_attention
    args = lambda opts, mcl=100: (ctypes.byref(d), fake, fake, fake, fake, 8, fake, 2, 32, mcl, 0.0, opts, fake, 2,
                                  None, None, 0, None)
    split = pkv.DecodeOpts(0, 0, None, 0, 64, fake, 4096)
    assert call(*args(ctypes.byref(split))) == 4        # scores with fixed partitions
    short = pkv.DecodeOpts(0, 0, None, 0, 0, fake, 99)
    assert call(*args(ctypes.byref(short))) == 2        # stride below the context bound
    part = lib.paged_decode_attention_partial
    assert part(ctypes.byref(d), fake, fake, fake, fake, 8, fake, 2, 32, 100, 0.0, ctypes.byref(scored),
                fake, fake, fake, 1, None) == 4         # the partial call exports no scores


def test_device_errors_validation(pkv):
    # a missing output pointer is rejected before any device call
    assert pkv._lib.pkv_device_errors(None, 1, None) == 1


def test_select_pages_validation(pkv):
    """paged_select_pages rejects bad shapes and limits on the host (no launch)."""
    sel = pkv._lib.paged_select_pages
    fake = ctypes.c_void_p(256)  # never dereferenced
    assert sel(fake, 4, 100, fake, 2, 16, 65, 1, fake, None) == 3      # k above 64
    assert sel(fake, 4, 100, fake, 2, 16, 4, 5, fake, None) == 2       # recent above k
    assert sel(fake, 4, 15361, fake, 2, 16, 4, 1, fake, None) == 3     # pages beyond the LDS table
    assert sel(fake, 0, 100, fake, 2, 16, 4, 1, fake, None) == 2       # no heads
    assert sel(None, 4, 100, fake, 2, 16, 4, 1, fake, None) == 1       # missing scores
    assert sel(None, 4, 100, None, 0, 16, 4, 1, None, None) == 0       # empty batch
    d = _desc(pkv)
    call = pkv._lib.paged_decode_attention
    args = lambda opts: (ctypes.byref(d), fake, fake, fake, fake, 8, fake, 2, 32, 100, 0.0, opts, fake, 2,
                         None, None, 0, None)
    # per-page entries: 100 tokens in pages of 16 need 7 entries
    assert call(*args(ctypes.byref(pkv.DecodeOpts(0, 0, None, 0, 0, fake, 6, 16)))) == 2
    assert call(*args(ctypes.byref(pkv.DecodeOpts(0, 0, None, 0, 0, fake, 7, -2)))) == 2
