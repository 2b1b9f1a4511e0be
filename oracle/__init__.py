"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (``paged_kv_cache_16_amd``)
never imports it, and it never imports the product path.

This module is argument marshalling around ``oracle.c`` (plain fp64 C, built with
gcc into ``liboracle.so``): numpy arrays in, numpy arrays out. Element types are
passed as raw bits: ``uint16`` arrays for bf16/fp16, ``float32`` for fp32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "i8bf16": 3, "i8f16": 4}
# INT8 caches: the pool is raw bytes (int8 data plane, then the fp32 scale plane); their
# inputs (q, appended rows) are of the named 16-bit type.
INPUT_DTYPE = {"i8bf16": "bf16", "i8f16": "f16"}


def pool_elems(nb, Hkv, P, d, dtype):
    """Length of a flat pool array (elements for float dtypes, bytes for INT8 ones)."""
    return nb * Hkv * P * (d + 4) if dtype in INPUT_DTYPE else nb * Hkv * P * d


def compile_oracle(src: str, so: str) -> str:
    """gcc -O2, no fast-math: the oracle's summation order stays as written."""
    tmp = so + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                    "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, so)
    return so


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO):
        compile_oracle(SOURCE, _SO)
    return _SO


class OracleError(RuntimeError):
    pass


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_D = ctypes.c_double


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _raw(a: np.ndarray, dtype: str) -> np.ndarray:
    """Input arrays (q, rows): raw bits of the input dtype."""
    dtype = INPUT_DTYPE.get(dtype, dtype)
    want = np.float32 if dtype == "f32" else np.uint16
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"{dtype} data must be passed as {np.dtype(want).name}, got {a.dtype}")
    return a


def _raw_pool(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype in INPUT_DTYPE:
        a = np.ascontiguousarray(a)
        if a.dtype != np.uint8:
            raise TypeError(f"{dtype} pools must be passed as uint8 bytes, got {a.dtype}")
        return a
    return _raw(a, dtype)


def _nb(pool, Hkv, P, d, dtype):
    return pool.size // (Hkv * P * (d + 4 if dtype in INPUT_DTYPE else d))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Oracle:
    """One loaded build of oracle.c (the default build, or a test's mutated copy)."""

    def __init__(self, so_path: str):
        L = ctypes.CDLL(so_path)
        L.oracle_k_index.restype = _I64
        L.oracle_k_index.argtypes = [_I64, _I, _I, _I, _I, _I, _I, _I]
        L.oracle_v_index.restype = _I64
        L.oracle_v_index.argtypes = [_I64, _I, _I, _I, _I, _I, _I, _I]
        L.oracle_kv_append.restype = _I
        L.oracle_kv_append.argtypes = [_I, _I64, _I, _I, _I, _P, _P, _P, _P, _P, _I64]
        L.oracle_decode_attention.restype = _I
        L.oracle_decode_attention.argtypes = [_I, _I64, _I, _I, _I, _P, _P, _P, _I, _I, _P, _I,
                                              _P, _D, _I, _I, _P, _I, _P, _P]
        L.oracle_decode_attention_split.restype = _I
        L.oracle_decode_attention_split.argtypes = [_I, _I64, _I, _I, _I, _P, _P, _P, _I, _I,
                                                    _P, _I, _P, _D, _I, _I, _P, _I, _I, _I, _P,
                                                    _P, _P, _P, _P]
        L.oracle_decode_scores.restype = _I
        L.oracle_decode_scores.argtypes = [_I, _I64, _I, _I, _I, _P, _P, _I, _I, _P, _I, _P, _D, _I,
                                           _I, _P, _I, _P, _I64, _I]
        L.oracle_select_pages.restype = _I
        L.oracle_select_pages.argtypes = [_P, _I, _I64, _P, _I, _I, _I, _I, _P]
        L.oracle_bruteforce.restype = _I
        L.oracle_bruteforce.argtypes = [_I, _P, _P, _I, _P, _I, _I, _I, _I, _P, _D, _I, _I, _I,
                                        _P, _I, _P, _P]
        L.oracle_quantise_rows.restype = _I
        L.oracle_quantise_rows.argtypes = [_P, _I, _I, _P, _P]
        L.oracle_ring_pages.restype = _I
        L.oracle_ring_pages.argtypes = [_I, _I]
        L.oracle_ring_column.restype = _I64
        L.oracle_ring_column.argtypes = [_I64, _I, _I, _I]
        L.oracle_ring_expand.restype = _I
        L.oracle_ring_expand.argtypes = [_P, _I, _I, _I, _I, _I, _I, _P]
        L.oracle_policy_blocks.restype = _I64
        L.oracle_policy_blocks.argtypes = [_I64, _I, _I, _I, _I]
        L.oracle_kv_cache_bytes.restype = ctypes.c_uint64
        L.oracle_kv_cache_bytes.argtypes = [_I64] * 7
        self.lib = L

    @staticmethod
    def _check(rc: int, what: str) -> None:
        if rc != 0:
            raise OracleError(f"{what}: oracle returned {rc}")

    def k_index(self, blk, h, t, x, Hkv, P, d, dtype) -> int:
        return int(self.lib.oracle_k_index(blk, h, t, x, Hkv, P, d, DTYPE_CODE[dtype]))

    def v_index(self, blk, h, t, x, Hkv, P, d, dtype) -> int:
        return int(self.lib.oracle_v_index(blk, h, t, x, Hkv, P, d, DTYPE_CODE[dtype]))

    def kv_append(self, dtype, kpool, vpool, k_new, v_new, slots, *, P, Hkv, d):
        """Writes k_new/v_new ([N][Hkv][d] raw) into the flat raw pools, in place."""
        for a in (kpool, vpool):
            if not (isinstance(a, np.ndarray) and a.flags.c_contiguous):
                raise TypeError("pools must be C-contiguous numpy arrays (written in place)")
        kpool, vpool = _raw_pool(kpool, dtype), _raw_pool(vpool, dtype)
        k_new, v_new = _raw(k_new, dtype), _raw(v_new, dtype)
        slots = _i32(slots)
        nb = _nb(kpool, Hkv, P, d, dtype)
        self._check(self.lib.oracle_kv_append(DTYPE_CODE[dtype], nb, P, Hkv, d, _ptr(kpool),
                                              _ptr(vpool), _ptr(k_new), _ptr(v_new),
                                              _ptr(slots), slots.size), "kv_append")
        return kpool, vpool

    def ring_pages(self, window, P) -> int:
        return int(self.lib.oracle_ring_pages(int(window), int(P)))

    def ring_column(self, page, *, sinks, P, ring_pages) -> int:
        return int(self.lib.oracle_ring_column(int(page), int(sinks), int(P), int(ring_pages)))

    def ring_expand(self, ring_table, *, sinks, P, ring_pages, pages):
        """[B][cols] ring rows -> [B][pages] plain rows (logical page j in column j)."""
        rt = _i32(ring_table)
        B, cols = rt.shape
        plain = np.full((B, pages), -1, np.int32)
        self._check(self.lib.oracle_ring_expand(_ptr(rt), B, cols, int(sinks), int(P), int(ring_pages),
                                                int(pages), _ptr(plain)), "ring_expand")
        return plain

    def policy_blocks(self, L, *, P, window, sinks=0, ring_pages=0) -> int:
        n = int(self.lib.oracle_policy_blocks(int(L), int(P), int(window), int(sinks), int(ring_pages)))
        if n < 0:
            raise OracleError("policy_blocks: bad arguments")
        return n

    def _plain_table(self, block_table, context_lens, P, sinks, ring_pages):
        """A ring table (ring_pages > 0) as the plain table that addresses the same blocks."""
        if not ring_pages:
            return block_table
        cl = _i32(context_lens).reshape(-1)
        pages = max(1, (int(cl.max(initial=0)) + P - 1) // P)
        return self.ring_expand(block_table, sinks=sinks, P=P, ring_pages=ring_pages, pages=pages)

    def _common(self, dtype, kpool, vpool, q, block_table, context_lens, P, Hkv, d, page_list):
        kpool, vpool, q = _raw_pool(kpool, dtype), _raw_pool(vpool, dtype), _raw(q, dtype)
        bt = _i32(block_table)
        cl = _i32(context_lens).reshape(-1)
        B = cl.size
        Hq = q.size // (B * d) if B else 1
        mb = bt.shape[1] if bt.ndim == 2 else 0
        pl = None if page_list is None else _i32(page_list)
        pps = 0 if pl is None else pl.shape[1]
        nb = _nb(kpool, Hkv, P, d, dtype)
        return kpool, vpool, q, bt, cl, B, Hq, mb, pl, pps, nb

    def decode_attention(self, dtype, kpool, vpool, q, block_table, context_lens, *, P, Hkv, d,
                         scale=0.0, window=0, sinks=0, page_list=None, ring_pages=0):
        """Returns (out [B][Hq][d] float64, lse [B][Hq] float64). ring_pages > 0: block_table
        is a window layer's ring table."""
        block_table = self._plain_table(block_table, context_lens, P, sinks, ring_pages)
        kpool, vpool, q, bt, cl, B, Hq, mb, pl, pps, nb = self._common(
            dtype, kpool, vpool, q, block_table, context_lens, P, Hkv, d, page_list)
        out = np.zeros((B, Hq, d), np.float64)
        lse = np.zeros((B, Hq), np.float64)
        self._check(self.lib.oracle_decode_attention(
            DTYPE_CODE[dtype], nb, P, Hkv, d, _ptr(kpool), _ptr(vpool), _ptr(q), B, Hq, _ptr(bt),
            mb, _ptr(cl), float(scale), int(window), int(sinks), _ptr(pl), pps, _ptr(out),
            _ptr(lse)), "decode_attention")
        return out, lse

    def decode_scores(self, dtype, kpool, q, block_table, context_lens, *, P, Hkv, d, stride,
                      scale=0.0, window=0, sinks=0, page_list=None, score=None, block=1, ring_pages=0):
        """Adds one step's scores into `score` ([B][Hkv][stride] float64, zeros when None) and
        returns it. block: tokens per score entry."""
        block_table = self._plain_table(block_table, context_lens, P, sinks, ring_pages)
        kpool, _, q, bt, cl, B, Hq, mb, pl, pps, nb = self._common(
            dtype, kpool, kpool, q, block_table, context_lens, P, Hkv, d, page_list)
        if score is None:
            score = np.zeros((B, Hkv, stride), np.float64)
        score = np.ascontiguousarray(score, dtype=np.float64)
        if score.shape != (B, Hkv, stride):
            raise ValueError(f"score must be [{B}][{Hkv}][{stride}], got {score.shape}")
        self._check(self.lib.oracle_decode_scores(
            DTYPE_CODE[dtype], nb, P, Hkv, d, _ptr(kpool), _ptr(q), B, Hq, _ptr(bt), mb, _ptr(cl),
            float(scale), int(window), int(sinks), _ptr(pl), pps, _ptr(score), int(stride), int(block)),
            "decode_scores")
        return score

    def select_pages(self, scores, context_lens, *, P, k, recent=1):
        """scores: [B][H][stride] float32 page weights. Returns the [B][k] int32 page lists."""
        sc = np.ascontiguousarray(scores, dtype=np.float32)
        if sc.ndim != 3:
            raise ValueError("scores must be [B][H][stride]")
        cl = _i32(context_lens).reshape(-1)
        B, H, stride = sc.shape
        out = np.full((B, k), -7, np.int32)
        self._check(self.lib.oracle_select_pages(_ptr(sc), H, stride, _ptr(cl), B, int(P), int(k), int(recent),
                                                 _ptr(out)), "select_pages")
        return out

    def decode_attention_split(self, dtype, kpool, vpool, q, block_table, context_lens, *, P,
                               Hkv, d, units, max_splits, scale=0.0, window=0, sinks=0,
                               page_list=None, ring_pages=0):
        """Returns (o_part, m_part, l_part, out, lse), all float64."""
        block_table = self._plain_table(block_table, context_lens, P, sinks, ring_pages)
        kpool, vpool, q, bt, cl, B, Hq, mb, pl, pps, nb = self._common(
            dtype, kpool, vpool, q, block_table, context_lens, P, Hkv, d, page_list)
        o_part = np.zeros((B, Hq, max_splits, d), np.float64)
        m_part = np.zeros((B, Hq, max_splits), np.float64)
        l_part = np.zeros((B, Hq, max_splits), np.float64)
        out = np.zeros((B, Hq, d), np.float64)
        lse = np.zeros((B, Hq), np.float64)
        self._check(self.lib.oracle_decode_attention_split(
            DTYPE_CODE[dtype], nb, P, Hkv, d, _ptr(kpool), _ptr(vpool), _ptr(q), B, Hq, _ptr(bt),
            mb, _ptr(cl), float(scale), int(window), int(sinks), _ptr(pl), pps, int(units),
            int(max_splits), _ptr(o_part), _ptr(m_part), _ptr(l_part), _ptr(out), _ptr(lse)),
            "decode_attention_split")
        return o_part, m_part, l_part, out, lse

    def bruteforce(self, dtype, K_log, V_log, q, context_lens, *, Hkv, d, scale=0.0, P=16,
                   window=0, sinks=0, page_list=None):
        """Contiguous-cache reference; K_log/V_log: [B][Lmax][Hkv][d] raw. Long doubles out."""
        K_log, V_log, q = _raw(K_log, dtype), _raw(V_log, dtype), _raw(q, dtype)
        cl = _i32(context_lens).reshape(-1)
        B = cl.size
        Lmax = K_log.shape[1]
        Hq = q.size // (B * d) if B else 1
        pl = None if page_list is None else _i32(page_list)
        pps = 0 if pl is None else pl.shape[1]
        out = np.zeros((B, Hq, d), np.longdouble)
        lse = np.zeros((B, Hq), np.longdouble)
        self._check(self.lib.oracle_bruteforce(
            DTYPE_CODE[dtype], _ptr(K_log), _ptr(V_log), Lmax, _ptr(q), B, Hq, Hkv, d, _ptr(cl),
            float(scale), int(P), int(window), int(sinks), _ptr(pl), pps, _ptr(out), _ptr(lse)),
            "bruteforce")
        return out, lse

    def quantise_rows(self, x):
        """x: [n][d] float32 rows -> (int8 [n][d], float32 scales [n])."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        n, d = x.shape
        q = np.zeros((n, d), np.int8)
        sc = np.zeros(n, np.float32)
        self._check(self.lib.oracle_quantise_rows(_ptr(x), n, d, _ptr(q), _ptr(sc)), "quantise_rows")
        return q, sc

    def kv_cache_bytes(self, batch, layers, heads, head_dim, seq_len, dtype_bytes,
                       block_size=0) -> int:
        return int(self.lib.oracle_kv_cache_bytes(batch, layers, heads, head_dim, seq_len,
                                                  dtype_bytes, block_size))


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(SOURCE):
            build(force=True)
        _default = Oracle(_SO)
    return _default


def k_index(*a, **k):
    return default().k_index(*a, **k)


def v_index(*a, **k):
    return default().v_index(*a, **k)


def kv_append(*a, **k):
    return default().kv_append(*a, **k)


def decode_attention(*a, **k):
    return default().decode_attention(*a, **k)


def decode_attention_split(*a, **k):
    return default().decode_attention_split(*a, **k)


def decode_scores(*a, **k):
    return default().decode_scores(*a, **k)


def select_pages(*a, **k):
    return default().select_pages(*a, **k)


def bruteforce(*a, **k):
    return default().bruteforce(*a, **k)


def quantise_rows(*a, **k):
    return default().quantise_rows(*a, **k)


def kv_cache_bytes(*a, **k):
    return default().kv_cache_bytes(*a, **k)


def ring_pages(*a, **k):
    return default().ring_pages(*a, **k)


def ring_column(*a, **k):
    return default().ring_column(*a, **k)


def ring_expand(*a, **k):
    return default().ring_expand(*a, **k)


def policy_blocks(*a, **k):
    return default().policy_blocks(*a, **k)
