// pkv_device.h — device-side building blocks of the gfx950 paged decode-attention kernels.
//
// Element types, 16-byte chunk loads, the matrix-core (MFMA) tile products and the
// cache-layout arithmetic shared by the append and attention kernels of this library.
//
// Lane conventions (wave64). Lane l is written (j, c) with j = l / 16 and c = l % 16.
// The 16x16 MFMA shapes used here hand lane (j, c) row/column c of each operand and
// rows 4j..4j+3 of column c of the 16x16 fp32 result. The decode kernel computes
//   S^T = K . Q^T   (A = a 16-token sub-tile of K, B = Q^T, query heads in the columns)
// so lane (j, c) ends up holding the logits of column c's head for tokens 4j..4j+3, and
//   O^T += V^T . P^T (A = V^T straight from the loaded chunk, B = P^T built in place from
// the lane's own logits), so P never moves between lanes. Every value a lane needs from the
// cache is one 16-byte chunk at index (chunk group) * 64 + l of the sub-tile, by
// construction of the cache layout (see include/pagedkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// dtype tags -----------------------------------------------------------------------------
// kBytes / kE: bytes and elements of one cache element / 16-byte chunk. In: the type of q
// (and of the new rows and 2-byte outputs). Mma: the type of the MFMA operands. kQ8: an INT8
// cache (int8 data plane + fp32 row-scale plane).
struct F32 {
    static constexpr int kBytes = 4;
    static constexpr int kE = 4;  // elements per 16-byte chunk
    static constexpr bool kQ8 = false;
    using In = F32;
    using Mma = F32;
};
struct F16 {
    static constexpr int kBytes = 2;
    static constexpr int kE = 8;
    static constexpr bool kQ8 = false;
    using In = F16;
    using Mma = F16;
};
struct BF16 {
    static constexpr int kBytes = 2;
    static constexpr int kE = 8;
    static constexpr bool kQ8 = false;
    using In = BF16;
    using Mma = BF16;
};
// INT8 caches with bf16 / fp16 inputs. A 16-byte chunk holds 16 elements; widened, it is
// exactly two fp16 chunks (int8 values are exact in fp16), and the MFMAs run in fp16 for either
// input type: a bf16 query is converted once per run (exact for |q| in [2^-14, 65504], the
// bf16 values fp16 holds; smaller ones round toward zero by less than 2^-24).
struct I8B {
    static constexpr int kBytes = 1;
    static constexpr int kE = 16;
    static constexpr bool kQ8 = true;
    using In = BF16;
    using Mma = F16;
};
struct I8H {
    static constexpr int kBytes = 1;
    static constexpr int kE = 16;
    static constexpr bool kQ8 = true;
    using In = F16;
    using Mma = F16;
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 16 int8 values -> two chunks of 8 fp16 (elements 0..7, 8..15) holding x + kI8Bias, exact.
// A byte x becomes k = x + 128 (its sign bit flipped); the fp16 with bits 0x6400 | k is
// 1024 + k = x + 1152 (exponent 10, unit spacing): one byte permute builds two such halves.
// The constant offset is taken out after the products, once per head (attention subtracts
// kI8Bias * sum(q) from each logit and kI8Bias * sum(p) from each output element).
constexpr float kI8Bias = 1152.0f;
__device__ __forceinline__ void widen_i8_f16_biased(const u32x4& c, u32x4& lo, u32x4& hi) {
    unsigned o[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const unsigned k = c[w] ^ 0x80808080u;
        // result bytes: selector 0..3 take bytes of k, 4 takes a 0x64 byte
        o[2 * w] = __builtin_amdgcn_perm(0x64646464u, k, 0x04010400u);      // halves 0x64k0, 0x64k1
        o[2 * w + 1] = __builtin_amdgcn_perm(0x64646464u, k, 0x04030402u);  // halves 0x64k2, 0x64k3
    }
    lo = u32x4{o[0], o[1], o[2], o[3]};
    hi = u32x4{o[4], o[5], o[6], o[7]};
}

// Two bf16 values (one dword) -> two fp16 values (one dword), rounding toward zero: exact for
// the bf16 values fp16 holds.
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned w) {
    const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Streaming load for data read exactly once (K/V tiles): the nontemporal hint keeps the
// line from being allocated for reuse, which lifts sustained HBM read bandwidth.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Buffer-resource loads for cache tiles. The wave-uniform tile base sits in scalar registers
// and each lane adds a fixed 32-bit offset, so loading a tile forms no per-lane 64-bit
// address: with global loads the compiler builds one in vector registers per tile and then
// recycles those registers as load destinations, which makes it wait for every load in
// flight before the next tile's loads can be issued. Offsets at or past `bytes` read as zero
// (the resource's range check), never outside the tile.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int bytes) {
    // raw buffer (stride 0); word 3 = 32-bit data format, as gfx9 untyped loads require
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, 0x00020000);
}
// 16 bytes at byte offset `voff` of the resource, nontemporal (read once).
__device__ __forceinline__ u32x4 load16_tile_stream(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 2);
}
// 4 bytes at byte offset `voff` of the resource, default cache policy.
__device__ __forceinline__ float load4_buf(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
}
// PER consecutive floats (1, 2 or 4) at byte offset `voff` of the resource, one load.
template <int PER>
__device__ __forceinline__ void load_f32_buf(__amdgpu_buffer_rsrc_t r, unsigned voff, float (&x)[PER]) {
    static_assert(PER == 1 || PER == 2 || PER == 4, "one 4-, 8- or 16-byte load");
    if constexpr (PER == 1) {
        x[0] = load4_buf(r, voff);
    } else if constexpr (PER == 2) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0);
        x[0] = __uint_as_float(t[0]);
        x[1] = __uint_as_float(t[1]);
    } else {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(t[i]);
    }
}
// 16 bytes at byte offset `voff` of the resource, default cache policy.
__device__ __forceinline__ u32x4 load16_tile(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

// Cross-lane steps on the VALU (no trip through the LDS crossbar, which __shfl takes). Callers
// run them with all 64 lanes active.
// xor-16 / xor-32 reductions: the gfx950 permlane swaps exchange 16-lane rows (odd rows of one
// copy with even rows of the other) or wave halves, so combining the two swapped copies gives
// every lane op(x[l], x[l ^ 16]) or op(x[l], x[l ^ 32]).
__device__ __forceinline__ float xor32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max / sum over each 16-lane row with DPP (swap neighbours, swap pairs, mirror each half-row,
// mirror the row): every lane of the row ends with the row's value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
    return fmaxf(x, dpp_f<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    return x + dpp_f<0x140>(x);
}

// Inclusive prefix sum over the wave with DPP: shifts by 1, 2, 4 and 8 lanes inside each
// 16-lane row (lanes shifted in from outside the row add 0), then the last lane of row 0 is
// added to row 1 and that of row 2 to row 3 (row_bcast:15 under row mask 0b1010), and lane 31,
// by then the total of rows 0-1, to rows 2 and 3 (row_bcast:31 under row mask 0b1100).
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}
// Sum over the wave (uniform).
__device__ __forceinline__ int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_incl_scan(v), 63); }

// Softmax probability 2^(x - lse2) of a log2-domain logit under its row's log2 normaliser. A
// masked logit (-inf) gives exactly 0, whatever the normaliser: a row none of whose tokens was
// read has lse2 = -inf, where the difference alone would be NaN.
__device__ __forceinline__ float prob2(float x, float lse2) {
    return x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(x - lse2);
}

// Packs two fp32 values into bf16 (round to nearest even, hardware conversion).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (unsigned)__builtin_bit_cast(unsigned short, a) |
           ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
}
__device__ __forceinline__ float bf16_lo_f32(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_f32(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ unsigned pack_f16(float lo, float hi) {
    _Float16 a = (_Float16)lo, b = (_Float16)hi;
    return (unsigned)__builtin_bit_cast(unsigned short, a) |
           ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
}
__device__ __forceinline__ float f16_lo_f32(unsigned w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi_f32(unsigned w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// Tile products for one 16-token sub-tile ----------------------------------------------------
//
// Query heads: a kv head's G <= 8 query heads sit in MFMA columns c and c + 8 (column c holds
// head c % 8), so both halves of the 16 columns compute the same logits.
//
// 2-byte types. S^T (+)= K . Q^T with 16x16x32 MFMAs, one per chunk group of 32 dims.
// PV: a lane's V chunk np holds tokens 4j..4j+3 of dim 32np + c (elements 0..3) and of dim
// 32np + 16 + c (elements 4..7). Used as the A operand of a 16x16x32 MFMA against a B operand
// whose lane (j, c) carries P[head c % 8][4j..4j+3] in elements 0..3 when c < 8 and in
// elements 4..7 when c >= 8 (zeros elsewhere), one instruction yields dims 32np + r for the
// columns c < 8 and dims 32np + 16 + r for the columns c >= 8. Accumulator np of lane (j, c)
// therefore holds head c % 8, dims 32np + 16 * (c / 8) + 4j + i. P is split into a high part
// and a residual of the 2-byte type (two instructions), keeping ~16 significant bits.
template <class DT, int NC>
struct Tile;

template <class DT>
struct Pack2;
template <>
struct Pack2<BF16> {
    __device__ __forceinline__ static unsigned pack(float lo, float hi) { return pack_bf16(lo, hi); }
    __device__ __forceinline__ static float lo(unsigned w) { return bf16_lo_f32(w); }
    __device__ __forceinline__ static float hi(unsigned w) { return bf16_hi_f32(w); }
    __device__ __forceinline__ static f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <>
struct Pack2<F16> {
    __device__ __forceinline__ static unsigned pack(float lo, float hi) { return pack_f16(lo, hi); }
    __device__ __forceinline__ static float lo(unsigned w) { return f16_lo_f32(w); }
    __device__ __forceinline__ static float hi(unsigned w) { return f16_hi_f32(w); }
    __device__ __forceinline__ static f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

template <class DT, int NC>
struct Tile2B {
    static constexpr int kAcc = NC;  // accumulators per lane
    __device__ __forceinline__ static void qk(f32x4& s, const u32x4 (&k)[NC], const u32x4 (&q)[NC]) {
#pragma unroll
        for (int kk = 0; kk < NC; ++kk) s = Pack2<DT>::mfma(k[kk], q[kk], s);
    }
    __device__ __forceinline__ static void pv(f32x4 (&acc)[NC], const u32x4 (&v)[NC], const f32x4& p,
                                              bool upper) {
        const unsigned h01 = Pack2<DT>::pack(p.x, p.y);
        const unsigned h23 = Pack2<DT>::pack(p.z, p.w);
        const unsigned l01 = Pack2<DT>::pack(p.x - Pack2<DT>::lo(h01), p.y - Pack2<DT>::hi(h01));
        const unsigned l23 = Pack2<DT>::pack(p.z - Pack2<DT>::lo(h23), p.w - Pack2<DT>::hi(h23));
        const u32x4 bh = upper ? u32x4{0u, 0u, h01, h23} : u32x4{h01, h23, 0u, 0u};
        const u32x4 bl = upper ? u32x4{0u, 0u, l01, l23} : u32x4{l01, l23, 0u, 0u};
#pragma unroll
        for (int np = 0; np < NC; ++np) {
            acc[np] = Pack2<DT>::mfma(v[np], bh, acc[np]);
            acc[np] = Pack2<DT>::mfma(v[np], bl, acc[np]);
        }
    }
    // Zero the V elements of tokens 4j+i whose bit i of `keep` is clear (exact zero, even for NaN).
    __device__ __forceinline__ static void mask_v(u32x4 (&v)[NC], unsigned keep) {
        const unsigned m01 = ((keep & 1) ? 0x0000ffffu : 0u) | ((keep & 2) ? 0xffff0000u : 0u);
        const unsigned m23 = ((keep & 4) ? 0x0000ffffu : 0u) | ((keep & 8) ? 0xffff0000u : 0u);
#pragma unroll
        for (int np = 0; np < NC; ++np) {
            v[np].x &= m01;
            v[np].y &= m23;
            v[np].z &= m01;
            v[np].w &= m23;
        }
    }
    // Head and first dim of accumulator a in lane (j, c).
    __device__ __forceinline__ static int acc_head(int c) { return c & 7; }
    __device__ __forceinline__ static int acc_dim(int a, int j, int c) { return 32 * a + 16 * (c >> 3) + 4 * j; }
    __device__ __forceinline__ static bool acc_owner(int c) { return true; }
};

template <int NC>
struct Tile<BF16, NC> : Tile2B<BF16, NC> {};
template <int NC>
struct Tile<F16, NC> : Tile2B<F16, NC> {};

// fp32: 16x16x4 MFMAs, one element per lane. K chunk kk of lane (j, c) carries dims
// 16kk + 4j .. +3 of token c; V chunk n carries tokens 4j..4j+3 of dim 16n + c, and MFMA
// number i contracts token 4j+i of every lane group j, i.e. element i of the chunk with
// element i of P. Accumulator n of lane (j, c) holds head c % 8, dims 16n + 4j + i (the
// columns c >= 8 duplicate the columns c < 8).
template <int NC>
struct Tile<F32, NC> {
    static constexpr int kAcc = NC;
    __device__ __forceinline__ static void qk(f32x4& s, const u32x4 (&k)[NC], const u32x4 (&q)[NC]) {
#pragma unroll
        for (int kk = 0; kk < NC; ++kk) {
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k[kk].x), __uint_as_float(q[kk].x), s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k[kk].y), __uint_as_float(q[kk].y), s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k[kk].z), __uint_as_float(q[kk].z), s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k[kk].w), __uint_as_float(q[kk].w), s, 0, 0, 0);
        }
    }
    __device__ __forceinline__ static void pv(f32x4 (&acc)[NC], const u32x4 (&v)[NC], const f32x4& p, bool) {
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v[n].x), p.x, acc[n], 0, 0, 0);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v[n].y), p.y, acc[n], 0, 0, 0);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v[n].z), p.z, acc[n], 0, 0, 0);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v[n].w), p.w, acc[n], 0, 0, 0);
        }
    }
    __device__ __forceinline__ static void mask_v(u32x4 (&v)[NC], unsigned keep) {
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            v[n].x &= (keep & 1) ? ~0u : 0u;
            v[n].y &= (keep & 2) ? ~0u : 0u;
            v[n].z &= (keep & 4) ? ~0u : 0u;
            v[n].w &= (keep & 8) ? ~0u : 0u;
        }
    }
    __device__ __forceinline__ static int acc_head(int c) { return c & 7; }
    __device__ __forceinline__ static int acc_dim(int a, int j, int c) { return 16 * a + 4 * j; }
    __device__ __forceinline__ static bool acc_owner(int c) { return c < 8; }
};

}  // namespace pkv
