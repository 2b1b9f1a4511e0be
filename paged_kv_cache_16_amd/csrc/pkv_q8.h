// pkv_q8.h — the INT8 cache's row quantisation, as the quantising append applies it ([primer]
// "从一次线上事故说起…" §4.2: an int8 KV cache halves the bytes per token; symmetric, one fp32
// scale per (token, kv head) row of K and of V): amax = max |x| in fp32, scale = amax / 127, q = rint(x * (127 / amax)) clamped to
// [-127, 127], both divisions correctly rounded in fp32, a zero row giving scale 0 and q = 0.
#pragma once

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

__device__ __forceinline__ float q8_inv(float amax) { return amax > 0.f ? __fdiv_rn(127.f, amax) : 0.f; }
__device__ __forceinline__ float q8_scale(float amax) { return amax > 0.f ? __fdiv_rn(amax, 127.f) : 0.f; }
// The code of x (as a float) for a row with max |x| = amax and inv = q8_inv(amax).
__device__ __forceinline__ float q8_code(float x, float amax, float inv) {
    const float r = amax > 0.f ? rintf(x * inv) : 0.f;
    return fminf(fmaxf(r, -127.f), 127.f);
}

// A 2-byte input element (bf16 or fp16) as fp32.
template <class In>
__device__ __forceinline__ float in_f32(const void* base, size_t idx) {
    const unsigned short h = reinterpret_cast<const unsigned short*>(base)[idx];
    if constexpr (__is_same(In, BF16))
        return __uint_as_float((unsigned)h << 16);
    else
        return (float)__builtin_bit_cast(_Float16, h);
}

// Max over the wave of two values side by side (their cross-lane steps overlap).
__device__ __forceinline__ void wave_max2(float& a, float& b) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ta = __shfl_xor(a, off), tb = __shfl_xor(b, off);
        a = fmaxf(a, ta);
        b = fmaxf(b, tb);
    }
}

// Stores one (token, kv head h) row of K and of V at `slot` of the int8 pools: the lane holds
// dims lane + 64e of the row (xk, xv) and the wave-wide maxima ak, av. The bytes go to the row's
// lane-chunk positions (16 elements per chunk) and the scale to the pool's fp32 scale plane
// [num_blocks][Hkv][P], which follows the data plane. A slot < 0 is skipped; a slot past the
// pool is skipped and reported (by kv head 0).
template <int D>
__device__ __forceinline__ void q8_store_row(char* kpool, char* vpool, const float (&xk)[D / 64],
                                             const float (&xv)[D / 64], float ak, float av, int64_t slot,
                                             int block_size, int kv_heads, int h, int64_t num_slots,
                                             unsigned* err, int lane) {
    constexpr int PER = D / 64;
    if (slot < 0) return;
    if (slot >= num_slots) {
        if (h == 0 && lane == 0) report(err, kDevSlot);
        return;
    }
    const int64_t blk = slot / block_size;
    const int t = (int)(slot - blk * block_size);
    const int tau = t & 15;
    const size_t sub = (((size_t)blk * kv_heads + h) * block_size + (t - tau)) * (size_t)D;
    const size_t plane = (size_t)num_slots * kv_heads * D;  // bytes of the data plane
    const size_t srow = ((size_t)blk * kv_heads + h) * block_size + t;
#pragma unroll
    for (int is_v = 0; is_v < 2; ++is_v) {
        char* pool = is_v ? vpool : kpool;
        const float amax = is_v ? av : ak;
        const float inv = q8_inv(amax);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const float r = q8_code(is_v ? xv[e] : xk[e], amax, inv);
            const int xd = lane + 64 * e;
            size_t pos;
            if (is_v) {
                const int n = xd >> 4;
                pos = (((size_t)(n >> 2) * 4 + (tau >> 2)) * 16 + (xd & 15)) * 16 + (size_t)(n & 3) * 4 + (tau & 3);
            } else {
                pos = ((size_t)(xd >> 6) * 64 + (size_t)((xd >> 4) & 3) * 16 + tau) * 16 + (xd & 15);
            }
            pool[sub + pos] = (char)(signed char)(int)r;
        }
        if (lane == 0) *reinterpret_cast<float*>(pool + plane + srow * 4) = q8_scale(amax);
    }
}

// The fused decode step on an INT8 cache: the new (token, kv head) row quantised as above,
// cut the way a lane of the attention kernel holds token tau of a sub-tile.
//   K: lane (j, c) holds, in its chunk m, the 16 codes of dims 64m + 16j .. +15 of token c;
//   V: lane (j, c) holds, in byte (n % 4) * 4 + i of its chunk n / 4, the code of dim 16n + c of
//      token 4j + i.
// Every lane quantises its own slice (the lanes that hold the token take it): the K maximum is
// taken over the 4 lanes of a column (each holds 32 of the 128 dims at d = 128), the V maximum
// over the 16 lanes of a row.
template <int D>
struct NewRowQ8 {
    static constexpr int NC = D / 64;  // 16-byte chunks per lane
    u32x4 k[NC];                       // K codes of the lane's chunks
    unsigned v[NC];                    // V codes of dims 16n + c, n = 4m .. 4m + 3, byte n % 4
    float ks, vs;                      // the row's K and V scales
};

__device__ __forceinline__ unsigned q8_byte(float code) { return (unsigned)(int)code & 0xffu; }

template <class In>
__device__ __forceinline__ float in_lo(unsigned w) {
    if constexpr (__is_same(In, BF16))
        return __uint_as_float(w << 16);
    else
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
template <class In>
__device__ __forceinline__ float in_hi(unsigned w) {
    if constexpr (__is_same(In, BF16))
        return __uint_as_float(w & 0xffff0000u);
    else
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// The new row as loaded: lane l holds elements l * DPL .. l * DPL + DPL - 1 of K and of V
// (DPL = D / 64 two-byte elements, one 2- or 4-byte load each). It is requested when a run starts
// and quantised once the run's first K/V loads are out, so no wait for it sits in the run's
// set-up (quantising right after the request held every run's first loads back by one round
// trip).
template <int D>
struct NewRowRaw {
    static constexpr int DPL = D / 64;
    unsigned k, v;
};

template <int D>
__device__ __forceinline__ void load_new_row_raw(const DecodeParams& p, NewRowRaw<D>& raw, int b, int kvh, int lane) {
    constexpr int DPL = D / 64;
    static_assert(DPL == 1 || DPL == 2, "head dim 64 or 128");
    const size_t src = (((size_t)b * p.kv_heads + kvh) * D + (size_t)lane * DPL) * 2;
    if constexpr (DPL == 2) {
        raw.k = *reinterpret_cast<const unsigned*>(p.k_new + src);
        raw.v = *reinterpret_cast<const unsigned*>(p.v_new + src);
    } else {
        raw.k = *reinterpret_cast<const unsigned short*>(p.k_new + src);
        raw.v = *reinterpret_cast<const unsigned short*>(p.v_new + src);
    }
}

// Quantises the row (each lane its DPL elements; the maxima over the wave) and deals the codes
// out through a 2 * D byte LDS stage of the wave's own into the layout NewRowQ8 holds: K codes
// as row j's bytes j * D/4 + 16m + e (dim 64m + 16j + e), V codes as lane c's bytes c * D/16 + n
// (dim 16n + c). All 64 lanes take part. The row passes through an empty asm statement first:
// the conversions below are loop-invariant where this is called inside a loop, and hoisted out
// of it they would wait for the row's loads where they were issued.
template <class In, int D>
__device__ __forceinline__ void quantise_new_row(NewRowRaw<D> raw, NewRowQ8<D>& nr, unsigned char* stage, int lane,
                                                 int j, int c) {
    constexpr int DPL = D / 64, NC = D / 64, NV = D / 16;
    asm volatile("" : "+v"(raw.k), "+v"(raw.v));
    float xk[DPL], xv[DPL];
    xk[0] = in_lo<In>(raw.k);
    xv[0] = in_lo<In>(raw.v);
    if constexpr (DPL == 2) {
        xk[1] = in_hi<In>(raw.k);
        xv[1] = in_hi<In>(raw.v);
    }
    float ak = 0.f, av = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        ak = fmaxf(ak, fabsf(xk[e]));
        av = fmaxf(av, fabsf(xv[e]));
    }
    ak = xor32_max(xor16_max(row16_max(ak)));
    av = xor32_max(xor16_max(row16_max(av)));
    const float ik = q8_inv(ak), iv = q8_inv(av);
    nr.ks = q8_scale(ak);
    nr.vs = q8_scale(av);
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        const int x = lane * DPL + e;
        stage[((x >> 4) & 3) * (D / 4) + (x >> 6) * 16 + (x & 15)] = (unsigned char)q8_byte(q8_code(xk[e], ak, ik));
        stage[D + (x & 15) * NV + (x >> 4)] = (unsigned char)q8_byte(q8_code(xv[e], av, iv));
    }
#pragma unroll
    for (int m = 0; m < NC; ++m) nr.k[m] = *reinterpret_cast<const u32x4*>(stage + j * (D / 4) + m * 16);
    if constexpr (NC == 2) {
        const uint2 w = *reinterpret_cast<const uint2*>(stage + D + c * NV);
        nr.v[0] = w.x;
        nr.v[1] = w.y;
    } else {
        nr.v[0] = *reinterpret_cast<const unsigned*>(stage + D + c * NV);
    }
}

// Replaces token tau of a loaded INT8 sub-tile (codes and the two row scales) by the new row.
template <int D>
__device__ __forceinline__ void patch_tile_q8(u32x4 (&k)[D / 64], u32x4 (&v)[D / 64], f32x4& ks, f32x4& vs,
                                             const NewRowQ8<D>& nr, int tau, int j, int c) {
    constexpr int NC = D / 64;
    if (c == tau) {
#pragma unroll
        for (int m = 0; m < NC; ++m) k[m] = nr.k[m];
    }
    if (j == (tau >> 2)) {
        const int i = tau & 3;
        const unsigned sh = 8u * (unsigned)i;
#pragma unroll
        for (int m = 0; m < NC; ++m) {
#pragma unroll
            for (int w = 0; w < 4; ++w)
                v[m][w] = (v[m][w] & ~(0xffu << sh)) | (((nr.v[m] >> (8 * w)) & 0xffu) << sh);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ks[e] = e == i ? nr.ks : ks[e];
            vs[e] = e == i ? nr.vs : vs[e];
        }
    }
}

// Stores the fused step's new row (sequence b, kv head h; r = b * kv_heads + h) into the INT8
// pools, one wave per row, exactly as the quantising append does.
template <class In, int D>
__device__ __forceinline__ void write_new_row_q8(const DecodeParams& p, int r, int lane) {
    constexpr int PER = D / 64;
    const int b = r / p.kv_heads, h = r - b * p.kv_heads;
    float xk[PER], xv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        xk[e] = in_f32<In>(p.k_new, (size_t)r * D + lane + 64 * e);
        xv[e] = in_f32<In>(p.v_new, (size_t)r * D + lane + 64 * e);
    }
    const int64_t slot = p.new_slots[b];
    float ak = 0.f, av = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        ak = fmaxf(ak, fabsf(xk[e]));
        av = fmaxf(av, fabsf(xv[e]));
    }
    wave_max2(ak, av);
    q8_store_row<D>(p.k_cache_w, p.v_cache_w, xk, xv, ak, av, slot, p.block_size, p.kv_heads, h, p.num_slots,
                    p.err, lane);
}

}  // namespace pkv
