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

}  // namespace pkv
