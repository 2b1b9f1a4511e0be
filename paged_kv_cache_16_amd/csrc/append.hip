// append.hip — kv_cache_append: scatter the new tokens' K/V rows into their pages.
//
// Decode step ([primer] "从一次线上事故说起…" §2.2; [naive] koas-w "naive KV cache" post,
// §"KV cache的思想"): the new token's K and V are written once into the cache before
// attention reads it; with a paged cache ([primer] §4.1) the destination is the slot
// block * P + offset of a physical block that need not be contiguous with the others.
//
// One thread moves one 16-byte chunk of one (token, kv head) row. The K chunk lands as a
// whole 16-byte chunk of the lane-chunk layout; the V chunk's elements are spread over
// the sub-tile (each V chunk of the layout interleaves 4 tokens), so they are stored one
// element at a time. Bytes are copied, never converted.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <class DT>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    constexpr int E = DT::kE;
    constexpr int ES = DT::kBytes;
    constexpr int R = E / 4;
    const int D = p.head_dim;
    const int chunks = D / E;
    const int64_t per_token = (int64_t)p.kv_heads * chunks;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= p.num_tokens * per_token) return;
    const int64_t i = gid / per_token;
    const int rem = (int)(gid - i * per_token);
    const int h = rem / chunks;
    const int qc = rem - h * chunks;

    const int64_t slot = p.slots[i];
    if (slot < 0) return;
    if (slot >= p.num_slots) {
        if (rem == 0) report(p.err, kDevSlot);
        return;
    }
    const int64_t blk = slot / p.block_size;
    const int t = (int)(slot - blk * p.block_size);
    const int tau = t & 15;
    // first element of the 16-token sub-tile holding token t of (blk, h)
    const size_t sub = (((size_t)blk * p.kv_heads + h) * p.block_size + (t - tau)) * (size_t)D;
    const size_t src = ((size_t)i * p.kv_heads + h) * D + (size_t)qc * E;

    // K: chunk (qc / 4) * 64 + (qc % 4) * 16 + tau of the sub-tile
    const u32x4 kv = load16((const char*)p.k_new + src * ES);
    const size_t kchunk = (size_t)(qc >> 2) * 64 + (size_t)(qc & 3) * 16 + tau;
    *reinterpret_cast<u32x4*>((char*)p.k_cache + (sub + kchunk * E) * ES) = kv;

    // V: element x = qc*E + e goes to chunk ((n / R) * 4 + tau / 4) * 16 + x % 16, position
    // (n % R) * 4 + tau % 4, with n = x / 16.
    const u32x4 vv = load16((const char*)p.v_new + src * ES);
    const int jj = tau >> 2, ii = tau & 3;
    char* vbase = (char*)p.v_cache + sub * ES;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int x = qc * E + e;
        const int n = x >> 4;
        const size_t chunk = ((size_t)(n / R) * 4 + jj) * 16 + (x & 15);
        const size_t pos = (size_t)(n % R) * 4 + ii;
        if constexpr (ES == 2) {
            const unsigned wv = vv[e >> 1];
            const unsigned short hv = (e & 1) ? (unsigned short)(wv >> 16) : (unsigned short)(wv & 0xffffu);
            *reinterpret_cast<unsigned short*>(vbase + (chunk * E + pos) * 2) = hv;
        } else {
            *reinterpret_cast<unsigned*>(vbase + (chunk * E + pos) * 4) = vv[e];
        }
    }
}

// INT8 cache ([primer] §4.2: the int8 KV cache halves the bytes per token). One wavefront
// quantises one (token, kv head) row of K and of V: amax = max |x| in fp32 (a wave-wide
// max), scale = amax / 127, q = rint(x * (127 / amax)) clamped to [-127, 127], both
// divisions correctly rounded in fp32, a zero row giving scale 0 and q = 0 (symmetric, one
// scale per row, so no earlier token is ever re-quantised). The bytes go to the row's
// lane-chunk positions (16 elements per chunk) and the scale to the pool's fp32 scale
// plane [num_blocks][Hkv][P], which follows the data plane.
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

template <class In, int D>
__global__ __launch_bounds__(256) void append_q8_kernel(AppendParams p) {
    constexpr int PER = D / 64;  // elements per lane
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.num_tokens * p.kv_heads) return;
    const int64_t i = row / p.kv_heads;
    const int h = (int)(row - i * p.kv_heads);
    // The row's K and V values do not depend on its slot: they are requested together with
    // it, and the row maxima (cross-lane steps, which stay where they are written) come
    // before the slot's checks, so the wave waits for one round trip instead of three.
    float xk[PER], xv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        xk[e] = in_f32<In>(p.k_new, (size_t)row * D + lane + 64 * e);
        xv[e] = in_f32<In>(p.v_new, (size_t)row * D + lane + 64 * e);
    }
    const int64_t slot = p.slots[i];
    float ak = 0.f, av = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        ak = fmaxf(ak, fabsf(xk[e]));
        av = fmaxf(av, fabsf(xv[e]));
    }
    wave_max2(ak, av);
    if (slot < 0) return;
    if (slot >= p.num_slots) {
        if (h == 0 && lane == 0) report(p.err, kDevSlot);
        return;
    }
    const int64_t blk = slot / p.block_size;
    const int t = (int)(slot - blk * p.block_size);
    const int tau = t & 15;
    const size_t sub = (((size_t)blk * p.kv_heads + h) * p.block_size + (t - tau)) * (size_t)D;
    const size_t plane = (size_t)p.num_slots * p.kv_heads * D;  // bytes of the data plane
    const size_t srow = ((size_t)blk * p.kv_heads + h) * p.block_size + t;
#pragma unroll
    for (int is_v = 0; is_v < 2; ++is_v) {
        char* pool = (char*)(is_v ? p.v_cache : p.k_cache);
        const float amax = is_v ? av : ak;
        const float inv = amax > 0.f ? __fdiv_rn(127.f, amax) : 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            float r = amax > 0.f ? rintf((is_v ? xv[e] : xk[e]) * inv) : 0.f;
            r = fminf(fmaxf(r, -127.f), 127.f);
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
        if (lane == 0) *reinterpret_cast<float*>(pool + plane + srow * 4) = amax > 0.f ? __fdiv_rn(amax, 127.f) : 0.f;
    }
}

hipError_t launch_append(int dtype, const AppendParams& p, hipStream_t s) {
    if (dtype == kI8B || dtype == kI8H) {
        const int64_t rows = p.num_tokens * p.kv_heads;
        const int64_t blocks = (rows + 3) / 4;
        if (blocks <= 0) return hipSuccess;
        if (blocks > 0x7fffffff) return hipErrorInvalidValue;
        const dim3 g((unsigned)blocks), b(256);
        if (dtype == kI8B)
            p.head_dim == 64 ? append_q8_kernel<BF16, 64><<<g, b, 0, s>>>(p) : append_q8_kernel<BF16, 128><<<g, b, 0, s>>>(p);
        else
            p.head_dim == 64 ? append_q8_kernel<F16, 64><<<g, b, 0, s>>>(p) : append_q8_kernel<F16, 128><<<g, b, 0, s>>>(p);
        return hipGetLastError();
    }
    const int E = dtype == kF32 ? 4 : 8;
    const int64_t threads = p.num_tokens * p.kv_heads * (p.head_dim / E);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    switch (dtype) {
        case kF32: append_kernel<F32><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p); break;
        case kF16: append_kernel<F16><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p); break;
        default: append_kernel<BF16><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p); break;
    }
    return hipGetLastError();
}

}  // namespace pkv
