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
    if (slot < 0 || slot >= p.num_slots) return;
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

hipError_t launch_append(int dtype, const AppendParams& p, hipStream_t s) {
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
