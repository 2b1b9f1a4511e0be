// append.hip — kv_cache_append: scatter the new tokens' K/V rows into their pages.
//
// Decode step ([primer] "从一次线上事故说起…" §2.2; [naive] koas-w "naive KV cache" post,
// §"KV cache的思想"): the new token's K and V are written once into the cache before
// attention reads it; with a paged cache ([primer] §4.1) the destination is the slot
// block * P + offset of a physical block that need not be contiguous with the others.
//
// A few tokens: one thread moves one 16-byte chunk of one (token, kv head) row. Many tokens:
// one workgroup per 16 tokens and kv head (a wave per 64 chunks), which writes whole sub-tiles
// when the tokens fill one. Bytes are copied, never converted (an INT8 cache's rows are
// quantised: append_q8_kernel).
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_q8.h"

namespace pkv {

// Moves chunk qc of token i's (kv head h) row: the K chunk lands as a whole 16-byte chunk of
// the lane-chunk layout; the V chunk's elements are spread over the sub-tile (each V chunk of
// the layout interleaves 4 tokens), so they are stored one element at a time.
template <class DT>
__device__ __forceinline__ void append_chunk(const AppendParams& p, int64_t i, int h, int qc, bool report_slot) {
    constexpr int E = DT::kE;
    constexpr int ES = DT::kBytes;
    constexpr int R = E / 4;
    const int D = p.head_dim;
    const int64_t slot = p.slots[i];
    if (slot < 0) return;
    if (slot >= p.num_slots) {
        if (report_slot) report(p.err, kDevSlot);
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

// One thread per 16-byte chunk of a (token, kv head) row: few tokens (a decode step).
template <class DT>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    const int chunks = p.head_dim / DT::kE;
    const int64_t per_token = (int64_t)p.kv_heads * chunks;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= p.num_tokens * per_token) return;
    const int64_t i = gid / per_token;
    const int rem = (int)(gid - i * per_token);
    const int h = rem / chunks;
    append_chunk<DT>(p, i, h, rem - h * chunks, rem == 0);
}

// Many tokens (a prefill, or a long append): one workgroup per (16 consecutive input tokens,
// kv head), one wave per group of 64 chunks of the sub-tile (D / 4E waves: the waves read the
// quarters of the same 128-byte lines together). When the 16 tokens go to the 16 consecutive
// slots of one sub-tile (slots s0 .. s0 + 15 with s0 a multiple of 16), each wave writes its 64
// chunks of the sub-tile whole: a K chunk is 8 (fp32: 4) dims of one token, taken with one
// 16-byte load; a V chunk holds 4 tokens x 2 (fp32: 1) dims, read back from the 16 rows' block
// staged in LDS (one 16-byte load per lane); every store is a 16-byte chunk, 1 KiB per wave
// instruction. Other groups store chunk by chunk as append_kernel does, the group's waves
// sharing the chunks.
template <class DT>
__global__ __launch_bounds__(512) void append_tile_kernel(AppendParams p) {
    constexpr int E = DT::kE;
    constexpr int ES = DT::kBytes;
    constexpr int R = E / 4;
    const int D = p.head_dim;
    const int lane = threadIdx.x & 63;
    const int kk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // the wave's 64 chunks of the sub-tile
    const int h = blockIdx.y;
    const int64_t i0 = (int64_t)blockIdx.x * 16;
    const int nt = p.num_tokens - i0 < 16 ? (int)(p.num_tokens - i0) : 16;
    const int my_slot = lane < nt ? p.slots[i0 + lane] : -1;
    const int s0 = __builtin_amdgcn_readfirstlane(my_slot);
    const unsigned long long run = __ballot(lane < 16 && (long long)my_slot == (long long)s0 + lane);
    const bool tile = nt == 16 && s0 >= 0 && (s0 & 15) == 0 && (long long)s0 + 15 < p.num_slots && run == 0xffffull;
    if (!tile) {
        const int chunks = D / E;
        for (int job = threadIdx.x; job < nt * chunks; job += blockDim.x)
            append_chunk<DT>(p, i0 + job / chunks, h, job % chunks, job % chunks == 0 && h == 0);
        return;
    }
    const int64_t blk = s0 / p.block_size;
    const int t = (int)(s0 - blk * p.block_size);  // a multiple of 16
    const size_t sub = (((size_t)blk * p.kv_heads + h) * p.block_size + t) * (size_t)D;
    const size_t row_stride = (size_t)p.kv_heads * D;  // elements between consecutive tokens' rows
    const char* krows = (const char*)p.k_new + ((size_t)i0 * p.kv_heads + h) * D * ES;
    const char* vrows = (const char*)p.v_new + ((size_t)i0 * p.kv_heads + h) * D * ES;
    const int j = lane >> 4, c = lane & 15;
    {
        // K chunk kk * 64 + lane: token c, dims kk*4E + j*E .. + E - 1
        const u32x4 kv = load16(krows + ((size_t)c * row_stride + kk * 4 * E + j * E) * ES);
        *reinterpret_cast<u32x4*>((char*)p.k_cache + (sub + ((size_t)kk * 64 + lane) * E) * ES) = kv;
        // V: the wave's 64 chunks hold tokens 0..15 x dims kk*4E .. kk*4E + 4E - 1, the same
        // 64 bytes of each token's row. Lane (token l / 4, quarter l % 4) loads 16 of them into
        // LDS (rows 80 bytes apart), and lane (j, c) reads back the elements of its chunk:
        // position (n % R) * 4 + i holds token 4j + i, dim 16n + c, n = kk * R + position / 4,
        // which is local dim 16 * (position / 4) + c of the block.
        __shared__ __attribute__((aligned(16))) unsigned char vblks[8][16 * 80];
        unsigned char* vblk = vblks[kk];
        {
            const int tk = lane >> 2, qt = lane & 3;
            *reinterpret_cast<u32x4*>(vblk + tk * 80 + qt * 16) =
                load16(vrows + ((size_t)tk * row_stride + kk * 4 * E + qt * E) * ES);
        }
        __syncthreads();  // every wave of the group takes this path (the same slots decide it)
        unsigned w[4];
        if constexpr (ES == 2) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // dword q: positions 2q, 2q + 1
                unsigned short e2[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int pos = 2 * q + hh;
                    e2[hh] = *reinterpret_cast<const unsigned short*>(vblk + (4 * j + pos % 4) * 80 +
                                                                      (16 * (pos / 4) + c) * 2);
                }
                w[q] = (unsigned)e2[0] | ((unsigned)e2[1] << 16);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)  // position q: token 4j + q, dim 16 kk + c
                w[q] = *reinterpret_cast<const unsigned*>(vblk + (4 * j + q) * 80 + c * 4);
        }
        *reinterpret_cast<u32x4*>((char*)p.v_cache + (sub + ((size_t)kk * 64 + lane) * E) * ES) =
            u32x4{w[0], w[1], w[2], w[3]};
    }
}

// INT8 cache: one wavefront quantises and stores one (token, kv head) row of K and of V
// (q8_store_row: per-row amax and scale, codes at the row's lane-chunk positions).
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
    q8_store_row<D>((char*)p.k_cache, (char*)p.v_cache, xk, xv, ak, av, slot, p.block_size, p.kv_heads, h,
                    p.num_slots, p.err, lane);
}

// Appends of at least this many tokens take the sub-tile kernel (a decode step's few tokens, one
// per sequence, never fill a sub-tile).
constexpr int64_t kAppendTileMin = 64;

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
    if (p.num_tokens <= 0) return hipSuccess;
    if (p.num_tokens >= kAppendTileMin) {
        const int64_t groups = (p.num_tokens + 15) / 16;
        if (groups > 0x7fffffff || p.kv_heads > 65535) return hipErrorInvalidValue;
        // one wave per 64-chunk group of the sub-tile (D / (4 E) of them)
        const dim3 g((unsigned)groups, (unsigned)p.kv_heads), b(64 * (unsigned)(p.head_dim / (dtype == kF32 ? 16 : 32)));
        switch (dtype) {
            case kF32: append_tile_kernel<F32><<<g, b, 0, s>>>(p); break;
            case kF16: append_tile_kernel<F16><<<g, b, 0, s>>>(p); break;
            default: append_tile_kernel<BF16><<<g, b, 0, s>>>(p); break;
        }
        return hipGetLastError();
    }
    const int E = dtype == kF32 ? 4 : 8;
    const int64_t threads = p.num_tokens * p.kv_heads * (p.head_dim / E);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    switch (dtype) {
        case kF32: append_kernel<F32><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p); break;
        case kF16: append_kernel<F16><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p); break;
        default: append_kernel<BF16><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p); break;
    }
    return hipGetLastError();
}

}  // namespace pkv
