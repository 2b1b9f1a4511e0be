// select.hip — page selection for the next decode step ([OVAL] §3.3: each step keeps the k
// pages of highest weight and passes their ids to attention; the newest pages are always
// kept). One 1024-thread workgroup per sequence; thread t owns a contiguous range of the
// older pages.
//   1. Weights of the older pages [0, n - recent) become order-preserving 32-bit keys in LDS,
//      each page's weight summed over the heads in index order in fp32 (the stated
//      definition, so the result is exact and deterministic). The score rows are first
//      staged in LDS with 16-byte loads (a 4-byte load per lane moves a quarter of the bytes
//      per address cycle, which left this phase bound by the CU's load issue rate); when all
//      of them fit, as one contiguous copy through a buffer resource.
//   2. A radix select (four 8-bit digits, most significant first) finds the key T of the
//      want-th best page and how many pages with key T are taken (want = k - recent, capped
//      by the number of older pages). Every wave reads the histogram and derives the digit
//      itself, so a pass costs one barrier.
//   3. One prefix count over the thread ranges gives, for each thread, the pages before it
//      with key > T and with key == T; the taken pages (key > T, and the lowest-id `taken
//      ties` of key == T) are written in ascending id order, then the newest pages and -1.
#include <atomic>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kHeadBatch = 32;     // unstaged path: head loads per page in flight before the adds
constexpr int kPagesInFlight = 2;  // unstaged path: pages per thread fetched together
constexpr int kStageLoads = 8;     // staged path: 16-byte loads per thread in flight
constexpr int kStaticLds = 8192;   // bytes kept free for the kernel's static LDS

// Larger float -> larger unsigned key (finite inputs; -0 and +0 compare equal as floats,
// so both get the key of +0).
__device__ __forceinline__ unsigned order_key(float f) {
    const unsigned u = f == 0.f ? 0u : __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the workgroup, and the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) wave_tot[wv] = x;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int t = wave_tot[i];
        before += i < wv ? t : 0;
        total += t;
    }
    return before + x - v;
}

// Histogram count of one digit. A wave whose counting lanes all hold the same digit (the
// leading digits of weights of one sign and magnitude range mostly do) adds once.
__device__ __forceinline__ void count_digit(int* hist, bool hit, unsigned d, int lane) {
    const unsigned long long act = __ballot(hit);
    if (!act) return;
    const int lead = __ffsll((long long)act) - 1;
    const unsigned d0 = (unsigned)__builtin_amdgcn_readlane((int)d, lead);
    if (__ballot(hit && d == d0) == act) {
        if (lane == lead) atomicAdd(&hist[d0], __popcll(act));
    } else if (hit) {
        atomicAdd(&hist[d], 1);
    }
}

__global__ __launch_bounds__(kThreads) void select_pages_kernel(SelectParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned lds[];
    unsigned* key = lds;  // [stride rounded up to 4]; staged score rows follow
    __shared__ int hist[4][256];  // one per radix pass, all cleared up front
    __shared__ int wave_tot[kWaves];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    hist[tid >> 8][tid & 255] = 0;  // kThreads == 4 * 256; ordered before the counts by the barrier below

    // 1. weights -> keys, for every page below the stride (always inside the array), so the
    //    loads need not wait for the context length.
    const float* sc = p.scores + (size_t)b * p.heads * p.stride;
    if (p.stage_pages > 0) {
        // Staged: chunks of C pages x all heads, 16-byte loads (stride % 4 == 0 and a 16-byte
        // aligned array, checked on the host), then each page's ordered sum from LDS.
        float* stg = reinterpret_cast<float*>(lds + ((p.stride + 3) & ~3));
        const int C = p.stage_pages;  // a multiple of 4
        if (C >= p.stride) {
            // One chunk: the staging rows are the score rows as they lie in memory, a contiguous
            // copy. Every 16-byte load goes out through a buffer resource (no per-lane address
            // arithmetic; loads past the block read zeros) before any is stored.
            const int total = p.heads * (p.stride >> 2);
            const __amdgpu_buffer_rsrc_t r = tile_rsrc(reinterpret_cast<const char*>(sc), total * 16);
            for (int f0 = tid; f0 < total; f0 += kThreads * kStageLoads) {
                u32x4 v[kStageLoads];
#pragma unroll
                for (int i = 0; i < kStageLoads; ++i) v[i] = load16_tile_stream(r, (unsigned)(f0 + i * kThreads) * 16u);
#pragma unroll
                for (int i = 0; i < kStageLoads; ++i) {
                    const int f = f0 + i * kThreads;
                    if (f < total) *reinterpret_cast<u32x4*>(stg + 4 * (size_t)f) = v[i];
                }
            }
            __syncthreads();
            for (int q = tid; q < p.stride; q += kThreads) {
                float acc = 0.f;
                for (int h = 0; h < p.heads; ++h) acc += stg[(size_t)h * p.stride + q];
                key[q] = order_key(acc);
            }
        } else
        for (int c0 = 0; c0 < p.stride; c0 += C) {
            const int cn = p.stride - c0 < C ? p.stride - c0 : C;
            const int nq4 = cn >> 2;
            const int total = p.heads * nq4;
            for (int f0 = tid; f0 < total; f0 += kThreads * kStageLoads) {
                f32x4 v[kStageLoads];
#pragma unroll
                for (int i = 0; i < kStageLoads; ++i) {
                    const int f = f0 + i * kThreads;
                    if (f < total) {
                        const int h = f / nq4, g = f - h * nq4;
                        v[i] = *reinterpret_cast<const f32x4*>(sc + (size_t)h * p.stride + c0 + 4 * g);
                    }
                }
#pragma unroll
                for (int i = 0; i < kStageLoads; ++i) {
                    const int f = f0 + i * kThreads;
                    if (f < total) {
                        const int h = f / nq4, g = f - h * nq4;
                        *reinterpret_cast<f32x4*>(stg + (size_t)h * C + 4 * g) = v[i];
                    }
                }
            }
            __syncthreads();
            for (int q = tid; q < cn; q += kThreads) {
                float acc = 0.f;
                for (int h = 0; h < p.heads; ++h) acc += stg[(size_t)h * C + q];
                key[c0 + q] = order_key(acc);
            }
            if (c0 + C < p.stride) __syncthreads();  // the next chunk reuses the staging rows
        }
    } else {
        // Unstaged: consecutive threads read consecutive pages; a thread fetches
        // kPagesInFlight pages x kHeadBatch heads before adding, so that one memory round trip
        // serves them all, and adds each page's heads in index order.
        for (int q0 = tid; q0 < p.stride; q0 += kThreads * kPagesInFlight) {
            float acc[kPagesInFlight];
#pragma unroll
            for (int j = 0; j < kPagesInFlight; ++j) acc[j] = 0.f;
            for (int h0 = 0; h0 < p.heads; h0 += kHeadBatch) {
                float v[kPagesInFlight][kHeadBatch];
#pragma unroll
                for (int j = 0; j < kPagesInFlight; ++j) {
                    const int q = q0 + j * kThreads;
#pragma unroll
                    for (int i = 0; i < kHeadBatch; ++i)
                        v[j][i] = (q < p.stride && h0 + i < p.heads) ? sc[(size_t)(h0 + i) * p.stride + q] : 0.f;
                }
#pragma unroll
                for (int j = 0; j < kPagesInFlight; ++j)
#pragma unroll
                    for (int i = 0; i < kHeadBatch; ++i)
                        if (h0 + i < p.heads) acc[j] += v[j][i];
            }
#pragma unroll
            for (int j = 0; j < kPagesInFlight; ++j)
                if (q0 + j * kThreads < p.stride) key[q0 + j * kThreads] = order_key(acc[j]);
        }
    }
    const int L_raw = p.context_lens[b];
    const int L = L_raw < 0 ? 0 : L_raw;
    long long n = ((long long)L + p.block_size - 1) / p.block_size;
    if (n > p.stride) {
        if (tid == 0) report(p.err, kDevPages);  // pages past the stride are never read
        n = p.stride;
    }
    const int first_recent = (int)(n - p.recent > 0 ? n - p.recent : 0);
    const int want = p.k - p.recent < first_recent ? p.k - p.recent : first_recent;
    const int chunk = (first_recent + kThreads - 1) / kThreads;
    const int q_lo = tid * chunk, q_hi = q_lo + chunk < first_recent ? q_lo + chunk : first_recent;
    __syncthreads();  // keys and cleared histograms visible

    // 2. radix select of the want-th largest key
    unsigned prefix = 0u, mask = 0u;
    int remaining = want;
    if (want > 0) {
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            int* h = hist[pass];
            for (int q = q_lo; q < q_hi; ++q) {
                const unsigned kq = key[q];
                count_digit(h, (kq & mask) == prefix, (kq >> shift) & 255u, lane);
            }
            __syncthreads();
            // lane l covers digits 255-4l .. 252-4l (descending); suffix counts from the top.
            // Every wave does this on the same counts, so all agree without another barrier.
            int c[4], s = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[i] = h[255 - 4 * lane - i];
                s += c[i];
            }
            int above = wave_incl_scan(s) - s;  // keys in digits above this lane's range
            int found = -1, rem_new = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (above < remaining && above + c[i] >= remaining) {  // the want-th best key has this digit
                    found = 255 - 4 * lane - i;
                    rem_new = remaining - above;
                }
                above += c[i];
            }
            // exactly one lane finds the digit (0 < remaining <= the keys counted)
            const int src = __ffsll((long long)__ballot(found >= 0)) - 1;
            prefix |= (unsigned)__builtin_amdgcn_readlane(found, src) << shift;
            remaining = __builtin_amdgcn_readlane(rem_new, src);
            mask |= 255u << shift;
        }
    }
    const unsigned T = prefix;  // key of the want-th best page; `remaining` pages with key T are taken

    // 3. per thread: pages with key > T and key == T (packed: each count < 2^16, at most
    //    kSelectMaxPages pages), one prefix count, then the taken ids in ascending order
    int my_gt = 0, my_tie = 0;
    if (want > 0)
        for (int q = q_lo; q < q_hi; ++q) {
            const unsigned kq = key[q];
            my_gt += kq > T ? 1 : 0;
            my_tie += kq == T ? 1 : 0;
        }
    int total;
    const int before = block_exclusive_scan((my_gt << 16) | my_tie, wave_tot, total);
    int32_t* row = p.page_list + (size_t)b * p.k;
    if (want > 0) {
        int t = before & 0xffff;  // ties before this thread's range
        int pos = (before >> 16) + (t < remaining ? t : remaining);
        for (int q = q_lo; q < q_hi; ++q) {
            const unsigned kq = key[q];
            const bool tie = kq == T;
            if (kq > T || (tie && t < remaining)) row[pos++] = q;
            t += tie ? 1 : 0;
        }
    }
    const int n_new = (int)(n - first_recent);
    for (int i = tid; i < p.k - want; i += kThreads) row[want + i] = i < n_new ? first_recent + i : -1;
}

std::atomic<int> g_lds_max[64];  // per device: LDS bytes one workgroup may use (0 = not yet asked)

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t s) {
    if (p.batch <= 0) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int lds_max = dev >= 0 && dev < 64 ? g_lds_max[dev].load(std::memory_order_relaxed) : 0;
    if (lds_max == 0) {
        e = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute((const void*)select_pages_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                lds_max - kStaticLds);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) g_lds_max[dev].store(lds_max, std::memory_order_relaxed);
    }
    SelectParams q = p;
    const long long key_bytes = (long long)((p.stride + 3) & ~3) * 4;
    q.stage_pages = 0;
    if (p.stride % 4 == 0 && ((uintptr_t)p.scores % 16) == 0) {
        long long C = ((long long)lds_max - kStaticLds - key_bytes) / (4LL * p.heads) / 4 * 4;
        if (C > p.stride) C = p.stride;
        if (C >= 4) q.stage_pages = (int)C;
    }
    const size_t dyn = (size_t)key_bytes + (size_t)q.stage_pages * p.heads * 4;
    if ((long long)dyn > (long long)lds_max - kStaticLds) return hipErrorInvalidValue;
    select_pages_kernel<<<dim3((unsigned)p.batch), dim3(kThreads), dyn, s>>>(q);
    return hipGetLastError();
}

}  // namespace pkv
