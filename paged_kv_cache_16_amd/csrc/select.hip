// select.hip — page selection for the next decode step ([OVAL] §3.3: each step keeps the k
// pages of highest weight and passes their ids to attention; the newest pages are always
// kept). One 1024-thread workgroup per sequence; thread t owns a contiguous range of the
// older pages.
//   1. Weights of the older pages [0, n - recent) go to LDS, each summed over the heads in
//      index order in fp32 (the stated definition, so the result is exact and
//      deterministic); they are kept as order-preserving 32-bit keys.
//   2. A radix select (four 8-bit digits, most significant first) finds the key T of the
//      want-th best page and how many pages beat it (want = k - recent, capped by the
//      number of older pages).
//   3. Pages with key > T are taken, and of the pages with key == T the ones with the
//      lowest ids fill the remaining places (a prefix count over the thread ranges).
//   4. A second prefix count places the taken ids in ascending order; the newest pages
//      follow and -1 fills the row.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kThreads = 1024;
constexpr int kHeadBatch = 32;     // head loads per page in flight before the ordered adds
constexpr int kPagesInFlight = 2;  // pages per thread fetched together

// Larger float -> larger unsigned key (finite inputs; -0 and +0 compare equal as floats,
// so both get the key of +0).
__device__ __forceinline__ unsigned order_key(float f) {
    const unsigned u = f == 0.f ? 0u : __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the 256 threads, and the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(x, off);
        if (lane >= off) x += t;
    }
    if (lane == 63) wave_tot[wv] = x;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
        const int t = wave_tot[i];
        before += i < wv ? t : 0;
        total += t;
    }
    __syncthreads();  // wave_tot may be reused by the next scan
    return before + x - v;
}

__global__ __launch_bounds__(kThreads) void select_pages_kernel(SelectParams p) {
    __shared__ unsigned key[kSelectMaxPages];
    __shared__ int hist[256];
    __shared__ int wave_tot[kThreads / 64];
    __shared__ unsigned s_prefix;
    __shared__ int s_remaining;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    // 1. weights -> keys, for every page below the stride (always inside the array), so the
    //    loads need not wait for the context length. Consecutive threads read consecutive
    //    pages; a thread fetches kPagesInFlight pages x kHeadBatch heads before adding, so
    //    that one memory round trip serves them all, and adds each page's heads in index
    //    order.
    const int L_raw = p.context_lens[b];
    const float* sc = p.scores + (size_t)b * p.heads * p.stride;
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
    if (tid == 0) {
        s_prefix = 0u;
        s_remaining = want;
    }
    __syncthreads();

    // 2. radix select of the want-th largest key
    unsigned prefix = 0u, mask = 0u;
    int remaining = want;
    if (want > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            for (int q = q_lo; q < q_hi; ++q) {
                const unsigned kq = key[q];
                if ((kq & mask) == prefix) atomicAdd(&hist[(kq >> shift) & 255u], 1);
            }
            __syncthreads();
            if (tid < 64) {
                // lane l covers digits 255-4l .. 252-4l (descending); suffix counts from the top
                int c[4], s = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    c[i] = hist[255 - 4 * tid - i];
                    s += c[i];
                }
                int incl = s;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int t = __shfl_up(incl, off);
                    if (tid >= off) incl += t;
                }
                int above = incl - s;  // keys in digits above this lane's range
                const int rem = s_remaining;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (above < rem && above + c[i] >= rem) {  // the want-th best key has this digit
                        s_prefix = prefix | ((unsigned)(255 - 4 * tid - i) << shift);
                        s_remaining = rem - above;
                    }
                    above += c[i];
                }
            }
            __syncthreads();
            prefix = s_prefix;
            remaining = s_remaining;
            mask |= 255u << shift;
        }
    }
    const unsigned T = prefix;  // key of the want-th best page; `remaining` pages with key T are taken

    // 3. ties at T: the lowest ids (thread ranges are in id order)
    int my_ties = 0;
    if (want > 0)
        for (int q = q_lo; q < q_hi; ++q) my_ties += key[q] == T ? 1 : 0;
    int total;
    const int ties_before = block_exclusive_scan(my_ties, wave_tot, total);

    // 4. taken ids ascending
    int my_taken = 0;
    if (want > 0) {
        int t = ties_before;
        for (int q = q_lo; q < q_hi; ++q) {
            const unsigned kq = key[q];
            const bool tie = kq == T;
            my_taken += (kq > T || (tie && t < remaining)) ? 1 : 0;
            t += tie ? 1 : 0;
        }
    }
    const int pos0 = block_exclusive_scan(my_taken, wave_tot, total);
    int32_t* row = p.page_list + (size_t)b * p.k;
    if (want > 0) {
        int t = ties_before, pos = pos0;
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

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t s) {
    if (p.batch <= 0) return hipSuccess;
    select_pages_kernel<<<dim3((unsigned)p.batch), dim3(kThreads), 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace pkv
