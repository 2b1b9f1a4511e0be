// pkv_plan.h — per-sequence token-set planning shared by the decode kernels.
//
// The attended token set of a sequence (full; sliding window plus sinks; listed pages) is
// enumerated as aligned 16-token "units" (one MFMA sub-tile each). A unit is processed
// whole; tokens of it outside the attended set are masked.
#pragma once

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

struct SeqPlan {
    int L;        // context length, clamped to the table / grid bounds
    int e0;       // attended: t < e0 (sinks) or t >= s1 (window); full: e0 = s1 = 0
    int s1;
    int n0;       // units of the sink range
    int u1a;      // unit index (t / 16) where the window range starts
    int n_units;  // units enumerated for this sequence
};

// Plan of a sequence whose context_lens entry is L (clamped here).
template <int MODE>
__device__ __forceinline__ SeqPlan make_plan_len(const DecodeParams& p, int L) {
    SeqPlan sp;
    if (L > p.len_cap) report(p.err, kDevContext);  // clamped: beyond max_context_len or the table
    L = L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
    sp.L = L;
    sp.e0 = 0;
    sp.s1 = 0;
    sp.n0 = 0;
    sp.u1a = 0;
    const int nu_full = (L + 15) >> 4;
    if (MODE == kPages) {
        sp.n_units = p.pages_per_seq * (p.block_size >> 4);
    } else if (MODE == kWindow && p.window < L) {
        const int e0 = p.sinks < L ? p.sinks : L;
        int s1 = L - p.window;
        if (s1 < e0) s1 = e0;
        sp.e0 = e0;
        sp.s1 = s1;
        sp.n0 = (e0 + 15) >> 4;
        sp.u1a = (s1 >> 4) > sp.n0 ? (s1 >> 4) : sp.n0;
        sp.n_units = sp.n0 + (nu_full - sp.u1a);
    } else {
        sp.n_units = nu_full;
    }
    return sp;
}

template <int MODE>
__device__ __forceinline__ SeqPlan make_plan(const DecodeParams& p, int b) {
    return make_plan_len<MODE>(p, p.context_lens[b]);
}

// First logical token of unit u, or -1 when the unit holds no attended token.
template <int MODE>
__device__ __forceinline__ int unit_token(const DecodeParams& p, const SeqPlan& sp, int b, int u) {
    if (MODE == kPages) {
        const int per = p.block_size >> 4;
        const int k = u / per;
        const int pg = p.page_list[(size_t)b * p.pages_per_seq + k];
        if (pg < 0) return -1;
        const int64_t t0 = (int64_t)pg * p.block_size + (int64_t)(u - k * per) * 16;
        return t0 < sp.L ? (int)t0 : -1;
    } else if (MODE == kWindow) {
        return (u < sp.n0 ? u : sp.u1a + (u - sp.n0)) << 4;
    }
    return u << 4;
}

// Block-table column of logical page `page`: the page itself, or on a window layer's ring
// table ([Novita] §關鍵技術 1: a window layer keeps fewer blocks) the sink columns first and
// then page - sink_pages taken modulo the ring size.
__device__ __forceinline__ int table_col(const DecodeParams& p, int page) {
    if (p.ring_pages > 0 && page >= p.ring_sink_pages)
        return p.ring_sink_pages + (page - p.ring_sink_pages) % p.ring_pages;
    return page;
}

// Bit i set: token t0 + 4j + i is attended.
__device__ __forceinline__ unsigned token_keep(const SeqPlan& sp, int t0, int j) {
    if (t0 < 0) return 0u;
    unsigned keep = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * j + i;
        const bool ok = t < sp.L && (t < sp.e0 || t >= sp.s1);
        keep |= ok ? (1u << i) : 0u;
    }
    return keep;
}

// Whole unit attended (uniform across the wave).
__device__ __forceinline__ bool unit_full(const SeqPlan& sp, int t0) {
    return t0 >= 0 && t0 + 16 <= sp.L && (t0 >= sp.s1 || t0 + 16 <= sp.e0);
}

__device__ __forceinline__ void store_out(void* out, int out_dtype, size_t idx, float v) {
    if (out_dtype == kF32) {
        reinterpret_cast<float*>(out)[idx] = v;
    } else if (out_dtype == kF16) {
        reinterpret_cast<_Float16*>(out)[idx] = (_Float16)v;
    } else {
        reinterpret_cast<__bf16*>(out)[idx] = (__bf16)v;
    }
}

}  // namespace pkv
