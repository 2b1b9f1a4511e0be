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

// Fused append ----------------------------------------------------------------------------

// Cache write of the fused decode step, one new row (sequence b, kv head h) per call: stored
// at slot new_slots[b] in the cache's lane-chunk order. It runs after every read of that
// (sequence, kv head) row set has returned (in the combine kernel on the persistent path, at
// the end of the segment's own workgroup on the one-kernel path); attention takes the new
// token from k_new/v_new directly.
template <int ES, int D>
__device__ __forceinline__ void write_new_row(const DecodeParams& p, int r, int lane) {
    constexpr int E = 16 / ES, R = E / 4;
    const int b = r / p.kv_heads, h = r - b * p.kv_heads;
    const int64_t slot = p.new_slots[b];
    if (slot < 0) return;
    if (slot >= p.num_slots) {
        if (h == 0 && lane == 0) report(p.err, kDevSlot);
        return;
    }
    const int64_t blk = slot / p.block_size;
    const int t = (int)(slot - blk * p.block_size);
    const int tau = t & 15;
    const size_t sub = (((size_t)blk * p.kv_heads + h) * p.block_size + (t - tau)) * D;
    const size_t src = (size_t)r * D;
    if (lane < D / E) {  // K: one whole 16-byte chunk per lane
        const size_t chunk = (size_t)(lane >> 2) * 64 + (size_t)(lane & 3) * 16 + tau;
        *reinterpret_cast<u32x4*>(p.k_cache_w + (sub + chunk * E) * ES) = load16(p.k_new + (src + lane * E) * ES);
    }
    for (int x = lane; x < D; x += 64) {  // V: element by element
        const int n = x >> 4;
        const size_t chunk = ((size_t)(n / R) * 4 + (tau >> 2)) * 16 + (x & 15);
        const size_t pos = (size_t)(n % R) * 4 + (tau & 3);
        if constexpr (ES == 2)
            *reinterpret_cast<unsigned short*>(p.v_cache_w + (sub + chunk * E + pos) * 2) =
                *reinterpret_cast<const unsigned short*>(p.v_new + (src + x) * 2);
        else
            *reinterpret_cast<unsigned*>(p.v_cache_w + (sub + chunk * E + pos) * 4) =
                *reinterpret_cast<const unsigned*>(p.v_new + (src + x) * 4);
    }
}

// The new token's values as lane (j, c) holds them in a tile: K chunks of token c (dims
// kk*4E + j*E ..), and the V elements of dims 16n + c. Loaded once per run of the fused step.
template <class DT, int D>
struct NewRow {
    static constexpr int NC = D / (4 * DT::kE);
    static constexpr int NV = D / 16;  // V dims 16n + c, n < D/16
    u32x4 k[NC];
    unsigned v[NV];  // raw element bits (low 16 bits for 2-byte types)
};

template <class DT, int D>
__device__ __forceinline__ void load_new_row(const DecodeParams& p, NewRow<DT, D>& nr, int b, int kvh, int j,
                                             int c) {
    constexpr int E = DT::kE, ES = DT::kBytes;
    const size_t src = ((size_t)b * p.kv_heads + kvh) * D;
#pragma unroll
    for (int kk = 0; kk < NewRow<DT, D>::NC; ++kk) nr.k[kk] = load16(p.k_new + (src + kk * 4 * E + j * E) * ES);
#pragma unroll
    for (int n = 0; n < NewRow<DT, D>::NV; ++n) {
        if constexpr (ES == 2)
            nr.v[n] = *reinterpret_cast<const unsigned short*>(p.v_new + (src + 16 * n + c) * 2);
        else
            nr.v[n] = *reinterpret_cast<const unsigned*>(p.v_new + (src + 16 * n + c) * 4);
    }
}

// Replaces token tau of a loaded tile by the new row (lanes that hold it).
template <class DT, int D>
__device__ __forceinline__ void patch_tile(u32x4 (&k)[D / (4 * DT::kE)], u32x4 (&v)[D / (4 * DT::kE)],
                                          const NewRow<DT, D>& nr, int tau, int j, int c) {
    constexpr int NC = D / (4 * DT::kE);
    constexpr int R = DT::kE / 4;
    if (c == tau) {
#pragma unroll
        for (int kk = 0; kk < NC; ++kk) k[kk] = nr.k[kk];
    }
    if (j == (tau >> 2)) {
        const int i = tau & 3;
#pragma unroll
        for (int n = 0; n < D / 16; ++n) {
            // token 4j+i of dim 16n + c is element (n % R) * 4 + i of chunk n / R
            if constexpr (DT::kBytes == 2) {
                const int target = (n % R) * 2 + (i >> 1);  // dword holding the element
                // one byte permute puts the element's two bytes in the high or low half of the
                // dword (bytes 0-3 select from wd, 4-7 from the new row); nothing here depends
                // on the new row alone, so its loads are not waited for before the tile is
                const unsigned sel = (i & 1) ? 0x05040100u : 0x03020504u;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const unsigned wd = v[n / R][w];
                    const unsigned upd = __builtin_amdgcn_perm(nr.v[n], wd, sel);
                    v[n / R][w] = w == target ? upd : wd;
                }
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) v[n][w] = w == i ? nr.v[n] : v[n][w];
            }
        }
    }
}

}  // namespace pkv
