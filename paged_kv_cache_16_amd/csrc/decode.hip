// decode.hip — split-K paged decode attention and the cross-split log-sum-exp combine.
//
// What is computed ([TF] "Transformer模型中的KV Cache优化推理策略", §"为什么传统推理方式难以为继？":
// softmax(q K^T / sqrt(d)) V for the one new query of each sequence; [primer]
// "从一次线上事故说起…" §4.1: the keys and values sit in fixed-size blocks reached through
// a per-sequence block table; [primer] §4.3 and [Novita] "How KV Sparsity Achieves 1.5x
// Acceleration for vLLM" §關鍵技術 1: a per-layer sliding window; [OVAL] "Output-Aware Local
// Page Bases for KV Cache Retrieval" §2.2/§3.3: a per-step list of pages to read).
//
// How (gfx950):
//  * One workgroup = 4 wavefronts = one (partition, kv head, sequence). The attended token
//    set of a sequence is enumerated as aligned 16-token units; a partition is a run of
//    consecutive units, dealt round-robin to the 4 waves, two units per step.
//  * All G query heads of a kv head ride in the N dimension of the matrix instructions, so
//    every K/V sub-tile is read from HBM once per group.
//  * Per unit a lane issues 2 * D / (4E) 16-byte loads; each load instruction of a wave
//    reads 1 KiB of consecutive bytes (the pool layout puts each lane's operand chunk in
//    lane order). Loads of the next pair of units are in flight while the current pair is
//    multiplied.
//  * S^T = K . Q^T and O^T += V^T . P^T on the matrix cores; the logits land in exactly the
//    registers the second product takes as its B operand, so P never moves between lanes.
//  * Online softmax per head in the log2 domain ([Novita] §關鍵技術 2: one pass keeping the
//    running max and the running sum l); the running max is shared by the 4 lanes that hold
//    one head's column (two cross-lane exchanges per pair of units).
//  * Masked tokens get weight exactly 0 by selection, and their V elements are zeroed before
//    the product, so stale or NaN memory past the context never leaks in ([OVAL] §3.2:
//    never read uninitialised memory past the cache length).
//  * Waves merge through LDS; the workgroup writes (o, m, l) of its partition, or the final
//    normalised row when the whole sequence is one partition.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_plan.h"

namespace pkv {

template <class DT, int D>
struct UnitBuf {
    static constexpr int NC = D / (4 * DT::kE);
    u32x4 k[NC], v[NC];
    int t0;    // first logical token, -1 = no unit
    int slot;  // the wave's unit number (unit u_begin + w + slot * kWaves)
};

// Issues the loads of this wave's unit number k (its descriptor sits in lane k), whether or not
// there is such a unit: an empty resource reads zeros and touches no memory. With no branch
// around the loads the compiler counts exactly how many are younger than the ones a pair of
// units waits for, so a wave keeps both pairs in flight (at two waves per SIMD this measured
// faster than the conservative count a branch leaves: page-selected MHA-7B step 26.8 -> 25.9 us).
template <class DT, int D>
__device__ __forceinline__ void load_unit(const DecodeParams& p, UnitBuf<DT, D>& ub, int my_tok,
                                          unsigned my_off, int k, int nk, int lane) {
    constexpr int NC = D / (4 * DT::kE);
    const bool live = k < nk && __builtin_amdgcn_readlane(my_tok, k < nk ? k : 0) >= 0;
    ub.t0 = live ? __builtin_amdgcn_readlane(my_tok, k) : -1;
    ub.slot = k;
    const size_t off = live ? (size_t)(unsigned)__builtin_amdgcn_readlane((int)my_off, k) * 16 : 0;
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(p.k_cache + off, live ? NC * 1024 : 0);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(p.v_cache + off, live ? NC * 1024 : 0);
    const unsigned lane_off = (unsigned)lane * 16u;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) ub.k[cc] = load16_tile_stream(kr, lane_off + cc * 1024);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) ub.v[cc] = load16_tile_stream(vr, lane_off + cc * 1024);
}

// FUSED (one-kernel path only): the step's new token enters attention from k_new/v_new,
// patched into the tile that holds position L-1, and the workgroup stores it to the cache
// after its own reads; no other workgroup reads that (sequence, kv head) row.
// SCORES (one-kernel path only): score export. Each unit's masked log2-domain logits are
// staged in LDS as they are computed; once the merge has the rows' normalisers, the
// workgroup adds each entry's softmax mass to the caller's score row of its (sequence,
// kv head), one thread per entry, in the same order as the work-split path's score kernels.
template <class DT, int D, int MODE, bool DIRECT, bool FUSED, bool SCORES>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_kernel(DecodeParams p) {
    static_assert(DIRECT || !FUSED, "the fused append needs the whole sequence in one workgroup");
    static_assert(DIRECT || !SCORES, "score export needs the whole sequence in one workgroup");
    using T = Tile<DT, D / (4 * DT::kE)>;
    constexpr int NC = D / (4 * DT::kE);
    constexpr int NACC = T::kAcc;
    __shared__ float s_m[kWaves][kMaxGroup];
    __shared__ float s_l[kWaves][kMaxGroup];
    __shared__ __attribute__((aligned(16))) float s_o[kWaves][kMaxGroup][D + 4];
    __shared__ float s_lg[SCORES ? kDirectMaxUnits : 1][kMaxGroup][16];  // [unit][head][token]
    __shared__ float s_lse2[kMaxGroup];

    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane >> 4, c = lane & 15;
    const int G = p.group;

    const int u_begin = split * p.units_per_split;
    // Page list: the lane's entry does not depend on the context length, so it is requested
    // together with it (one round trip before the block-table read instead of two).
    // The load is unconditional (a lane past the list reads entry 0 and drops it): a load
    // under a branch made the compiler wait for it before requesting the length.
    const int L_b = p.context_lens[b];
    int pg_lane = -1;
    if constexpr (MODE == kPages) {
        const int k = (u_begin + w + lane * kWaves) / (p.block_size >> 4);
        const int pg = p.page_list[(size_t)b * p.pages_per_seq + (k < p.pages_per_seq ? k : 0)];
        pg_lane = k < p.pages_per_seq ? pg : -1;
    }
    const SeqPlan sp = make_plan_len<MODE>(p, L_b);
    int u_end = u_begin + p.units_per_split;
    if (u_end > sp.n_units) u_end = sp.n_units;

    if (u_begin >= u_end) {  // empty partition
        if constexpr (FUSED)
            if (w == kWaves - 1) write_new_row<DT::kBytes, D>(p, b * p.kv_heads + kvh, lane);
        if (DIRECT) {
            for (int idx = tid; idx < G * D; idx += 64 * kWaves) {
                const int g = idx / D, x = idx - g * D;
                const size_t h = (size_t)b * p.q_heads + kvh * G + g;
                store_out(p.out, p.out_dtype, h * D + x, 0.f);
                if (x == 0 && p.lse) p.lse[h] = kNegInf;
            }
        } else if (tid < G) {
            const size_t r = ((size_t)b * p.q_heads + kvh * G + tid) * p.num_splits + split;
            p.m_part[r] = kNegInf;
            p.l_part[r] = 0.f;
        }
        return;
    }

    // Descriptors of this wave's units, one per lane: unit u_begin + w + k * kWaves in lane k.
    const int span = u_end - u_begin;
    const int nk = span > w ? (span - w + kWaves - 1) / kWaves : 0;
    int my_tok = -1;
    unsigned my_off = 0;
    if (lane < nk) {
        const int u = u_begin + w + lane * kWaves;
        int t0;
        if constexpr (MODE == kPages) {  // unit_token's page-list case, from the entry read above
            const int per = p.block_size >> 4;
            const int64_t tp = (int64_t)pg_lane * p.block_size + (int64_t)(u - (u / per) * per) * 16;
            t0 = pg_lane >= 0 && tp < sp.L ? (int)tp : -1;
        } else {
            t0 = unit_token<MODE>(p, sp, b, u);
        }
        if (t0 >= 0) {
            const int phys = p.block_table[(size_t)b * p.max_blocks + table_col(p, t0 / p.block_size)];
            if (phys >= 0 && phys < p.num_blocks) {
                const size_t elem = (((size_t)phys * p.kv_heads + kvh) * p.block_size + (t0 % p.block_size)) * D;
                my_off = (unsigned)(elem * DT::kBytes / 16);
                my_tok = t0;
            } else {
                report(p.err, kDevBlockId);  // the unit is skipped
            }
        }
    }

    // Q^T operand: lane (j, c) holds head (c % 8)'s dims [kk*4E + j*E, +E) for chunk group kk.
    const int qhead = c & 7;
    u32x4 q[NC];
#pragma unroll
    for (int kk = 0; kk < NC; ++kk) q[kk] = u32x4{0u, 0u, 0u, 0u};
    if (qhead < G) {
        const char* qp = p.q + (((size_t)b * p.q_heads + kvh * G + qhead) * D + j * DT::kE) * DT::kBytes;
#pragma unroll
        for (int kk = 0; kk < NC; ++kk) q[kk] = load16(qp + kk * 4 * DT::kE * DT::kBytes);
    }

    float m_run = kNegInf, l_run = 0.f;
    f32x4 acc[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[a] = zero4();

    NewRow<DT, D> nrow;
    // the token this step appends (past every attended unit when the length was clamped)
    const int t_new = L_b - 1;
    if constexpr (FUSED) load_new_row<DT, D>(p, nrow, b, kvh, j, c);

    const float qk_scale = p.qk_scale_log2;
    const bool upper = c >= 8;
    auto process = [&](UnitBuf<DT, D>& X, UnitBuf<DT, D>& Y) __attribute__((always_inline)) {
        if constexpr (FUSED) {
            if ((unsigned)(t_new - X.t0) < 16u) patch_tile<DT, D>(X.k, X.v, nrow, t_new - X.t0, j, c);
            if ((unsigned)(t_new - Y.t0) < 16u) patch_tile<DT, D>(Y.k, Y.v, nrow, t_new - Y.t0, j, c);
        }
        f32x4 s0 = zero4(), s1 = zero4();
        T::qk(s0, X.k, q);
        T::qk(s1, Y.k, q);
        const unsigned keep0 = token_keep(sp, X.t0, j);
        const unsigned keep1 = token_keep(sp, Y.t0, j);
        float x0[4], x1[4];
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x0[i] = (keep0 >> i) & 1 ? s0[i] * qk_scale : kNegInf;
            x1[i] = (keep1 >> i) & 1 ? s1[i] * qk_scale : kNegInf;
            mx = fmaxf(mx, fmaxf(x0[i], x1[i]));
        }
        if constexpr (SCORES) {
            // lanes c < 8 hold the first copy of head c's column: tokens 4j .. 4j+3 of the unit.
            // A unit skipped for an invalid block id (t0 = -1) stages -inf logits (keep = 0), so
            // the score phase, which takes the unit's tokens from the plan, adds nothing for it.
            const int ux = w + X.slot * kWaves, uy = w + Y.slot * kWaves;
            if (c < 8 && c < G) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (ux < kDirectMaxUnits) s_lg[ux][c][4 * j + i] = x0[i];
                    if (uy < kDirectMaxUnits) s_lg[uy][c][4 * j + i] = x1[i];
                }
            }
        }
        mx = xor32_max(xor16_max(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        f32x4 p0, p1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p0[i] = __builtin_amdgcn_exp2f(x0[i] - m_use);
            p1[i] = __builtin_amdgcn_exp2f(x1[i] - m_use);
        }
        l_run = l_run * alpha + ((p0.x + p0.y) + (p0.z + p0.w)) + ((p1.x + p1.y) + (p1.z + p1.w));
        // after the first units the running max rarely moves: when no lane's did (alpha = 1
        // everywhere) the accumulators are left as they are
        if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
#pragma unroll
            for (int a = 0; a < NACC; ++a) acc[a] *= alpha;
        }
        if (!unit_full(sp, X.t0)) T::mask_v(X.v, keep0);
        if (!unit_full(sp, Y.t0)) T::mask_v(Y.v, keep1);
        T::pv(acc, X.v, p0, upper);
        T::pv(acc, Y.v, p1, upper);
        m_run = m_new;
    };

    UnitBuf<DT, D> A0, A1, B0, B1;
    load_unit<DT, D>(p, A0, my_tok, my_off, 0, nk, lane);
    load_unit<DT, D>(p, A1, my_tok, my_off, 1, nk, lane);
    for (int k = 0; k < nk; k += 4) {
        load_unit<DT, D>(p, B0, my_tok, my_off, k + 2, nk, lane);
        load_unit<DT, D>(p, B1, my_tok, my_off, k + 3, nk, lane);
        process(A0, A1);
        if (k + 2 >= nk) break;
        load_unit<DT, D>(p, A0, my_tok, my_off, k + 4, nk, lane);
        load_unit<DT, D>(p, A1, my_tok, my_off, k + 5, nk, lane);
        process(B0, B1);
    }

    // The 4 lanes of one column hold partial sums of the same head under the same max.
    l_run = xor32_sum(xor16_sum(l_run));
    const int head = T::acc_head(c);
    if (j == 0 && c < 8 && head < G) {
        s_m[w][head] = m_run;
        s_l[w][head] = l_run;
    }
    if (head < G && T::acc_owner(c)) {
#pragma unroll
        for (int a = 0; a < NACC; ++a) *reinterpret_cast<f32x4*>(&s_o[w][head][T::acc_dim(a, j, c)]) = acc[a];
    }
    __syncthreads();
    // every wave's loads have returned: the segment's row can take the new token
    if constexpr (FUSED)
        if (w == kWaves - 1) write_new_row<DT::kBytes, D>(p, b * p.kv_heads + kvh, lane);

    for (int idx = tid; idx < G * D; idx += 64 * kWaves) {
        const int g = idx / D, x = idx - g * D;
        float M = kNegInf;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][g]);
        float Ls = 0.f, O = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float mw = s_m[ww][g];
            const float sc = mw == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            Ls += s_l[ww][g] * sc;
            O += s_o[ww][g][x] * sc;
        }
        const size_t h = (size_t)b * p.q_heads + kvh * G + g;
        if (DIRECT) {
            store_out(p.out, p.out_dtype, h * D + x, Ls > 0.f ? O / Ls : 0.f);
            if (x == 0 && p.lse) p.lse[h] = Ls > 0.f ? M * kLn2 + logf(Ls) : kNegInf;
            if constexpr (SCORES)
                if (x == 0) s_lse2[g] = Ls > 0.f ? M + __log2f(Ls) : kNegInf;
        } else {
            const size_t r = h * p.num_splits + split;
            p.o_part[r * D + x] = O;
            if (x == 0) {
                p.m_part[r] = Ls > 0.f ? M * kLn2 : kNegInf;
                p.l_part[r] = Ls;
            }
        }
    }

    if constexpr (SCORES) {
        __syncthreads();  // the rows' normalisers
        float l2[kMaxGroup];
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) l2[g] = g < G ? s_lse2[g] : 0.f;
        // softmax mass of the 16 tokens of staged unit u, the heads summed in order; a masked
        // logit (-inf) adds exactly 0, also in a row whose normaliser is -inf (no token of it
        // was read), where the difference would be NaN
        auto unit_mass = [&](int u, float (&m)[16]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) m[i] = 0.f;
#pragma unroll
            for (int g = 0; g < kMaxGroup; ++g)
                if (g < G) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) m[i] += prob2(s_lg[u][g][i], l2[g]);
                }
        };
        const int nu = sp.n_units < kDirectMaxUnits ? sp.n_units : kDirectMaxUnits;
        float* row = p.score + (size_t)(b * p.kv_heads + kvh) * p.score_stride;
        if (p.score_block <= 1) {
            // one entry per attended token
            for (int idx = tid; idx < nu * 16; idx += 64 * kWaves) {
                const int u = idx >> 4, i = idx & 15;
                const int t0 = unit_token<MODE>(p, sp, b, u);
                const int t = t0 + i;
                if (t0 < 0 || !(t < sp.L && (t < sp.e0 || t >= sp.s1))) continue;
                float mass = 0.f;
#pragma unroll
                for (int g = 0; g < kMaxGroup; ++g)
                    if (g < G) mass += prob2(s_lg[u][g][i], l2[g]);
                row[t] += mass;
            }
        } else if (MODE == kPages) {
            // one entry per listed page (score_block == block_size): list entry kk holds units
            // kk * P/16 .. (kk + 1) * P/16 - 1, and its entry is the page id
            const int per = p.block_size >> 4;
            for (int kk = tid; kk < p.pages_per_seq; kk += 64 * kWaves) {
                const int pg = p.page_list[(size_t)b * p.pages_per_seq + kk];
                if (pg < 0 || (long long)pg * p.block_size >= sp.L) continue;
                float accs = 0.f;
                for (int cc = 0; cc < per; ++cc) {
                    const int c0 = pg * p.block_size + 16 * cc;
                    const int u = kk * per + cc;
                    if (c0 >= sp.L || u >= nu) break;
                    float m[16];
                    unit_mass(u, m);
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (c0 + i < sp.L) accs += m[i];
                }
                row[pg] += accs;
            }
        } else {
            // entries of score_block tokens over the attended token ranges
            const int B = p.score_block;
            const int n_ent = (sp.L + B - 1) / B;
            for (int e = tid; e < n_ent; e += 64 * kWaves) {
                const int t_lo = e * B;
                const int t_hi = (e + 1) * B < sp.L ? (e + 1) * B : sp.L;
                float accs = 0.f;
                bool any = false;
                for (int c0 = t_lo & ~15; c0 < t_hi; c0 += 16) {
                    const int cu = c0 >> 4;
                    int u = cu;
                    if (MODE == kWindow) u = cu < sp.n0 ? cu : (cu >= sp.u1a ? sp.n0 + (cu - sp.u1a) : -1);
                    if (u < 0 || u >= nu) continue;
                    float m[16];
                    unit_mass(u, m);
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int t = c0 + i;
                        if (t >= t_lo && t < t_hi && (MODE != kWindow || t < sp.e0 || t >= sp.s1)) {
                            accs += m[i];
                            any = true;
                        }
                    }
                }
                if (any) row[e] += accs;
            }
        }
    }
}

// Cross-split combine: one wavefront per (sequence, query head) row.
__global__ __launch_bounds__(64) void combine_kernel(CombineParams p) {
    const int r = blockIdx.x;
    const int lane = threadIdx.x;
    const int S = p.num_splits, D = p.head_dim;
    const float* mr = p.m_part + (size_t)r * S;
    const float* lr = p.l_part + (size_t)r * S;
    float M = kNegInf;
    for (int s = 0; s < S; ++s)
        if (lr[s] > 0.f) M = fmaxf(M, mr[s]);
    float Ls = 0.f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};  // D <= 256
    for (int s = 0; s < S; ++s) {
        const float l = lr[s];
        if (!(l > 0.f)) continue;
        const float wgt = expf(mr[s] - M);
        Ls += wgt * l;
        const float* op = p.o_part + ((size_t)r * S + s) * D;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (lane + 64 * e < D) o[e] += wgt * op[lane + 64 * e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int x = lane + 64 * e;
        if (x < D) store_out(p.out, p.out_dtype, (size_t)r * D + x, M == kNegInf ? 0.f : o[e] / Ls);
    }
    if (lane == 0 && p.lse) p.lse[r] = M == kNegInf ? kNegInf : M + logf(Ls);
}

template <class DT, int D, int MODE>
static hipError_t launch_decode_t(bool direct, const DecodeParams& p, int batch, hipStream_t s) {
    const dim3 grid((unsigned)p.num_splits, (unsigned)p.kv_heads, (unsigned)batch);
    const dim3 block(64 * kWaves);
    if (direct) {
        // one partition holding every unit of a segment (with score export, at most
        // kDirectMaxUnits of them: the logits are staged in LDS)
        if (p.num_splits != 1 || (p.score && p.units_per_split > kDirectMaxUnits)) return hipErrorInvalidValue;
        if (p.new_slots && p.score)
            decode_split_kernel<DT, D, MODE, true, true, true><<<grid, block, 0, s>>>(p);
        else if (p.new_slots)
            decode_split_kernel<DT, D, MODE, true, true, false><<<grid, block, 0, s>>>(p);
        else if (p.score)
            decode_split_kernel<DT, D, MODE, true, false, true><<<grid, block, 0, s>>>(p);
        else
            decode_split_kernel<DT, D, MODE, true, false, false><<<grid, block, 0, s>>>(p);
    } else {
        if (p.new_slots || p.score) return hipErrorInvalidValue;
        decode_split_kernel<DT, D, MODE, false, false, false><<<grid, block, 0, s>>>(p);
    }
    return hipGetLastError();
}

template <class DT, int D>
static hipError_t launch_decode_m(int mode, bool direct, const DecodeParams& p, int batch, hipStream_t s) {
    switch (mode) {
        case kWindow: return launch_decode_t<DT, D, kWindow>(direct, p, batch, s);
        case kPages: return launch_decode_t<DT, D, kPages>(direct, p, batch, s);
        default: return launch_decode_t<DT, D, kFull>(direct, p, batch, s);
    }
}

template <class DT>
static hipError_t launch_decode_d(int head_dim, int mode, bool direct, const DecodeParams& p, int batch,
                                  hipStream_t s) {
    return head_dim == 64 ? launch_decode_m<DT, 64>(mode, direct, p, batch, s)
                          : launch_decode_m<DT, 128>(mode, direct, p, batch, s);
}

hipError_t launch_decode(int dtype, int head_dim, int mode, bool direct, const DecodeParams& p, int batch,
                         hipStream_t s) {
    if (batch <= 0 || p.num_splits <= 0) return hipSuccess;
    switch (dtype) {
        case kF32: return launch_decode_d<F32>(head_dim, mode, direct, p, batch, s);
        case kF16: return launch_decode_d<F16>(head_dim, mode, direct, p, batch, s);
        case kI8B:
        case kI8H: return hipErrorInvalidValue;  // INT8 caches take the stream path only
        default: return launch_decode_d<BF16>(head_dim, mode, direct, p, batch, s);
    }
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
    if (p.rows <= 0) return hipSuccess;
    combine_kernel<<<dim3((unsigned)p.rows), dim3(64), 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace pkv
