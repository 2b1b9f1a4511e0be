// stream.hip — persistent ("stream-K") paged decode attention and its combine.
//
// The computation is the one described in decode.hip (softmax(q K^T * scale) V over the paged
// cache, [TF] formula, [primer] §4.1 block table, [primer] §4.3 / [Novita] §關鍵技術 1 window,
// [OVAL] §2.2/§3.3 page list); what differs is how the work is cut.
//
// All (sequence, kv head) segments of the batch are laid end to end as one flat list of
// 16-token units, b-major then kv head then unit. The launch holds exactly the waves that
// are resident on the GPU at once; wave w takes the contiguous units [w*C, (w+1)*C) with
// C = max(ceil(N / waves), chunk_min), so every wave streams the same number of bytes no
// matter how ragged the context lengths are, and no wave waits for a second launch round.
// A wave streams its units through a small ring of register buffers (2-deep for 2- and 4-byte
// caches, 3-deep for INT8), refilled at every segment boundary. At the end of its part of a
// segment it writes either the finished, normalised row (when it holds the whole segment) or an
// (o, m, l) partial: piece k = w - first_wave(segment) goes to the segment's own slot k when
// k < kSegSlots, else to wave w's overflow slot (a piece k >= 1 is the first run of its wave,
// so a wave fills at most one overflow slot). The wave holding a segment's last unit records
// the piece count and the first wave. The combine kernel then merges the pieces by
// log-sum-exp ([Novita] §關鍵技術 2: partial softmax results merge through max and sum): one
// round trip covers the first 8, 12 or 16 pieces, a second the rest of the segment's own slots and
// up to kCombineWide overflow pieces, and each later one kCombineWide more.
// Workspace rows: (B * Hkv * kSegSlots + waves) x G, whatever the context lengths.
// In the fused decode step (FUSED) the run that reaches a segment's newest position takes the
// new token from k_new / v_new in registers and patches it into the sub-tile that holds it (on
// an INT8 cache after quantising it in the kernel exactly as the append would store it); the
// combine's extra workgroups store the new rows once every read of them has returned.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_plan.h"
#include "pkv_q8.h"

namespace pkv {

template <int MODE>
__device__ __forceinline__ int seq_units(const DecodeParams& p, int b) {
    return make_plan<MODE>(p, b).n_units;
}

// Position of a unit: sequence, kv head, unit index within the sequence.
struct UnitPos {
    int b, kvh, u, nu;
};

// Advances a position by k units (k >= 0), skipping sequences without units (units_of(b):
// the units of sequence b). Returns b == batch when it runs off the end.
template <class UnitsOf>
__device__ __forceinline__ UnitPos advance(const DecodeParams& p, UnitPos s, int k, UnitsOf units_of) {
    while (s.b < p.batch) {
        const int rem = s.nu - s.u;
        if (k < rem) {
            s.u += k;
            return s;
        }
        k -= rem;
        s.u = 0;
        if (++s.kvh == p.kv_heads) {
            s.kvh = 0;
            do {
                ++s.b;
            } while (s.b < p.batch && (s.nu = units_of(s.b)) == 0);
        }
    }
    return s;
}

template <class DT, int D>
struct RingBuf {
    static constexpr int NC = D / (4 * DT::kE);
    u32x4 k[NC], v[NC];
    f32x4 ks, vs;  // INT8 caches: row scales of the lane's tokens 4j..4j+3 (K, V)
    int t0;
    int u;  // unit index within the segment
};

template <class DT, int D>
__device__ __forceinline__ void ring_load(const DecodeParams& p, RingBuf<DT, D>& rb, int my_tok, unsigned my_off,
                                          int k, int n, int lane, int u_base) {
    constexpr int NC = D / (4 * DT::kE);
    if constexpr (!DT::kQ8) {
        // 2- and 4-byte caches: global loads under a branch. At the branch joins the
        // compiler's count of loads in flight is conservative, so before a unit is processed
        // the wave waits for all but the newest unit's loads: about one unit in flight per
        // wave, 8 MiB over the chip at the benchmark shape. Counting exactly (the INT8 form
        // below) keeps the whole ring in flight and measured slower at the Llama-3-8B layer
        // shape (step 61.7 -> 64.1 us with a 4-deep ring, 63.1 us with a 2-deep one): more
        // bytes in flight only queue.
        const int t0 = k < n ? __builtin_amdgcn_readlane(my_tok, k) : -1;
        rb.t0 = t0;
        rb.u = u_base + k;
        if (t0 >= 0) {
            const size_t off = (size_t)(unsigned)__builtin_amdgcn_readlane((int)my_off, k) * 16;
            const char* kp = p.k_cache + off + lane * 16;
            const char* vp = p.v_cache + off + lane * 16;
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) rb.k[cc] = load16_stream(kp + cc * 1024);
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) rb.v[cc] = load16_stream(vp + cc * 1024);
        }
    } else {
        // INT8: the loads are issued whether or not the slot holds a unit (an empty resource
        // reads zeros and touches no memory). With no branch around them the compiler counts
        // exactly how many loads are younger than the ones a unit waits for, and a wave keeps
        // the whole ring in flight; the widening work per unit then hides behind the loads.
        const bool live = k < n && __builtin_amdgcn_readlane(my_tok, k < n ? k : 0) >= 0;
        rb.t0 = live ? __builtin_amdgcn_readlane(my_tok, k) : -1;
        rb.u = u_base + k;
        const size_t off = live ? (size_t)(unsigned)__builtin_amdgcn_readlane((int)my_off, k) * 16 : 0;
        const __amdgpu_buffer_rsrc_t kr = tile_rsrc(p.k_cache + off, live ? NC * 1024 : 0);
        const __amdgpu_buffer_rsrc_t vr = tile_rsrc(p.v_cache + off, live ? NC * 1024 : 0);
        const unsigned lane_off = (unsigned)lane * 16u;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) rb.k[cc] = load16_tile_stream(kr, lane_off + cc * 1024);
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) rb.v[cc] = load16_tile_stream(vr, lane_off + cc * 1024);
        // scale plane after the data plane; the sub-tile's first row is off / D, and lane
        // (j, c) takes rows 4j .. 4j+3
        const size_t plane = (size_t)p.num_blocks * p.kv_heads * p.block_size * D;
        const size_t srow = off / D;
        const __amdgpu_buffer_rsrc_t ksr = tile_rsrc(p.k_cache + plane + srow * 4, live ? 64 : 0);
        const __amdgpu_buffer_rsrc_t vsr = tile_rsrc(p.v_cache + plane + srow * 4, live ? 64 : 0);
        rb.ks = __builtin_bit_cast(f32x4, load16_tile(ksr, (unsigned)(lane >> 4) * 16u));
        rb.vs = __builtin_bit_cast(f32x4, load16_tile(vsr, (unsigned)(lane >> 4) * 16u));
    }
}

// Score export: each wave stages the logits of its current run in 16 KiB of LDS and stores
// them in contiguous full-wave bursts (a 16-lane store per unit cost about three times as
// much at the benchmark shape). 16 KiB holds a whole share at the Llama-3-8B layer shape, so
// the stores leave at the end of the run: stores count in the same in-order counter as loads,
// and a burst in mid-run made the next tile's wait cover it too (4 KiB: step 75.3 us, 16 KiB:
// 70.5 us).
constexpr int kLgFloats = 4096;

template <class DT, int D, int MODE, bool FUSED, bool SCORES>
__global__ __launch_bounds__(64 * kStreamWaves) __attribute__((amdgpu_waves_per_eu(2)))
void decode_stream_kernel(DecodeParams p) {
    using TI = typename DT::In;               // q type
    using TM = typename DT::Mma;              // MFMA operand type
    static_assert(TI::kE == TM::kE, "q chunks and operand chunks line up");
    constexpr int NC = D / (4 * TI::kE);      // operand chunks per lane (q, widened K/V)
    constexpr int NCC = D / (4 * DT::kE);     // cache chunks per lane (K, V)
    using T = Tile<TM, NC>;
    constexpr int NACC = T::kAcc;
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * kStreamWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane >> 4, c = lane & 15;
    const int B = p.batch, Hkv = p.kv_heads, G = p.group;

    // Context lengths of the first 64 sequences, one per lane, are read once: the work split,
    // every run's plan and the step to the next sequence take them from here by readlane
    // (sequences past 64 are read from memory).
    const int L_lane = lane < B ? p.context_lens[lane] : 0;
    auto len_of = [&](int b) -> int {  // b is wave-uniform
        return b < 64 ? __builtin_amdgcn_readlane(L_lane, b) : p.context_lens[b];
    };
    // Flat positions of a segment: its units plus `lead` virtual ones in front, which stand
    // for the set-up of a run (query and descriptors fetched, load ring refilled). A wave whose
    // share takes a segment's start therefore streams that many fewer units, and shares that
    // cross segment boundaries take as long as those that do not.
    const int lead = p.seg_lead;
    auto flat_of = [&](int nu) -> int { return nu > 0 ? nu + lead : 0; };
    auto units_of = [&](int b) -> int { return flat_of(make_plan_len<MODE>(p, len_of(b)).n_units); };

    // Total flat positions N of the batch (uniform: kept in scalar registers). The first 64
    // sequences' inclusive scan gives their total and also serves the search for the wave's
    // first position.
    const int nu_lane = lane < B ? flat_of(make_plan_len<MODE>(p, L_lane).n_units) : 0;
    const int incl_lane = wave_incl_scan(nu_lane * Hkv);
    int N = __builtin_amdgcn_readlane(incl_lane, 63);
    for (int b0 = 64; b0 < B; b0 += 64) {
        const int b = b0 + lane;
        N += __builtin_amdgcn_readfirstlane(wave_sum(b < B ? flat_of(seq_units<MODE>(p, b)) : 0)) * Hkv;
    }
    const int W = p.waves_total;
    int C = (N + W - 1) / W;
    if (C < p.chunk_min) C = p.chunk_min;
    if ((long long)wave * C >= N) return;
    const int f_begin = wave * C;
    const int f_end = (long long)f_begin + C < N ? f_begin + C : N;

    // Locate the first position: the sequence whose flat positions (times Hkv) cover f_begin.
    UnitPos pos = {B, 0, 0, 0};
    {
        int cum = 0;
        for (int b0 = 0; b0 < B; b0 += 64) {
            const int b = b0 + lane;
            const int nu = b0 == 0 ? nu_lane : (b < B ? flat_of(seq_units<MODE>(p, b)) : 0);
            const int incl = b0 == 0 ? incl_lane : wave_incl_scan(nu * Hkv);
            const int chunk_total = __builtin_amdgcn_readlane(incl, 63);
            if (cum + chunk_total > f_begin) {
                const unsigned long long hit = __ballot(cum + incl > f_begin);
                const int lf = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
                const int nu_b = __builtin_amdgcn_readlane(nu, lf);
                const int before = cum + __builtin_amdgcn_readlane(incl, lf) - nu_b * Hkv;
                const int rem = f_begin - before;
                pos.b = b0 + lf;
                pos.kvh = rem / nu_b;
                pos.u = rem - pos.kvh * nu_b;
                pos.nu = nu_b;
                break;
            }
            cum += chunk_total;
        }
    }

    // The wave's range, cut at segment boundaries into runs; each run is one (sequence,
    // kv head) segment piece with its own query, softmax state and load pipeline.
    const int qhead = c & 7;
    const bool upper = c >= 8;
    __shared__ float lg_stage[kStreamWaves * (SCORES ? kLgFloats : 1)];
    float* lgb = lg_stage + (SCORES ? (threadIdx.x >> 6) * kLgFloats : 0);
    // INT8 fused step: each wave's stage for dealing out the new row's codes
    __shared__ __attribute__((aligned(16))) unsigned char q8_stage[kStreamWaves][FUSED && DT::kQ8 ? 2 * D : 16];
    const float qk_scale = p.qk_scale_log2;
    int f_run = f_begin;
    while (f_run < f_end && pos.b < B) {
        // pos.u / pos.nu: flat positions within the segment; real units are u0 .. u0 + cnt
        const int b = pos.b, kvh = pos.kvh, v0 = pos.u, nv = pos.nu;
        const int cntv = f_end - f_run < nv - v0 ? f_end - f_run : nv - v0;
        const int nu = nv - lead;
        const int u0 = v0 > lead ? v0 - lead : 0;
        const int cnt = (v0 + cntv > lead ? v0 + cntv - lead : 0) - u0;
        // cnt == 0 (the share holds only virtual positions of this segment) leaves an empty
        // piece, l = 0, which the combine skips; it is never the segment's last piece
        const int seg = b * Hkv + kvh;
        const int L_b = len_of(b);
        const SeqPlan sp = make_plan_len<MODE>(p, L_b);

        u32x4 q[NC];
#pragma unroll
        for (int kk = 0; kk < NC; ++kk) q[kk] = u32x4{0u, 0u, 0u, 0u};
        if (qhead < G) {
            const char* qrow = p.q + ((size_t)b * p.q_heads + kvh * G + qhead) * D * TI::kBytes;
            if constexpr (DT::kQ8) {
                // widened INT8 chunk m of lane group j holds dims 64m + 16j .. +15: operand
                // chunks 2m and 2m + 1 take q's dims 64m + 16j .. +7 and .. +15
#pragma unroll
                for (int kk = 0; kk < NC; ++kk) {
                    q[kk] = load16(qrow + ((kk >> 1) * 64 + 16 * j + 8 * (kk & 1)) * TI::kBytes);
                    if constexpr (!__is_same(TI, TM)) {  // a bf16 query for fp16 MFMAs
#pragma unroll
                        for (int w = 0; w < 4; ++w) q[kk][w] = bf16x2_to_f16x2(q[kk][w]);
                    }
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < NC; ++kk) q[kk] = load16(qrow + (kk * 4 * TI::kE + j * TI::kE) * TI::kBytes);
            }
        }
        // INT8: the widened K carries kI8Bias on every element, so a logit comes out high by
        // kI8Bias * sum_d q[d] for its head: the fp16 query as the products take it, summed
        // over the lane's dims and then over the 4 lanes of the head's column.
        float qbias = 0.f;
        if constexpr (DT::kQ8) {
            float qs = 0.f;
#pragma unroll
            for (int kk = 0; kk < NC; ++kk) {
#pragma unroll
                for (int w = 0; w < 4; ++w) qs += f16_lo_f32(q[kk][w]) + f16_hi_f32(q[kk][w]);
            }
            qbias = kI8Bias * xor32_sum(xor16_sum(qs));
        }
        float m_run = kNegInf, l_run = 0.f;
        float pv_run = 0.f;  // INT8: running sum of the P operand (p times V's row scale)
        f32x4 acc[NACC];
#pragma unroll
        for (int a = 0; a < NACC; ++a) acc[a] = zero4();
        NewRow<TI, D> nrow;
        NewRowRaw<D> nraw;  // INT8: the new row as loaded, quantised into nq once the ring is primed
        NewRowQ8<D> nq;
        // the token this step appended (past every attended unit when the length was clamped)
        const int t_new = L_b - 1;
        if constexpr (FUSED) {
            if constexpr (DT::kQ8)
                load_new_row_raw<D>(p, nraw, b, kvh, lane);
            else
                load_new_row<TI, D>(p, nrow, b, kvh, j, c);
        }

        // score export: the run's logits are staged in LDS and stored in contiguous bursts
        int lg_n = 0, lg_u0 = u0;
        auto flush = [&]() __attribute__((always_inline)) {
            const int nf = lg_n * G * 16;
            float* dst = p.logits + ((size_t)seg * p.units_bound + lg_u0) * G * 16;
            for (int i = lane * 4; i < nf; i += 256)
                *reinterpret_cast<f32x4*>(dst + i) = *reinterpret_cast<const f32x4*>(lgb + i);
            lg_u0 += lg_n;
            lg_n = 0;
        };
        // One unit: kt / vt are the MFMA operands (the ring buffer's own chunks, or for an
        // INT8 cache their exact widening).
        auto unit = [&](RingBuf<DT, D>& rb, u32x4 (&kt)[NC], u32x4 (&vt)[NC]) __attribute__((always_inline)) {
            f32x4 s = zero4();
            T::qk(s, kt, q);
            const unsigned keep = token_keep(sp, rb.t0, j);
            float x[4];
            float mx = kNegInf;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float si = DT::kQ8 ? (s[i] - qbias) * rb.ks[i] : s[i];  // dequantised logit
                x[i] = (keep >> i) & 1 ? si * qk_scale : kNegInf;
                mx = fmaxf(mx, x[i]);
            }
            if constexpr (SCORES) {
                // score export: the unit's masked logits of head c (tokens 4j .. 4j+3)
                if (c < G) *reinterpret_cast<f32x4*>(lgb + (lg_n * G + c) * 16 + 4 * j) = f32x4{x[0], x[1], x[2], x[3]};
                ++lg_n;
            }
            mx = xor32_max(xor16_max(mx));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == kNegInf ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            f32x4 pr;
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(x[i] - m_use);
            l_run = l_run * alpha + ((pr.x + pr.y) + (pr.z + pr.w));
            // after the first units the running max rarely moves: when no lane's did (alpha = 1
            // everywhere) the accumulators are left as they are
            if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
#pragma unroll
                for (int a = 0; a < NACC; ++a) acc[a] *= alpha;
            }
            if constexpr (DT::kQ8) {
                // V's row scales enter through P (a masked token's scale is never multiplied).
                // A masked token's P is 0 and its widened V finite, so its V needs no masking.
                f32x4 pv;
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[i] = (keep >> i) & 1 ? pr[i] * rb.vs[i] : 0.f;
                pv_run = pv_run * alpha + ((pv.x + pv.y) + (pv.z + pv.w));
                T::pv(acc, vt, pv, upper);
            } else {
                if (!unit_full(sp, rb.t0)) T::mask_v(vt, keep);
                T::pv(acc, vt, pr, upper);
            }
            m_run = m_new;
        };
        auto process = [&](RingBuf<DT, D>& rb) __attribute__((always_inline)) {
            if constexpr (SCORES) {
                if ((lg_n + 1) * G * 16 > kLgFloats) flush();
                if (rb.t0 < 0) {
                    // no unit, or one skipped for an invalid block id: its slot holds -inf
                    // logits, which the score kernels turn into exactly 0
                    if (c < G)
                        *reinterpret_cast<f32x4*>(lgb + (lg_n * G + c) * 16 + 4 * j) =
                            f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
                    ++lg_n;
                    return;
                }
            }
            if (rb.t0 < 0) return;
            if constexpr (DT::kQ8) {
                if constexpr (FUSED) {
                    // the unit holding the new token: its row quantised as the append would store
                    // it, patched in over the cache's stale bytes and scales
                    // (one unit per segment: the patch is laid out away from the unit loop)
                    if (__builtin_expect((unsigned)(t_new - rb.t0) < 16u, 0))
                        patch_tile_q8<D>(rb.k, rb.v, rb.ks, rb.vs, nq, t_new - rb.t0, j, c);
                }
                u32x4 kt[NC], vt[NC];
#pragma unroll
                for (int m = 0; m < NCC; ++m) {
                    widen_i8_f16_biased(rb.k[m], kt[2 * m], kt[2 * m + 1]);
                    widen_i8_f16_biased(rb.v[m], vt[2 * m], vt[2 * m + 1]);
                }
                unit(rb, kt, vt);
            } else {
                if constexpr (FUSED) {
                    if ((unsigned)(t_new - rb.t0) < 16u) patch_tile<TI, D>(rb.k, rb.v, nrow, t_new - rb.t0, j, c);
                }
                unit(rb, rb.k, rb.v);
            }
        };

        for (int ub = 0; ub < cnt; ub += 64) {
            // Descriptor of the batch's unit k in lane k.
            const int n = cnt - ub < 64 ? cnt - ub : 64;
            int my_tok = -1;
            unsigned my_off = 0;
            if (lane < n) {
                const int t0 = unit_token<MODE>(p, sp, b, u0 + ub + lane);
                if (t0 >= 0) {
                    const int phys = p.block_table[(size_t)b * p.max_blocks + table_col(p, t0 / p.block_size)];
                    if (phys >= 0 && phys < p.num_blocks) {
                        const size_t elem = (((size_t)phys * Hkv + kvh) * p.block_size + (t0 % p.block_size)) * D;
                        my_off = (unsigned)(elem * DT::kBytes / 16);
                        my_tok = t0;
                    } else {
                        report(p.err, kDevBlockId);  // the unit is skipped
                    }
                }
            }
            // A ring of register buffers: unit k + depth - 1 is requested right before unit k is
            // processed. 2- and 4-byte caches take depth 2: their loads are counted
            // conservatively (ring_load), so about one unit is in flight per wave either way,
            // and the shallower ring asks for less at once when every wave starts (Llama-3-8B
            // layer step 61.3 -> 60.7 us; depth 3 61.0 us). INT8 caches, counted exactly, take
            // depth 3 (kernel 32.8 us against 33.3 us with depth 4 and 33.1 us with depth 2, now
            // that the widening is a byte permute per two values; more bytes in flight only queue).
            if constexpr (!DT::kQ8) {
                RingBuf<DT, D> R0, R1;
                ring_load<DT, D>(p, R0, my_tok, my_off, 0, n, lane, u0 + ub);
                for (int k = 0; k < n; k += 2) {
                    ring_load<DT, D>(p, R1, my_tok, my_off, k + 1, n, lane, u0 + ub);
                    process(R0);
                    if (k + 1 >= n) break;
                    ring_load<DT, D>(p, R0, my_tok, my_off, k + 2, n, lane, u0 + ub);
                    process(R1);
                }
            } else {
                RingBuf<DT, D> R0, R1, R2;
                ring_load<DT, D>(p, R0, my_tok, my_off, 0, n, lane, u0 + ub);
                ring_load<DT, D>(p, R1, my_tok, my_off, 1, n, lane, u0 + ub);
                // The fused step's new row was requested before the block table, so it has
                // arrived by now: quantised here, with the ring's first two units in flight, it
                // waits for nothing, and only its codes stay live through the run (quantising
                // after the third unit's request measured slower). Only a batch that holds the
                // new token quantises it (one run per segment).
                if constexpr (FUSED) {
                    const bool has_new =
                        __builtin_amdgcn_ballot_w64(lane < n && my_tok >= 0 && (unsigned)(t_new - my_tok) < 16u) != 0;
                    if (has_new) quantise_new_row<TI, D>(nraw, nq, q8_stage[threadIdx.x >> 6], lane, j, c);
                }
                for (int k = 0; k < n; k += 3) {
                    ring_load<DT, D>(p, R2, my_tok, my_off, k + 2, n, lane, u0 + ub);
                    process(R0);
                    if (k + 1 >= n) break;
                    ring_load<DT, D>(p, R0, my_tok, my_off, k + 3, n, lane, u0 + ub);
                    process(R1);
                    if (k + 2 >= n) break;
                    ring_load<DT, D>(p, R1, my_tok, my_off, k + 4, n, lane, u0 + ub);
                    process(R2);
                }
            }
        }

        if constexpr (SCORES) flush();
        // End of the run: the finished row, or a partial for the combine.
        const float l_tot = xor32_sum(xor16_sum(l_run));
        if constexpr (DT::kQ8) {
            // the widened V's offset: every output element of a head is high by kI8Bias times
            // the sum of that head's P operand
            const float vbias = kI8Bias * xor32_sum(xor16_sum(pv_run));
#pragma unroll
            for (int a = 0; a < NACC; ++a) acc[a] -= vbias;
        }
        const int head = T::acc_head(c);
        const bool writer = head < G && T::acc_owner(c);
        const bool last = u0 + cnt == nu;
        if (v0 == 0 && last) {
            const size_t hrow = (size_t)b * p.q_heads + kvh * G + head;
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            if (writer) {
#pragma unroll
                for (int a = 0; a < NACC; ++a) {
                    const int dim = T::acc_dim(a, j, c);
#pragma unroll
                    for (int i = 0; i < 4; ++i) store_out(p.out, p.out_dtype, hrow * D + dim + i, acc[a][i] * inv);
                }
            }
            if (j == 0 && c < 8 && head < G && p.lse)
                p.lse[hrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
            if constexpr (SCORES) {
                if (j == 0 && c < 8 && head < G) p.row_lse2[hrow] = l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf;
            }
            if (lane == 0) p.seg_count[2 * seg] = 0;
        } else {
            const int s_g = f_run - v0;  // flat index of the segment's first position
            const int w0 = s_g / C;      // the wave holding it
            const int k = wave - w0;     // this piece's index within the segment
            const size_t slot = k < kSegSlots ? (size_t)seg * kSegSlots + k
                                              : (size_t)B * Hkv * kSegSlots + wave;
            const size_t row = slot * G + head;
            if (writer) {
#pragma unroll
                for (int a = 0; a < NACC; ++a)
                    *reinterpret_cast<f32x4*>(p.o_part + row * D + T::acc_dim(a, j, c)) = acc[a];
            }
            if (j == 0 && c < 8 && head < G) {
                p.m_part[row] = m_run;  // log2 units, read only by the stream combine
                p.l_part[row] = l_tot;
            }
            if (lane == 0 && last) {
                p.seg_count[2 * seg] = k + 1;
                p.seg_count[2 * seg + 1] = w0;
            }
        }
        f_run += cntv;
        pos = advance(p, pos, cntv, units_of);
        pos.b = __builtin_amdgcn_readfirstlane(pos.b);
        pos.kvh = __builtin_amdgcn_readfirstlane(pos.kvh);
        pos.u = __builtin_amdgcn_readfirstlane(pos.u);
        pos.nu = __builtin_amdgcn_readfirstlane(pos.nu);
    }
}

// A batch of up to KX partials of one row, in consecutive slots G rows apart: lane u holds piece
// u's (m, l) (m in log2 units), every lane its D/64 dims of each piece's o.
template <int KX, int PER>
struct RowBatch {
    float v[KX][PER];
    float m, l;
};

// Requests pieces 0 .. n_load - 1 of a batch starting at row0, all at once, through resources
// that span only those pieces: reads past them return zero and touch no memory.
template <int KX, int D>
__device__ __forceinline__ void load_rows(const DecodeParams& p, RowBatch<KX, D / 64>& rb, size_t row0, int n_load,
                                          int G, int lane) {
    static_assert(KX <= 32, "(m, l) are reduced over lanes 0..31");
    constexpr int PER = D / 64;
    const __amdgpu_buffer_rsrc_t orr =
        tile_rsrc(reinterpret_cast<const char*>(p.o_part + row0 * D), n_load * G * D * 4);
    const __amdgpu_buffer_rsrc_t mr = tile_rsrc(reinterpret_cast<const char*>(p.m_part + row0), n_load * G * 4);
    const __amdgpu_buffer_rsrc_t lr = tile_rsrc(reinterpret_cast<const char*>(p.l_part + row0), n_load * G * 4);
#pragma unroll
    for (int u = 0; u < KX; ++u) load_f32_buf<PER>(orr, (unsigned)((u * G * D + lane * PER) * 4), rb.v[u]);
    rb.m = load4_buf(mr, (unsigned)(lane * G * 4));
    rb.l = load4_buf(lr, (unsigned)(lane * G * 4));
}

// Folds the batch's first n_live pieces, of those the ones that attended a token (l > 0), into
// the row's running (M, Ls, o).
template <int KX, int PER>
__device__ __forceinline__ void merge_rows(float& M, float& Ls, float (&o)[PER], const RowBatch<KX, PER>& rb,
                                           int n_live, int lane) {
    const bool live = lane < n_live && rb.l > 0.f;
    const float bm = __int_as_float(
        __builtin_amdgcn_readfirstlane(__float_as_int(xor16_max(row16_max(live ? rb.m : kNegInf)))));
    const float m_new = fmaxf(M, bm);
    if (m_new == kNegInf) return;
    const float sc = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - m_new);
    const float w_lane = live ? __builtin_amdgcn_exp2f(rb.m - m_new) : 0.f;
    const float lw = __int_as_float(
        __builtin_amdgcn_readfirstlane(__float_as_int(xor16_sum(row16_sum(live ? w_lane * rb.l : 0.f)))));
    Ls = Ls * sc + lw;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] *= sc;
    // pieces past n_live are dropped by selection here and in the sum above, not by a zero
    // weight: a stale slot may hold inf or NaN
#pragma unroll
    for (int u = 0; u < KX; ++u) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), u));
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] += u < n_live ? w * rb.v[u][i] : 0.f;
    }
    M = m_new;
}

// Merges the partials of one (sequence, query head) row per 64-thread workgroup.
// Rows of sequences without units get out = 0 and lse = -inf here; rows the stream kernel
// finished itself (count 0) are skipped.
// The first KB pieces (KB = 8, 12 or 16, the launch's estimate of the most pieces a segment has) sit
// in the segment's own slots and are requested whole, together with the count and the context
// length (the three loads share one round trip); those past the count are dropped by selection
// (their slots hold stale values, never multiplied in). The rest of the own slots and up to
// kCombineWide overflow pieces (slots of waves w0 + k) share the second round trip; longer
// segments take one more per kCombineWide pieces.
template <class DT, int D, int MODE, int KB>
__global__ __launch_bounds__(64) void stream_combine_kernel(DecodeParams p) {
    static_assert(KB <= kSegSlots, "the first batch is the segment's own slots");
    constexpr int PER = D / 64;
    const int r = blockIdx.x;
    if (r >= p.batch * p.q_heads) {
        // the fused step's new K/V rows, in workgroups of their own beside the merges (a merge
        // workgroup that also stored a row waited for the row before fetching its partials);
        // an INT8 cache takes the row quantised
        if constexpr (DT::kQ8)
            write_new_row_q8<typename DT::In, D>(p, r - p.batch * p.q_heads, threadIdx.x);
        else
            write_new_row<DT::kBytes, D>(p, r - p.batch * p.q_heads, threadIdx.x);
        return;
    }
    const int G = p.group;
    const int g = r / G, head = r - g * G;
    const int b = g / p.kv_heads, kvh = g - b * p.kv_heads;
    const int lane = threadIdx.x;
    const size_t hrow = (size_t)b * p.q_heads + kvh * G + head;
    const size_t base = (size_t)g * kSegSlots * G + head;  // piece k < kSegSlots: row base + k * G
    const size_t ovf = (size_t)p.batch * p.kv_heads * kSegSlots * G + head;  // later piece k: row ovf + (w0 + k) * G
    RowBatch<KB, PER> first;
    load_rows<KB, D>(p, first, base, KB, G, lane);
    int cnt = p.seg_count[2 * g];
    int w0 = p.seg_count[2 * g + 1];
    w0 = w0 < 0 ? 0 : (w0 >= p.waves_total ? p.waves_total - 1 : w0);  // in range by construction
    const int nu = seq_units<MODE>(p, b);
    // one branch on both values (no short circuit): with the count tested only past the
    // empty-sequence case, its load was issued after the first batch had returned
    if ((nu == 0) | (cnt == 0)) {
        if (nu == 0) {
#pragma unroll
            for (int i = 0; i < PER; ++i) store_out(p.out, p.out_dtype, hrow * D + lane * PER + i, 0.f);
            if (lane == 0 && p.lse) p.lse[hrow] = kNegInf;
            if (lane == 0 && p.row_lse2) p.row_lse2[hrow] = kNegInf;
        }
        return;
    }
    // never past the last wave by construction; keeps every read in bounds
    if (cnt > p.waves_total - w0) cnt = p.waves_total - w0;
    float M = kNegInf, Ls = 0.f;
    float o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    merge_rows<KB, PER>(M, Ls, o, first, cnt, lane);
    if (cnt > KB) {
        // The rest of the own slots (KB .. kSegSlots - 1) and the first overflow batch (pieces
        // kSegSlots, ... in the slots of waves w0 + kSegSlots, ...) depend only on the count and
        // w0: both are requested before either is merged, one round trip for the two.
        constexpr int KO = KB < kSegSlots ? kSegSlots - KB : 1;
        const int n_own = KB < kSegSlots ? (cnt < kSegSlots ? cnt : kSegSlots) - KB : 0;
        RowBatch<KO, PER> ro;
        load_rows<KO, D>(p, ro, base + (size_t)KB * G, n_own, G, lane);
        const int n_ov = cnt - kSegSlots;
        const size_t row_ov = ovf + (size_t)(w0 + kSegSlots) * G;
        if (n_ov <= 0) {
            merge_rows<KO, PER>(M, Ls, o, ro, n_own, lane);
        } else if (n_ov <= 8) {
            RowBatch<8, PER> rv;
            load_rows<8, D>(p, rv, row_ov, n_ov, G, lane);
            if (n_own > 0) merge_rows<KO, PER>(M, Ls, o, ro, n_own, lane);
            merge_rows<8, PER>(M, Ls, o, rv, n_ov, lane);
        } else {
            const int nx = n_ov < kCombineWide ? n_ov : kCombineWide;
            RowBatch<kCombineWide, PER> rv;
            load_rows<kCombineWide, D>(p, rv, row_ov, nx, G, lane);
            if (n_own > 0) merge_rows<KO, PER>(M, Ls, o, ro, n_own, lane);
            merge_rows<kCombineWide, PER>(M, Ls, o, rv, nx, lane);
            // longer segments: the rest of the overflow slots, up to kCombineWide per round trip
            for (int k = kSegSlots + nx; k < cnt;) {
                const int n = cnt - k < kCombineWide ? cnt - k : kCombineWide;
                RowBatch<kCombineWide, PER> rb;
                load_rows<kCombineWide, D>(p, rb, ovf + (size_t)(w0 + k) * G, n, G, lane);
                merge_rows<kCombineWide, PER>(M, Ls, o, rb, n, lane);
                k += n;
            }
        }
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) store_out(p.out, p.out_dtype, hrow * D + lane * PER + i, o[i] * inv);
    if (lane == 0 && p.lse) p.lse[hrow] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : kNegInf;
    if (lane == 0 && p.row_lse2) p.row_lse2[hrow] = Ls > 0.f ? M + __log2f(Ls) : kNegInf;
}

// Score export ([Novita] §關鍵技術 2: a token's score is its softmax probability
// p = exp(q.k - rowmax) / l, which needs only the row's max and sum besides the logit).
// Grid: (sequence, kv head) segments x chunks of kScoreUnits units. A thread owns four
// consecutive tokens of one unit: it reads their logits for each of the G query heads as
// one 16-byte load per head, and adds sum_g 2^(x_g - (m_g + log2 l_g)) to score[t] for the
// tokens that are attended. Each token has one owner and the heads are summed in order, so
// the result does not depend on timing.
constexpr int kScoreUnits = 64;  // units per workgroup (256 threads x 4 tokens)

template <int MODE>
__global__ __launch_bounds__(256) void score_kernel(DecodeParams p) {
    const int seg = blockIdx.x;
    const int u = blockIdx.y * kScoreUnits + (threadIdx.x >> 2);
    const int b = seg / p.kv_heads, kvh = seg - b * p.kv_heads;
    const int G = p.group;
    const SeqPlan sp = make_plan<MODE>(p, b);
    if (u >= sp.n_units) return;
    const int t0 = unit_token<MODE>(p, sp, b, u);
    if (t0 < 0) return;
    const int q4 = (threadIdx.x & 3) * 4;  // first token of the thread within the unit
    const float* lg = p.logits + (((size_t)seg * p.units_bound + u) * G) * 16 + q4;
    const float* lse2 = p.row_lse2 + (size_t)b * p.q_heads + kvh * G;
    f32x4 mass = zero4();
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
        if (g < G) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(lg + g * 16);
            const float l2 = lse2[g];
#pragma unroll
            for (int i = 0; i < 4; ++i) mass[i] += prob2(x[i], l2);
        }
    }
    float* row = p.score + (size_t)seg * p.score_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + q4 + i;
        if (t < sp.L && (t < sp.e0 || t >= sp.s1)) row[t] += mass[i];  // attended tokens only
    }
}

// Score export with entries of B > 1 tokens (e.g. one per page): thread e owns entry e of
// a (sequence, kv head) segment and walks its tokens [e*B, (e+1)*B) in 16-token chunks
// aligned to units. For a chunk whose unit was attended, the stored logits of all G heads
// (G x 16 floats, contiguous) arrive as 16-byte loads issued together; each token's mass
// sums its heads in order, and the masses of the entry's attended tokens are added in
// token order. Entries without attended tokens are not written.
template <int MODE>
__global__ __launch_bounds__(256) void score_block_kernel(DecodeParams p) {
    const int seg = blockIdx.x;
    const int e = blockIdx.y * 256 + threadIdx.x;
    const int b = seg / p.kv_heads, kvh = seg - b * p.kv_heads;
    const int G = p.group, B = p.score_block;
    // The plan's context length, the page list and the row normalisers are independent
    // loads: all are issued before any of them is used.
    const SeqPlan sp = make_plan<MODE>(p, b);
    float lse2[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) lse2[g] = g < G ? p.row_lse2[(size_t)b * p.q_heads + kvh * G + g] : 0.f;
    // page-list mode: the sequence's list in LDS, so that finding a page's place in the
    // list is a scan of LDS (entries beyond kListLds are looked up in memory)
    constexpr int kListLds = 256;
    __shared__ int list[MODE == kPages ? kListLds : 1];
    if (MODE == kPages) {
        for (int i = threadIdx.x; i < p.pages_per_seq && i < kListLds; i += 256)
            list[i] = p.page_list[(size_t)b * p.pages_per_seq + i];
        __syncthreads();
    }
    const long long t_lo = (long long)e * B;
    if (t_lo >= sp.L) return;
    const int t_hi = (long long)(e + 1) * B < sp.L ? (e + 1) * B : sp.L;
    const int per = p.block_size >> 4;  // units per page (page-list mode)
    float acc = 0.f;
    bool any = false;
    for (int c0 = (int)(t_lo & ~15LL); c0 < t_hi; c0 += 16) {
        const int cu = c0 >> 4;  // the chunk's unit position t / 16
        int u = -1;              // its index among the enumerated units, -1: not enumerated
        if (MODE == kPages) {
            const int pg = c0 / p.block_size;
            for (int kk = 0; kk < p.pages_per_seq; ++kk) {
                const int v = kk < kListLds ? list[kk] : p.page_list[(size_t)b * p.pages_per_seq + kk];
                if (v == pg) {
                    u = kk * per + (cu - pg * per);
                    break;
                }
            }
        } else if (MODE == kWindow) {
            if (cu < sp.n0) u = cu;
            else if (cu >= sp.u1a) u = sp.n0 + (cu - sp.u1a);
        } else {
            u = cu;
        }
        if (u < 0) continue;
        const float* lg = p.logits + ((size_t)seg * p.units_bound + u) * G * 16;
        float m[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) m[i] = 0.f;
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) {
            if (g < G) {
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(lg + g * 16 + v4 * 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) m[v4 * 4 + i] += prob2(x[i], lse2[g]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = c0 + i;
            const bool att = t >= t_lo && t < t_hi && (MODE != kWindow || t < sp.e0 || t >= sp.s1);
            if (att) {
                acc += m[i];
                any = true;
            }
        }
    }
    if (any) p.score[(size_t)seg * p.score_stride + e] += acc;
}

// Page-list mode with one score entry per page: thread (segment, kk) owns list entry kk,
// so only listed pages are visited and no search is needed; its page's units are
// kk * P/16 .. (kk + 1) * P/16 - 1 and its entry is the page id. Same arithmetic and order
// as score_block_kernel.
__global__ __launch_bounds__(256) void score_page_kernel(DecodeParams p) {
    const int seg = blockIdx.x;
    const int kk = blockIdx.y * 256 + threadIdx.x;
    if (kk >= p.pages_per_seq) return;
    const int b = seg / p.kv_heads, kvh = seg - b * p.kv_heads;
    const int G = p.group;
    const int pg = p.page_list[(size_t)b * p.pages_per_seq + kk];
    int L = p.context_lens[b];
    L = L < 0 ? 0 : (L > p.len_cap ? p.len_cap : L);
    float lse2[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) lse2[g] = g < G ? p.row_lse2[(size_t)b * p.q_heads + kvh * G + g] : 0.f;
    if (pg < 0 || (long long)pg * p.block_size >= L) return;
    const int per = p.block_size >> 4;
    float acc = 0.f;
    for (int c = 0; c < per; ++c) {
        const int c0 = pg * p.block_size + 16 * c;
        if (c0 >= L) break;
        const float* lg = p.logits + ((size_t)seg * p.units_bound + kk * per + c) * G * 16;
        float m[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) m[i] = 0.f;
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) {
            if (g < G) {
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(lg + g * 16 + v4 * 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) m[v4 * 4 + i] += prob2(x[i], lse2[g]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (c0 + i < L) acc += m[i];
    }
    p.score[(size_t)seg * p.score_stride + pg] += acc;
}

template <class DT, int D, int MODE>
static hipError_t launch_stream_t(bool fused, bool scores, const DecodeParams& p, hipStream_t s, hipEvent_t e0,
                                  hipEvent_t e1) {
    const unsigned blocks = (unsigned)(p.waves_total / kStreamWaves);
    if (e0) {
        hipError_t e = hipEventRecord(e0, s);
        if (e != hipSuccess) return e;
    }
    const dim3 grid(blocks), block(64 * kStreamWaves);
    if (scores) {
        if (fused)
            decode_stream_kernel<DT, D, MODE, true, true><<<grid, block, 0, s>>>(p);
        else
            decode_stream_kernel<DT, D, MODE, false, true><<<grid, block, 0, s>>>(p);
    } else {
        if (fused)
            decode_stream_kernel<DT, D, MODE, true, false><<<grid, block, 0, s>>>(p);
        else
            decode_stream_kernel<DT, D, MODE, false, false><<<grid, block, 0, s>>>(p);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (e1) {
        err = hipEventRecord(e1, s);
        if (err != hipSuccess) return err;
    }
    // First batch: as many own slots as a segment has pieces when the lengths are equal
    // (waves / segments + 1), rounded up to 8, 12 or 16. Where that is more than 16 the segments
    // need a second round trip anyway, and the narrow first batch costs less.
    const dim3 cgrid((unsigned)(p.batch * p.q_heads + (p.new_slots ? p.batch * p.kv_heads : 0)));
    const long long segs = (long long)p.batch * p.kv_heads;
    const long long est = segs > 0 ? (p.waves_total + segs - 1) / segs + 1 : 0;
    if (est > 8 && est <= 12)
        stream_combine_kernel<DT, D, MODE, 12><<<cgrid, dim3(64), 0, s>>>(p);
    else if (est > 12 && est <= 16)
        stream_combine_kernel<DT, D, MODE, 16><<<cgrid, dim3(64), 0, s>>>(p);
    else
        stream_combine_kernel<DT, D, MODE, 8><<<cgrid, dim3(64), 0, s>>>(p);
    err = hipGetLastError();
    if (err != hipSuccess || !scores) return err;
    if (MODE == kPages && p.score_block == p.block_size) {
        score_page_kernel<<<dim3((unsigned)(p.batch * p.kv_heads), (unsigned)((p.pages_per_seq + 255) / 256)),
                            dim3(256), 0, s>>>(p);
    } else if (p.score_block > 1) {
        const long long entries = ((long long)p.len_cap + p.score_block - 1) / p.score_block;
        if (entries > 0)
            score_block_kernel<MODE>
                <<<dim3((unsigned)(p.batch * p.kv_heads), (unsigned)((entries + 255) / 256)), dim3(256), 0, s>>>(p);
    } else if (p.units_bound > 0) {
        score_kernel<MODE><<<dim3((unsigned)(p.batch * p.kv_heads),
                                  (unsigned)((p.units_bound + kScoreUnits - 1) / kScoreUnits)),
                             dim3(256), 0, s>>>(p);
    }
    return hipGetLastError();
}

template <class DT, int D>
static hipError_t launch_stream_m(int mode, bool fused, bool scores, const DecodeParams& p, hipStream_t s,
                                  hipEvent_t e0, hipEvent_t e1) {
    switch (mode) {
        case kWindow: return launch_stream_t<DT, D, kWindow>(fused, scores, p, s, e0, e1);
        case kPages: return launch_stream_t<DT, D, kPages>(fused, scores, p, s, e0, e1);
        default: return launch_stream_t<DT, D, kFull>(fused, scores, p, s, e0, e1);
    }
}

template <class DT>
static hipError_t launch_stream_d(int head_dim, int mode, bool fused, bool scores, const DecodeParams& p,
                                  hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    return head_dim == 64 ? launch_stream_m<DT, 64>(mode, fused, scores, p, s, e0, e1)
                          : launch_stream_m<DT, 128>(mode, fused, scores, p, s, e0, e1);
}

hipError_t launch_decode_stream(int dtype, int head_dim, int mode, bool fused, bool scores,
                                const DecodeParams& p, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
    if (p.batch <= 0 || p.waves_total <= 0) return hipSuccess;
    switch (dtype) {
        case kF32: return launch_stream_d<F32>(head_dim, mode, fused, scores, p, s, ev_start, ev_stop);
        case kF16: return launch_stream_d<F16>(head_dim, mode, fused, scores, p, s, ev_start, ev_stop);
        case kI8B: return launch_stream_d<I8B>(head_dim, mode, fused, scores, p, s, ev_start, ev_stop);
        case kI8H: return launch_stream_d<I8H>(head_dim, mode, fused, scores, p, s, ev_start, ev_stop);
        default: return launch_stream_d<BF16>(head_dim, mode, fused, scores, p, s, ev_start, ev_stop);
    }
}

template <class DT, int D, int MODE>
static int occupancy_t() {
    int n = 0;
    // the least occupancy of the variants, so that every launch fits at once
    int m = 0;
    constexpr bool F = !DT::kQ8;  // the fused variants exist for the 16/32-bit caches
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<DT, D, MODE, F, false>, 64 * kStreamWaves,
                                                     0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&m, decode_stream_kernel<DT, D, MODE, F, true>, 64 * kStreamWaves,
                                                     0) != hipSuccess)
        return 1;
    n = m < n ? m : n;
    return n > 0 ? n : 1;
}

template <class DT>
static int occupancy_d(int head_dim, int mode) {
    if (head_dim == 64) {
        return mode == kWindow ? occupancy_t<DT, 64, kWindow>()
                               : mode == kPages ? occupancy_t<DT, 64, kPages>() : occupancy_t<DT, 64, kFull>();
    }
    return mode == kWindow ? occupancy_t<DT, 128, kWindow>()
                           : mode == kPages ? occupancy_t<DT, 128, kPages>() : occupancy_t<DT, 128, kFull>();
}

int stream_blocks_per_cu(int dtype, int head_dim, int mode) {
    switch (dtype) {
        case kF32: return occupancy_d<F32>(head_dim, mode);
        case kF16: return occupancy_d<F16>(head_dim, mode);
        case kI8B: return occupancy_d<I8B>(head_dim, mode);
        case kI8H: return occupancy_d<I8H>(head_dim, mode);
        default: return occupancy_d<BF16>(head_dim, mode);
    }
}

}  // namespace pkv
