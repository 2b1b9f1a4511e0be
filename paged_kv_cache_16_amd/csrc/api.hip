// api.hip — the C ABI declared in include/pagedkv.h: argument validation, split planning
// and kernel dispatch. Validation always runs before anything is enqueued.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/pagedkv.h"
#include "pkv_internal.h"

// The device error word: kernels OR a PKV_DEV_* bit into it when they skip an element whose
// device-side precondition does not hold; pkv_device_errors reads (and clears) it. Each device
// holds its own copy of this module global for the life of the process.
__device__ unsigned int g_pkv_dev_errors;

namespace {

using namespace pkv;

// Address of the current device's error word (nullptr if it cannot be had: reports are then
// dropped). Looked up once per device (0 = not yet, 1 = unavailable); two first calls racing
// store the same value.
std::atomic<uintptr_t> g_err_word[64];
unsigned* dev_err_word() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    uintptr_t w = g_err_word[dev].load(std::memory_order_relaxed);
    if (w == 0) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_pkv_dev_errors)) != hipSuccess || !ptr) ptr = nullptr;
        w = ptr ? (uintptr_t)ptr : 1;
        g_err_word[dev].store(w, std::memory_order_relaxed);
    }
    return w == 1 ? nullptr : reinterpret_cast<unsigned*>(w);
}

constexpr int kTargetWorkgroups = 2048;  // ~8 resident workgroups per CU over 256 CUs
constexpr int kStreamChunkMin = 2;       // minimum units per wave in the persistent kernel: small
                                         // problems spread over many waves (one wave streams only
                                         // a few GB/s, so bandwidth comes from wave count)
constexpr int kSimdsPerCu = 4;         // SIMD units per compute unit (CDNA)
constexpr long long kMaxStreamWaves = 2048;  // most waves of a persistent launch (MI355X: 256 CUs x
                                             // 4 SIMDs, two per SIMD over page lists)
constexpr int kRunSetupBytes = 24576;   // streaming time per wave of one run's set-up, in bytes
constexpr int kDirectShortUnits = 16;    // at most this many units per sequence: one kernel (a wave's
                                         // 4-unit load ring holds every unit of a segment)
constexpr int kDirectWideUnits = kDirectMaxUnits;  // ... or this many, with at least kDirectWideSegments
constexpr int kDirectWideSegments = 64;  // (sequence, kv head) segments, so no merge launch is needed
constexpr int kMinUnitsPerSplit = 2 * kWaves;  // one pair of 16-token units per wave
constexpr int kMaxUnitsPerSplit = kMaxUnitsPerWave * kWaves;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(pkv_dtype t) { return t == PKV_F32 ? 4 : t == PKV_I8 ? 1 : 2; }

bool dtype_ok(int t) { return t == PKV_F32 || t == PKV_F16 || t == PKV_BF16 || t == PKV_I8; }

// Library-internal element code of a cache (INT8 caches by their input type).
int kdt(const pkv_cache_desc* d) {
    if (d->dtype == PKV_I8) return d->input_dtype == PKV_F16 ? kI8H : kI8B;
    return (int)d->dtype;
}
// The type of q and of the outputs other than fp32.
pkv_dtype io_dtype(const pkv_cache_desc* d) { return d->dtype == PKV_I8 ? d->input_dtype : d->dtype; }

pkv_status check_desc(const pkv_cache_desc* d) {
    if (!d) return PKV_ERR_NULL;
    if (!dtype_ok(d->dtype)) return PKV_ERR_UNSUPPORTED;
    if (d->dtype == PKV_I8 && d->input_dtype != PKV_BF16 && d->input_dtype != PKV_F16) return PKV_ERR_UNSUPPORTED;
    if (d->num_blocks < 0 || d->num_kv_heads <= 0 || d->block_size <= 0) return PKV_ERR_SHAPE;
    if (d->head_dim != 64 && d->head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (d->block_size % 16 != 0 || d->block_size > 256) return PKV_ERR_UNSUPPORTED;
    // the split kernel addresses sub-tiles in 16-byte units with 32-bit offsets
    const double chunks = (double)d->num_blocks * d->num_kv_heads * d->block_size * d->head_dim *
                          elem_bytes(d->dtype) / 16.0;
    if (chunks > 4294967295.0) return PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

struct Plan {
    int mode = kFull;
    int units_bound = 0;  // upper bound on 16-token units per sequence
    int units_per_split = kMinUnitsPerSplit;
    int num_splits = 1;
    int len_cap = 0;
    // how paged_decode_attention runs: one kernel, fixed partitions + combine, or the
    // persistent kernel + combine
    enum Path { kDirect, kPartitions, kStream } path = kDirect;
    int chunk_min = 0;  // stream path: minimum units per wave
    int lead = 0;       // stream path: virtual units charged at each segment start
    int unit_bytes = 0;  // K and V bytes of one 16-token unit of one kv head
    bool q8 = false;    // INT8 cache: the stream path only
    long long segments = 0;  // (sequence, kv head) segments of the call
    int block_size = 16;
};

// Path selection for paged_decode_attention (the partial call always uses partitions).
void choose_path(Plan& pl, const pkv_decode_opts* o) {
    // INT8 caches take the stream path only; so does score export over a page list with
    // entries other than single tokens or whole pages (the one-kernel path's score phase
    // covers tokens, pages of a page list, and token ranges of full or windowed sequences)
    const bool scores = o && o->score_acc;
    const bool direct_scores = !scores || pl.mode != kPages || o->score_block <= 1 ||
                               o->score_block == pl.block_size;
    const bool stream_only = pl.q8 || !direct_scores;
    if (o && o->split_tokens > 0) {
        pl.path = pl.num_splits > 1 ? Plan::kPartitions : Plan::kDirect;
    } else if (!stream_only && (pl.units_bound <= kDirectShortUnits ||
                                (pl.units_bound <= kDirectWideUnits && pl.segments >= kDirectWideSegments))) {
        // one kernel, one workgroup per segment: short sequences, or up to kDirectWideUnits units
        // over at least kDirectWideSegments segments, where skipping the merge launch outweighs
        // using fewer CUs (measured: the page-selected MHA-7B shape, 512 segments of 32 units,
        // 31.8 -> 29.5 us per step; the KV-sparse window layers, 64 segments of 34 units, 32
        // layers 1.912 -> 1.880 ms per step once the one-kernel path kept its loads in flight)
        pl.path = Plan::kDirect;
        pl.num_splits = 1;
        pl.units_per_split = pl.units_bound <= kDirectShortUnits ? kDirectShortUnits : kDirectWideUnits;
    } else {
        pl.path = Plan::kStream;
        // at least kStreamChunkMin units per wave, and at most kMaxSlots pieces per segment
        // (past its first kSegSlots + kCombineWide pieces the combine takes one round trip
        // per kSegSlots more)
        // A run's set-up (query and descriptors fetched, load ring refilled, and the previous
        // run's partial stored) costs a wave about what streaming kRunSetupBytes does, so every
        // segment start counts as that many bytes' worth of units: a wave whose share crosses
        // into a new segment streams fewer units. The charge was set by timing the
        // Llama-3-8B layer shape at 0..8 units (24 KiB: 3 units of a 2-byte d=128 cache).
        // Page lists take no charge: their shares are short and their segments equal, and the
        // charge measured slower there (page-selected step 32.4 us with it, 30.6 us without).
        pl.lead = pl.unit_bytes > 0 ? (kRunSetupBytes + pl.unit_bytes / 2) / pl.unit_bytes : 1;
        if (pl.lead < 1) pl.lead = 1;
        if (pl.mode == kPages) pl.lead = 0;
        const int span = pl.units_bound + pl.lead;  // flat positions of the longest segment
        pl.chunk_min = kStreamChunkMin;
        while ((span + pl.chunk_min - 1) / pl.chunk_min + 1 > kMaxSlots) pl.chunk_min *= 2;
    }
}

// Per-device facts asked of the runtime once (0 = not yet asked; racing first calls store
// the same value).
struct DeviceInfo {
    std::atomic<int> cus{0};
    std::atomic<int> occupancy[5][2][3] = {};  // [internal dtype][head_dim 64/128][mode] workgroups per CU
};
DeviceInfo g_dev[64];

int device_cus(int dev) {
    if (dev < 0 || dev >= 64) return 256;
    int n = g_dev[dev].cus.load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_dev[dev].cus.store(n, std::memory_order_relaxed);
    }
    return n;
}

int device_occupancy(int dev, int dtype, int head_dim, int mode) {
    std::atomic<int>* slot = (dev >= 0 && dev < 64) ? &g_dev[dev].occupancy[dtype][head_dim == 128][mode] : nullptr;
    const int known = slot ? slot->load(std::memory_order_relaxed) : 0;
    if (known) return known;
    const int n = stream_blocks_per_cu(dtype, head_dim, mode);
    if (slot) slot->store(n, std::memory_order_relaxed);
    return n;
}

int ring_sink_pages(int sinks, int block_size) { return (int)(((long long)sinks + block_size - 1) / block_size); }

pkv_status check_opts(const pkv_decode_opts* o) {
    if (!o) return PKV_OK;
    if (o->num_sinks < 0 || o->split_tokens < 0) return PKV_ERR_MODE;
    if (o->ring_pages < 0 || (o->ring_pages > 0 && o->window <= 0)) return PKV_ERR_MODE;
    if (o->page_list && o->window > 0) return PKV_ERR_MODE;
    if (o->page_list && o->pages_per_seq <= 0) return PKV_ERR_MODE;
    if (o->score_acc && o->split_tokens > 0) return PKV_ERR_MODE;
    if (o->score_acc && o->score_stride < 0) return PKV_ERR_SHAPE;
    return PKV_OK;
}

// Split plan from host-known bounds only (never reads device data).
Plan make_plan(const pkv_cache_desc* d, int batch, int max_context_len, int max_blocks,
               const pkv_decode_opts* o) {
    Plan pl;
    pl.q8 = d->dtype == PKV_I8;
    pl.block_size = d->block_size;
    pl.segments = (long long)batch * d->num_kv_heads;
    pl.unit_bytes = 2 * 16 * (d->head_dim * elem_bytes(d->dtype) + (pl.q8 ? 4 : 0));
    const int P = d->block_size;
    long long cap = max_context_len;
    // a ring table addresses any length through its columns
    const bool ring = o && o->ring_pages > 0;
    if (!ring && max_blocks >= 0 && (long long)max_blocks * P < cap) cap = (long long)max_blocks * P;
    if (cap < 0) cap = 0;
    pl.len_cap = (int)cap;
    const int full_units = (int)((cap + 15) / 16);
    if (o && o->page_list) {
        pl.mode = kPages;
        long long u = (long long)o->pages_per_seq * (P / 16);
        pl.units_bound = (int)(u > 0x3fffffff ? 0x3fffffff : u);
    } else if (o && o->window > 0 && o->window < cap) {
        pl.mode = kWindow;
        const long long sinks = o->num_sinks < cap ? o->num_sinks : cap;
        long long u = (sinks + 15) / 16 + ((long long)o->window + 15) / 16 + 1;
        pl.units_bound = (int)(u < full_units ? u : full_units);
    } else {
        pl.mode = kFull;
        pl.units_bound = full_units;
    }
    int U;
    if (o && o->split_tokens > 0) {
        U = (o->split_tokens + 15) / 16;
    } else {
        const double total = (double)batch * d->num_kv_heads * pl.units_bound;
        U = (int)ceil(total / kTargetWorkgroups);
        U = (U + kMinUnitsPerSplit - 1) / kMinUnitsPerSplit * kMinUnitsPerSplit;
    }
    if (U < kMinUnitsPerSplit && !(o && o->split_tokens > 0)) U = kMinUnitsPerSplit;
    if (U < 1) U = 1;
    if (U > kMaxUnitsPerSplit) U = kMaxUnitsPerSplit;
    pl.units_per_split = U;
    pl.num_splits = pl.units_bound > 0 ? (pl.units_bound + U - 1) / U : 1;
    return pl;
}

struct WsLayout {
    size_t o_off, m_off, l_off, total;
};

struct StreamWs {
    size_t o_off, m_off, l_off, cnt_off, logits_off, lse2_off, total;
};

// Stream-path workspace: partial slots (kSegSlots per segment plus one overflow slot per wave,
// G rows each) and per-segment (piece count, first wave); with score export also the masked
// logits of every attended unit ([B*Hkv][units_bound][G][16] fp32) and the rows' log2
// normalisers ([B][Hq]).
StreamWs stream_ws(int batch, int kv_heads, int group, long long waves, int head_dim, bool scores, int units_bound) {
    StreamWs w;
    const size_t rows = ((size_t)batch * kv_heads * kSegSlots + (size_t)waves) * group;
    w.o_off = 0;
    w.m_off = align_up(rows * head_dim * sizeof(float));
    w.l_off = w.m_off + align_up(rows * sizeof(float));
    w.cnt_off = w.l_off + align_up(rows * sizeof(float));
    w.logits_off = w.cnt_off + align_up((size_t)batch * kv_heads * 2 * sizeof(int32_t));
    w.lse2_off = w.logits_off;
    w.total = w.logits_off;
    if (scores) {
        w.lse2_off = w.logits_off + align_up((size_t)batch * kv_heads * units_bound * group * 16 * sizeof(float));
        w.total = w.lse2_off + align_up((size_t)batch * kv_heads * group * sizeof(float));
    }
    return w;
}

WsLayout ws_layout(int batch, int q_heads, int splits, int head_dim) {
    WsLayout w;
    const size_t rows = (size_t)batch * q_heads * splits;
    w.o_off = 0;
    w.m_off = align_up(rows * head_dim * sizeof(float));
    w.l_off = w.m_off + align_up(rows * sizeof(float));
    w.total = w.l_off + align_up(rows * sizeof(float));
    return w;
}

// Waves the persistent kernel launches for this plan on the current device (0 if the device
// cannot be queried). One wave per SIMD, except over page lists: each wave keeps a unit or more
// of loads in flight, so 4 waves per CU already hold what the memory needs (more only queue),
// and fewer, longer shares spend less of the kernel on per-share set-up and even out the finish
// times. Page lists keep two waves per SIMD, whose second wave hides their longer set-up per run
// (measured both ways on the benchmark shapes; INT8 caches moved to one wave per SIMD once
// their loads were counted exactly: 44.5 -> 43.0 us per step).
// The most waves a launch of this plan can have on any device (at least one unit per wave,
// at most kMaxStreamWaves): sizes the workspace's overflow slots without asking the device.
long long stream_wave_bound(const Plan& pl, const pkv_cache_desc* d, int batch) {
    const long long n_bound = (long long)batch * d->num_kv_heads * (pl.units_bound + pl.lead);
    long long waves = (n_bound + pl.chunk_min - 1) / pl.chunk_min;
    waves = (waves + kStreamWaves - 1) / kStreamWaves * kStreamWaves;
    return waves < kMaxStreamWaves ? waves : kMaxStreamWaves;
}

long long stream_waves(const Plan& pl, const pkv_cache_desc* d, int batch) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const long long resident =
        (long long)device_cus(dev) * device_occupancy(dev, kdt(d), d->head_dim, pl.mode) * kStreamWaves;
    long long waves = stream_wave_bound(pl, d, batch);
    if (waves > resident) waves = resident / kStreamWaves * kStreamWaves;
    if (pl.mode != kPages && waves > (long long)device_cus(dev) * kSimdsPerCu)
        waves = (long long)device_cus(dev) * kSimdsPerCu / kStreamWaves * kStreamWaves;
    return waves;
}

pkv_status check_decode_args(const pkv_cache_desc* d, const void* k, const void* v, const void* q,
                             const int32_t* bt, int32_t max_blocks, const int32_t* cl, int32_t batch,
                             int32_t q_heads, int32_t max_context_len, const pkv_decode_opts* o) {
    pkv_status st = check_desc(d);
    if (st != PKV_OK) return st;
    if (batch < 0 || q_heads <= 0 || max_context_len < 0 || max_blocks < 0) return PKV_ERR_SHAPE;
    if (batch > 65535) return PKV_ERR_UNSUPPORTED;
    if (q_heads % d->num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (q_heads / d->num_kv_heads > kMaxGroup) return PKV_ERR_UNSUPPORTED;
    if (d->num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;
    st = check_opts(o);
    if (st != PKV_OK) return st;
    if (batch > 0 && (!k || !v || !q || !bt || !cl)) return PKV_ERR_NULL;
    if (batch > 0 && max_blocks == 0) return PKV_ERR_SHAPE;
    if (o && o->ring_pages > 0) {
        if (o->ring_pages < pkv_ring_pages(o->window, d->block_size)) return PKV_ERR_MODE;
        if ((long long)ring_sink_pages(o->num_sinks, d->block_size) + o->ring_pages > max_blocks) return PKV_ERR_SHAPE;
    }
    return PKV_OK;
}

DecodeParams fill_params(const pkv_cache_desc* d, const void* k, const void* v, const void* q,
                         const int32_t* bt, int32_t max_blocks, const int32_t* cl, int32_t q_heads,
                         float scale, const pkv_decode_opts* o, const Plan& pl) {
    DecodeParams p = {};
    p.err = dev_err_word();
    p.k_cache = (const char*)k;
    p.v_cache = (const char*)v;
    p.q = (const char*)q;
    p.block_table = bt;
    p.context_lens = cl;
    p.page_list = o ? o->page_list : nullptr;
    p.num_blocks = d->num_blocks;
    p.block_size = d->block_size;
    p.kv_heads = d->num_kv_heads;
    p.q_heads = q_heads;
    p.group = q_heads / d->num_kv_heads;
    p.max_blocks = max_blocks;
    p.len_cap = pl.len_cap;
    p.window = o ? o->window : 0;
    p.sinks = o ? o->num_sinks : 0;
    p.pages_per_seq = o ? o->pages_per_seq : 0;
    if (o && o->ring_pages > 0) {
        p.ring_sink_pages = ring_sink_pages(o->num_sinks, d->block_size);
        p.ring_pages = o->ring_pages;
    }
    p.units_per_split = pl.units_per_split;
    p.num_splits = pl.num_splits;
    const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d->head_dim);
    p.qk_scale_log2 = sc * 1.4426950408889634f;
    return p;
}

pkv_status hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace

// Scratch of paged_decode_attention_noalloc: the workspace of its calls, in a fixed device
// array instead of caller memory. Each device holds its own copy for the life of the process,
// shared by every call on that device (overlapping calls race); nothing in it has to start at
// zero, since every call writes each value it reads first. Host code never uses the array's name
// as an address (in host code it is a stand-in, not device memory): the device address comes
// from hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::atomic<uintptr_t> g_scratch[64];  // per device: 0 = not looked up yet, 1 = unavailable

void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    uintptr_t v = g_scratch[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        v = (e == hipSuccess && ptr) ? (uintptr_t)ptr : 1;
        g_scratch[dev].store(v, std::memory_order_relaxed);  // racing first calls store the same value
    }
    return v == 1 ? nullptr : reinterpret_cast<void*>(v);
}

}  // namespace

extern "C" {

pkv_status kv_cache_append(const pkv_cache_desc* desc, void* k_cache, void* v_cache, const void* k_new,
                           const void* v_new, const int32_t* slot_mapping, int32_t num_tokens,
                           void* stream) {
    pkv_status st = check_desc(desc);
    if (st != PKV_OK) return st;
    if (num_tokens < 0) return PKV_ERR_SHAPE;
    if (num_tokens == 0) return PKV_OK;
    if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return PKV_ERR_NULL;
    AppendParams p;
    p.err = dev_err_word();
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.k_new = k_new;
    p.v_new = v_new;
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_slots = (int64_t)desc->num_blocks * desc->block_size;
    p.block_size = desc->block_size;
    p.kv_heads = desc->num_kv_heads;
    p.head_dim = desc->head_dim;
    return hip_status(launch_append(kdt(desc), p, (hipStream_t)stream));
}

size_t paged_decode_attention_workspace_size(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                                             int32_t max_context_len, const pkv_decode_opts* opts) {
    if (check_desc(desc) != PKV_OK || check_opts(opts) != PKV_OK) return 0;
    if (batch <= 0 || num_q_heads <= 0 || max_context_len < 0) return 0;
    Plan pl = make_plan(desc, batch, max_context_len, -1, opts);
    choose_path(pl, opts);
    if (pl.path == Plan::kDirect) return 0;
    if (pl.path == Plan::kStream) {
        if (num_q_heads % desc->num_kv_heads) return 0;
        return stream_ws(batch, desc->num_kv_heads, num_q_heads / desc->num_kv_heads, stream_wave_bound(pl, desc, batch),
                         desc->head_dim, opts && opts->score_acc, pl.units_bound)
            .total;
    }
    return ws_layout(batch, num_q_heads, pl.num_splits, desc->head_dim).total;
}

int32_t paged_decode_attention_num_splits(const pkv_cache_desc* desc, int32_t batch, int32_t max_context_len,
                                          const pkv_decode_opts* opts) {
    if (check_desc(desc) != PKV_OK || check_opts(opts) != PKV_OK || max_context_len < 0 || batch < 0) return 0;
    return make_plan(desc, batch, max_context_len, -1, opts).num_splits;
}

}  // extern "C"

namespace {

// The calling thread's profiling events (pkv_profile_events), recorded around the main kernel.
thread_local hipEvent_t t_profile_start = nullptr;
thread_local hipEvent_t t_profile_stop = nullptr;

struct FusedAppend {
    void* k_cache;
    void* v_cache;
    const void* k_new;
    const void* v_new;
    const int32_t* slots;
};

// paged_decode_attention, optionally preceded by the append of one new token per sequence
// (fused into the attention kernel on the persistent and one-kernel paths, a separate
// append launch on the partition path and for INT8 caches).
pkv_status decode_impl(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache, const void* q,
                       const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t batch, int32_t num_q_heads, int32_t max_context_len, float scale,
                       const pkv_decode_opts* opts, void* out, pkv_dtype out_dtype, float* lse_out,
                       void* workspace, size_t workspace_bytes, void* stream, const FusedAppend* fa) {
    pkv_status st = check_decode_args(desc, k_cache, v_cache, q, block_table, max_blocks_per_seq,
                                      context_lens, batch, num_q_heads, max_context_len, opts);
    if (st != PKV_OK) return st;
    if (out_dtype != PKV_F32 && out_dtype != io_dtype(desc)) return PKV_ERR_UNSUPPORTED;
    if (desc->dtype == PKV_I8 && opts && opts->split_tokens > 0) return PKV_ERR_UNSUPPORTED;
    if (batch == 0) return PKV_OK;
    if (!out) return PKV_ERR_NULL;
    // The plan (and so the workspace size) ignores max_blocks_per_seq so that the size
    // query needs no block-table argument; the kernels clamp to the table separately.
    Plan pl = make_plan(desc, batch, max_context_len, -1, opts);
    choose_path(pl, opts);
    Plan run = pl;
    run.len_cap = make_plan(desc, batch, max_context_len, max_blocks_per_seq, opts).len_cap;
    DecodeParams p = fill_params(desc, k_cache, v_cache, q, block_table, max_blocks_per_seq, context_lens,
                                 num_q_heads, scale, opts, run);
    p.out_dtype = out_dtype;
    p.out = out;
    p.lse = lse_out;
    const hipStream_t s = (hipStream_t)stream;
    hipEvent_t ev0 = t_profile_start;
    hipEvent_t ev1 = t_profile_stop;

    // Validate the workspace and finish the launch parameters before anything is enqueued.
    const bool scores = opts && opts->score_acc;
    const int score_block = scores && opts->score_block > 1 ? opts->score_block : 1;
    if (scores && opts->score_block < 0) return PKV_ERR_SHAPE;
    if (scores && opts->score_stride < ((long long)run.len_cap + score_block - 1) / score_block) return PKV_ERR_SHAPE;
    if (scores && ((long long)run.len_cap + score_block - 1) / score_block > 65535LL * 256) return PKV_ERR_UNSUPPORTED;
    if (scores && (pl.units_bound + 63) / 64 > 65535) return PKV_ERR_UNSUPPORTED;  // score grid's y extent
    long long waves = 0;
    if (pl.path != Plan::kDirect) {
        if (!workspace || ((uintptr_t)workspace) % kAlign != 0) return PKV_ERR_WORKSPACE;
    }
    if (scores) {  // both paths; the stream path also takes its logit and normaliser buffers below
        p.score = opts->score_acc;
        p.score_stride = opts->score_stride;
        p.units_bound = pl.units_bound;
        p.score_block = score_block;
    }
    if (pl.path == Plan::kStream) {
        const int G = num_q_heads / desc->num_kv_heads;
        const long long n_bound = (long long)batch * desc->num_kv_heads * (pl.units_bound + pl.lead);
        if (n_bound > 0x7fffffffLL) return PKV_ERR_UNSUPPORTED;
        waves = stream_waves(pl, desc, batch);
        if (waves <= 0) return PKV_ERR_HIP;
        const StreamWs wl =
            stream_ws(batch, desc->num_kv_heads, G, stream_wave_bound(pl, desc, batch), desc->head_dim, scores,
                      pl.units_bound);
        if (workspace_bytes < wl.total) return PKV_ERR_WORKSPACE;
        p.o_part = (float*)((char*)workspace + wl.o_off);
        p.m_part = (float*)((char*)workspace + wl.m_off);
        p.l_part = (float*)((char*)workspace + wl.l_off);
        p.seg_count = (int32_t*)((char*)workspace + wl.cnt_off);
        p.batch = batch;
        p.waves_total = (int)waves;
        p.chunk_min = pl.chunk_min;
        p.seg_lead = pl.lead;
        if (scores) {
            p.logits = (float*)((char*)workspace + wl.logits_off);
            p.row_lse2 = (float*)((char*)workspace + wl.lse2_off);
        }
    } else if (pl.path == Plan::kPartitions) {
        const WsLayout wl = ws_layout(batch, num_q_heads, pl.num_splits, desc->head_dim);
        if (workspace_bytes < wl.total) return PKV_ERR_WORKSPACE;
        p.o_part = (float*)((char*)workspace + wl.o_off);
        p.m_part = (float*)((char*)workspace + wl.m_off);
        p.l_part = (float*)((char*)workspace + wl.l_off);
    }

    // INT8 caches take the stream path only, where the fused step quantises the new row in the kernels
    const bool fuse = fa && pl.path != Plan::kPartitions && (desc->dtype != PKV_I8 || pl.path == Plan::kStream);
    if (fuse) {
        p.k_cache_w = (char*)fa->k_cache;
        p.v_cache_w = (char*)fa->v_cache;
        p.k_new = (const char*)fa->k_new;
        p.v_new = (const char*)fa->v_new;
        p.new_slots = fa->slots;
        p.num_slots = (int64_t)desc->num_blocks * desc->block_size;
    }
    if (fa && !fuse) {  // separate append launch ahead of attention
        AppendParams ap;
        ap.err = p.err;
        ap.k_cache = fa->k_cache;
        ap.v_cache = fa->v_cache;
        ap.k_new = fa->k_new;
        ap.v_new = fa->v_new;
        ap.slots = fa->slots;
        ap.num_tokens = batch;
        ap.num_slots = (int64_t)desc->num_blocks * desc->block_size;
        ap.block_size = desc->block_size;
        ap.kv_heads = desc->num_kv_heads;
        ap.head_dim = desc->head_dim;
        st = hip_status(launch_append(kdt(desc), ap, s));
        if (st != PKV_OK) return st;
    }
    if (pl.path == Plan::kDirect) {
        if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return PKV_ERR_HIP;
        st = hip_status(launch_decode(kdt(desc), desc->head_dim, pl.mode, true, p, batch, s));
        if (st == PKV_OK && ev1 && hipEventRecord(ev1, s) != hipSuccess) return PKV_ERR_HIP;
        return st;
    }
    if (pl.path == Plan::kStream) {
        return hip_status(
            launch_decode_stream(kdt(desc), desc->head_dim, pl.mode, fuse, scores, p, s, ev0, ev1));
    }
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return PKV_ERR_HIP;
    st = hip_status(launch_decode(kdt(desc), desc->head_dim, pl.mode, false, p, batch, s));
    if (st != PKV_OK) return st;
    if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return PKV_ERR_HIP;
    CombineParams cp;
    cp.o_part = p.o_part;
    cp.m_part = p.m_part;
    cp.l_part = p.l_part;
    cp.out = out;
    cp.lse = lse_out;
    cp.rows = batch * num_q_heads;
    cp.num_splits = pl.num_splits;
    cp.head_dim = desc->head_dim;
    cp.out_dtype = out_dtype;
    return hip_status(launch_combine(cp, s));
}

}  // namespace

extern "C" {

pkv_status paged_decode_attention(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                                  const void* q, const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                                  int32_t max_context_len, float scale, const pkv_decode_opts* opts,
                                  void* out, pkv_dtype out_dtype, float* lse_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    return decode_impl(desc, k_cache, v_cache, q, block_table, max_blocks_per_seq, context_lens, batch,
                       num_q_heads, max_context_len, scale, opts, out, out_dtype, lse_out, workspace,
                       workspace_bytes, stream, nullptr);
}

pkv_status paged_decode_attention_noalloc(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                                          const void* q, const int32_t* block_table, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                                          int32_t max_context_len, float scale, const pkv_decode_opts* opts,
                                          void* out, pkv_dtype out_dtype, float* lse_out, void* stream) {
    // the same validation as paged_decode_attention first, so its errors come out unchanged
    pkv_status st = check_decode_args(desc, k_cache, v_cache, q, block_table, max_blocks_per_seq, context_lens,
                                      batch, num_q_heads, max_context_len, opts);
    if (st != PKV_OK) return st;
    const size_t need = paged_decode_attention_workspace_size(desc, batch, num_q_heads, max_context_len, opts);
    if (need > kScratchBytes) return PKV_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0 && !(ws = scratch_ptr())) return PKV_ERR_HIP;
    return decode_impl(desc, k_cache, v_cache, q, block_table, max_blocks_per_seq, context_lens, batch,
                       num_q_heads, max_context_len, scale, opts, out, out_dtype, lse_out, ws,
                       ws ? kScratchBytes : 0, stream, nullptr);
}

pkv_status paged_decode_append_attention(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                                         const void* k_new, const void* v_new, const int32_t* slot_mapping,
                                         const void* q, const int32_t* block_table, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                                         int32_t max_context_len, float scale, const pkv_decode_opts* opts,
                                         void* out, pkv_dtype out_dtype, float* lse_out, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    if (batch > 0 && (!k_new || !v_new || !slot_mapping)) {
        const pkv_status st = check_desc(desc);
        return st != PKV_OK ? st : PKV_ERR_NULL;
    }
    const FusedAppend fa = {k_cache, v_cache, k_new, v_new, slot_mapping};
    return decode_impl(desc, k_cache, v_cache, q, block_table, max_blocks_per_seq, context_lens, batch,
                       num_q_heads, max_context_len, scale, opts, out, out_dtype, lse_out, workspace,
                       workspace_bytes, stream, &fa);
}

pkv_status paged_decode_attention_partial(const pkv_cache_desc* desc, const void* k_cache,
                                          const void* v_cache, const void* q, const int32_t* block_table,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                                          float scale, const pkv_decode_opts* opts, float* o_part,
                                          float* m_part, float* l_part, int32_t num_splits, void* stream) {
    pkv_status st = check_decode_args(desc, k_cache, v_cache, q, block_table, max_blocks_per_seq,
                                      context_lens, batch, num_q_heads, max_context_len, opts);
    if (st != PKV_OK) return st;
    if (opts && opts->score_acc) return PKV_ERR_MODE;  // score export is not part of the partial call
    if (desc->dtype == PKV_I8) return PKV_ERR_UNSUPPORTED;
    const Plan pl = make_plan(desc, batch, max_context_len, -1, opts);
    if (num_splits != pl.num_splits) return PKV_ERR_SHAPE;
    if (batch == 0) return PKV_OK;
    if (!o_part || !m_part || !l_part) return PKV_ERR_NULL;
    Plan run = pl;
    run.len_cap = make_plan(desc, batch, max_context_len, max_blocks_per_seq, opts).len_cap;
    DecodeParams p = fill_params(desc, k_cache, v_cache, q, block_table, max_blocks_per_seq, context_lens,
                                 num_q_heads, scale, opts, run);
    p.o_part = o_part;
    p.m_part = m_part;
    p.l_part = l_part;
    const hipStream_t s = (hipStream_t)stream;
    if (t_profile_start && hipEventRecord(t_profile_start, s) != hipSuccess) return PKV_ERR_HIP;
    st = hip_status(launch_decode(kdt(desc), desc->head_dim, pl.mode, false, p, batch, s));
    if (st == PKV_OK && t_profile_stop && hipEventRecord(t_profile_stop, s) != hipSuccess) return PKV_ERR_HIP;
    return st;
}

pkv_status pkv_profile_events(void* start_event, void* stop_event) {
    t_profile_start = (hipEvent_t)start_event;
    t_profile_stop = (hipEvent_t)stop_event;
    return PKV_OK;
}

pkv_status paged_decode_combine(const float* o_part, const float* m_part, const float* l_part, int32_t batch,
                                int32_t num_q_heads, int32_t num_splits, int32_t head_dim, void* out,
                                pkv_dtype out_dtype, float* lse_out, void* stream) {
    if (batch < 0 || num_q_heads <= 0 || num_splits <= 0) return PKV_ERR_SHAPE;
    if (head_dim <= 0 || head_dim > 256) return PKV_ERR_UNSUPPORTED;
    if (!dtype_ok(out_dtype)) return PKV_ERR_UNSUPPORTED;
    if (batch == 0) return PKV_OK;
    if (!o_part || !m_part || !l_part || !out) return PKV_ERR_NULL;
    if ((long long)batch * num_q_heads > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
    CombineParams cp;
    cp.o_part = o_part;
    cp.m_part = m_part;
    cp.l_part = l_part;
    cp.out = out;
    cp.lse = lse_out;
    cp.rows = batch * num_q_heads;
    cp.num_splits = num_splits;
    cp.head_dim = head_dim;
    cp.out_dtype = out_dtype;
    return hip_status(launch_combine(cp, (hipStream_t)stream));
}

uint64_t pkv_kv_cache_bytes(int64_t batch, int64_t layers, int64_t kv_heads, int64_t head_dim, int64_t seq_len,
                            int64_t dtype_bytes, int64_t block_size) {
    if (batch < 0 || layers < 0 || kv_heads < 0 || head_dim < 0 || seq_len < 0 || dtype_bytes < 0) return 0;
    uint64_t seq = (uint64_t)seq_len;
    if (block_size > 0) seq = (seq + (uint64_t)block_size - 1) / (uint64_t)block_size * (uint64_t)block_size;
    return 2ull * (uint64_t)batch * (uint64_t)layers * (uint64_t)kv_heads * (uint64_t)head_dim * seq *
           (uint64_t)dtype_bytes;
}

const char* pkv_status_string(pkv_status s) {
    switch (s) {
        case PKV_OK: return "ok";
        case PKV_ERR_NULL: return "a required pointer is NULL";
        case PKV_ERR_SHAPE: return "inconsistent or non-positive size";
        case PKV_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, block_size or group size";
        case PKV_ERR_MODE: return "invalid sparsity options (window with page_list, bad field)";
        case PKV_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case PKV_ERR_HIP: return "HIP launch error";
        case PKV_ERR_NO_BLOCKS: return "too few free blocks";
        case PKV_ERR_SCRATCH: return "the call needs more workspace than the no-allocation scratch holds";
    }
    return "unknown status";
}

}  // extern "C"

extern "C" pkv_status paged_select_pages(const float* scores, int32_t heads, int32_t stride,
                                         const int32_t* context_lens, int32_t batch, int32_t block_size,
                                         int32_t k, int32_t recent, int32_t* page_list, void* stream) {
    if (batch < 0 || heads <= 0 || stride < 0 || block_size <= 0) return PKV_ERR_SHAPE;
    if (k <= 0 || recent < 0 || recent > k) return PKV_ERR_SHAPE;
    if (k > kSelectMaxK || stride > kSelectMaxPages || batch > 65535) return PKV_ERR_UNSUPPORTED;
    if (batch == 0) return PKV_OK;
    if (!scores || !context_lens || !page_list) return PKV_ERR_NULL;
    SelectParams p;
    p.err = dev_err_word();
    p.scores = scores;
    p.context_lens = context_lens;
    p.page_list = page_list;
    p.heads = heads;
    p.stride = stride;
    p.batch = batch;
    p.block_size = block_size;
    p.k = k;
    p.recent = recent;
    return hip_status(launch_select(p, (hipStream_t)stream));
}

extern "C" pkv_status pkv_device_errors(uint32_t* flags, int32_t clear, void* stream) {
    if (!flags) return PKV_ERR_NULL;
    unsigned* w = dev_err_word();
    if (!w) return PKV_ERR_HIP;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return PKV_ERR_HIP;
    unsigned v = 0;
    if (hipMemcpy(&v, w, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return PKV_ERR_HIP;
    *flags = v;
    if (clear && v) {
        const unsigned zero = 0;
        if (hipMemcpy(w, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return PKV_ERR_HIP;
    }
    return PKV_OK;
}
