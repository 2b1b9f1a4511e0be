// pkv_internal.h — kernel parameter blocks and launchers shared by the host dispatch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

enum Mode : int { kFull = 0, kWindow = 1, kPages = 2 };
// kI8B / kI8H: INT8 cache with bf16 / fp16 inputs (library-internal codes)
enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2, kI8B = 3, kI8H = 4 };

constexpr int kWaves = 4;           // wavefronts per workgroup of the split kernel
constexpr int kStreamWaves = 4;    // wavefronts per workgroup of the persistent kernel
constexpr int kMaxUnitsPerWave = 64;  // unit descriptors are held one per lane
constexpr int kMaxSlots = 512;      // most pieces a segment is cut into on the persistent path
constexpr int kSegSlots = 16;       // partial slots held per segment (its first pieces); later
                                    // pieces go to one overflow slot per wave
constexpr int kCombineWide = 24;   // pieces past the first kSegSlots that the combine requests in its
                                    // second round trip (at most 32: lanes 0..31 hold their (m, l))
static_assert(kCombineWide <= 32, "the combine reduces (m, l) over lanes 0..31");
constexpr int kMaxGroup = 8;        // query heads per kv head (each in 2 of the 16 MFMA columns)
constexpr int kDirectMaxUnits = 40;  // units per segment the one-kernel path takes (and stages
                                     // logits for, with score export)

// Bits of the device error word (the PKV_DEV_* values of the C ABI).
enum DevError : unsigned { kDevBlockId = 1u, kDevSlot = 2u, kDevContext = 4u, kDevPages = 8u };

// Records a skipped device-side precondition violation (vector atomic; error paths only).
__device__ __forceinline__ void report(unsigned* err, unsigned bit) {
    if (err) atomicOr(err, bit);
}

struct AppendParams {
    void* k_cache;
    void* v_cache;
    const void* k_new;
    const void* v_new;
    const int32_t* slots;
    int64_t num_tokens;
    int64_t num_slots;  // num_blocks * block_size
    int32_t block_size;
    int32_t kv_heads;
    int32_t head_dim;
    unsigned* err;  // device error word
};

struct DecodeParams {
    const char* k_cache;  // byte pointers to the pools
    const char* v_cache;
    const char* q;
    const int32_t* block_table;
    const int32_t* context_lens;
    const int32_t* page_list;
    void* out;       // direct mode: [B][Hq][D] of out dtype
    float* lse;      // direct mode, nullable
    float* o_part;   // split mode: [B][Hq][S][D]
    float* m_part;   // split mode: [B][Hq][S]
    float* l_part;
    int32_t num_blocks;
    int32_t block_size;
    int32_t kv_heads;
    int32_t q_heads;
    int32_t group;
    int32_t max_blocks;
    int32_t len_cap;       // max_context_len, and with a plain table at most max_blocks * block_size
    int32_t ring_sink_pages;  // ring table: columns [0, ring_sink_pages) hold the sink pages
    int32_t ring_pages;       // ring table: pages past them cycle through this many columns (0: plain)
    int32_t window;
    int32_t sinks;
    int32_t pages_per_seq;
    int32_t units_per_split;
    int32_t num_splits;
    int32_t out_dtype;     // DType
    float qk_scale_log2;   // scale * log2(e)
    // stream (persistent) kernel only
    int32_t batch;
    int32_t waves_total;   // waves launched
    int32_t chunk_min;     // minimum units per wave
    int32_t seg_lead;      // virtual units charged at the start of every segment (run set-up)
    unsigned* err;         // device error word
    int32_t* seg_count;    // [B*Hkv][2]: pieces of the segment (0 = final row written), first piece's wave
    // fused decode step only: the batch's new rows ([B][Hkv][D]) and their slots ([B])
    char* k_cache_w;
    char* v_cache_w;
    const char* k_new;
    const char* v_new;
    const int32_t* new_slots;
    int64_t num_slots;
    // score export only: masked log2-domain logits [B*Hkv][units_bound][G][16], the rows'
    // log2 normalisers [B][Hq] (m + log2 l), and the caller's [B][Hkv][score_stride] sums
    float* logits;
    float* row_lse2;
    float* score;
    int32_t score_stride;
    int32_t units_bound;
    int32_t score_block;   // tokens per score entry (>= 1)
};

struct SelectParams {
    const float* scores;   // [batch][heads][stride]
    const int32_t* context_lens;
    int32_t* page_list;    // [batch][k]
    int32_t heads;
    int32_t stride;
    int32_t batch;
    int32_t block_size;
    int32_t k;
    int32_t recent;
    int32_t stage_pages;  // pages per LDS staging chunk (a multiple of 4), 0 = unstaged loads
    unsigned* err;  // device error word
};

struct CombineParams {
    const float* o_part;
    const float* m_part;
    const float* l_part;
    void* out;
    float* lse;
    int32_t rows;  // batch * q_heads
    int32_t num_splits;
    int32_t head_dim;
    int32_t out_dtype;
};

hipError_t launch_append(int dtype, const AppendParams& p, hipStream_t s);
hipError_t launch_decode(int dtype, int head_dim, int mode, bool direct, const DecodeParams& p,
                         int batch, hipStream_t s);
// Persistent stream kernel + its combine (the paged_decode_attention path). Events, when
// non-null, are recorded around the stream kernel.
hipError_t launch_decode_stream(int dtype, int head_dim, int mode, bool fused, bool scores,
                                const DecodeParams& p, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);
int stream_blocks_per_cu(int dtype, int head_dim, int mode);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
hipError_t launch_select(const SelectParams& p, hipStream_t s);
constexpr int kSelectMaxK = 64;
constexpr int kSelectMaxPages = 15360;  // page keys held in LDS (60 KiB)

}  // namespace pkv
