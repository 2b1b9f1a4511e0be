// probe.hip — the achievable HBM read rate, against which the attention kernel's rate is read
// ([primer] §7.1: every decode step reads the whole KV cache, so memory bandwidth, not
// arithmetic, bounds it). Every wave streams its own contiguous share of a buffer with the
// same 16-byte nontemporal loads the attention kernel issues (1 KiB per wave instruction,
// kProbeDepth instructions in flight) and does nothing else with the bytes.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "../../include/pagedkv.h"

namespace pkv {

namespace {

constexpr int kProbeDepth = 8;
constexpr size_t kProbeStep = 1024 * kProbeDepth;  // bytes one wave reads per loop trip

__global__ __launch_bounds__(256) void read_probe_kernel(const char* base, size_t per_wave, unsigned* sink) {
    const int lane = threadIdx.x & 63;
    const size_t wave = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const char* p = base + wave * per_wave + lane * 16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t off = 0; off < per_wave; off += kProbeStep) {
        u32x4 r[kProbeDepth];
#pragma unroll
        for (int i = 0; i < kProbeDepth; ++i) r[i] = load16_stream(p + off + i * 1024);
#pragma unroll
        for (int i = 0; i < kProbeDepth; ++i) acc ^= r[i];
    }
    // a store the compiler cannot prove dead, taken for one value pattern only
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[wave] = acc.x;
}

}  // namespace

}  // namespace pkv

extern "C" pkv_status pkv_read_probe(const void* buf, size_t bytes, int32_t waves_per_simd, uint32_t* sink,
                                     size_t sink_len, size_t* bytes_read, void* stream) {
    if (!buf || !sink || !bytes_read) return PKV_ERR_NULL;
    if (waves_per_simd < 1 || waves_per_simd > 8) return PKV_ERR_SHAPE;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return PKV_ERR_HIP;
    const size_t waves = (size_t)cus * 4 * waves_per_simd;  // 4 SIMDs per CU
    const size_t per_wave = bytes / waves / pkv::kProbeStep * pkv::kProbeStep;
    if (per_wave == 0) return PKV_ERR_SHAPE;  // fewer than kProbeStep bytes per wave
    if (sink_len < waves) return PKV_ERR_SHAPE;
    *bytes_read = per_wave * waves;
    pkv::read_probe_kernel<<<dim3((unsigned)(waves / 4)), dim3(256), 0, (hipStream_t)stream>>>(
        (const char*)buf, per_wave, sink);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
