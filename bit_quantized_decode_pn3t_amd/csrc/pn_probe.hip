// pn_probe.hip - streaming-read probe: the device's practical HBM read
// ceiling, measured in the same harness as the GEMV (the v100-skinny README,
// "Kernel benchmarks", quotes its kernels against a measured read-only
// ceiling rather than the rated bandwidth; this is that measurement).
//
// Each wave reads its own contiguous share of the buffer with 16-byte
// nontemporal buffer loads (64 lanes x 16 bytes = 1 KiB per instruction,
// 8 in flight), folds the data with XOR and writes one word per lane, so
// nothing but the read stream costs time.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pn.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;
constexpr int kProbeWgsPerCu = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe(const uint8_t *buf, uint64_t span, uint32_t *out)
{
    const int lane = threadIdx.x & 63;
    const uint64_t wave = (uint64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
    const uint8_t *base = buf + wave * span;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0,
                                                                       (int)span, 0x00020000);
    const int n = (int)(span / 1024);
    uint32_t acc = 0;
    int i = 0;
    for (; i + kProbeInFlight <= n; i += kProbeInFlight) {
        uint32_t v[kProbeInFlight][4];
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, (i + u) * 1024, 2);
            v[u][0] = t[0]; v[u][1] = t[1]; v[u][2] = t[2]; v[u][3] = t[3];
        }
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n; ++i) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, i * 1024, 2);
        acc ^= t[0] ^ t[1] ^ t[2] ^ t[3];
    }
    out[wave * 64 + lane] = acc;
}

}  // namespace

extern "C" {

size_t pn_read_probe_scratch_bytes(void)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return (size_t)cus * kProbeWgsPerCu * kProbeThreads * sizeof(uint32_t);
}

pn_status pn_read_probe(const void *buf, size_t bytes, void *scratch, size_t scratch_bytes, size_t *bytes_read,
                        void *stream)
{
    if (!buf || !scratch || !bytes_read) return PN_EINVAL;
    if (((uintptr_t)buf & 15) || ((uintptr_t)scratch & 3)) return PN_EALIGN;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return PN_ELAUNCH;
    const uint64_t grid = (uint64_t)cus * kProbeWgsPerCu;
    const uint64_t waves = grid * (kProbeThreads / 64);
    if (scratch_bytes < waves * 64 * sizeof(uint32_t)) return PN_ESHAPE;
    uint64_t span = bytes / waves;
    span -= span % 1024;
    if (span < 1024 || span > 0x7fffffffu) return PN_ESHAPE;
    hipLaunchKernelGGL(read_probe, dim3((unsigned)grid), dim3(kProbeThreads), 0, (hipStream_t)stream,
                       (const uint8_t *)buf, span, (uint32_t *)scratch);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    *bytes_read = (size_t)(span * waves);
    return PN_OK;
}

}  // extern "C"
