// pn_probe.hip - streaming-read probe: the device's practical HBM read
// ceiling, measured in the same harness as the GEMV (the v100-skinny README,
// "Kernel benchmarks", quotes its kernels against a measured read-only
// ceiling rather than the rated bandwidth; this is that measurement).
//
// Each wave reads its own contiguous share of the buffer through the path
// the fastest kernels here use: 16-byte nontemporal DMA loads into LDS
// (buffer_load_dwordx4 ... lds, 64 lanes x 16 bytes = 1 KiB per
// instruction), 16 KiB stages in a two-stage ring per wave, four waves per
// CU.  Each lane folds its own 16 bytes of every instruction back out of LDS
// with XOR and writes one word, so every byte read is accounted for and
// nothing else costs time.  (Register loads of the same shape, eight in
// flight per lane, measured 6.6-6.7 TB/s on MI355X; this path 7.0-7.1.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pn.h"
#include "pn_host.h"

namespace {

constexpr int kProbeWaves = 4;                 // per workgroup, one workgroup per CU
constexpr int kProbeThreads = 64 * kProbeWaves;
constexpr int kProbeInstr = 16;                // DMA instructions per stage
constexpr int kProbeStage = 1024 * kProbeInstr;
constexpr int kProbeLds = kProbeWaves * 2 * kProbeStage;

typedef __attribute__((address_space(3))) void probe_lds_t;
typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void probe_issue(const __amdgpu_buffer_rsrc_t &r, uint8_t *stage, int lane, int k)
{
#pragma unroll
    for (int i = 0; i < kProbeInstr; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (probe_lds_t *)(stage + 1024 * i), 16, lane * 16,
                                                 k * kProbeStage + 1024 * i, 0, 2 /* nontemporal */);
}

__global__ __launch_bounds__(kProbeThreads) void read_probe(const uint8_t *buf, uint32_t span, uint32_t *out)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t gw = (uint64_t)blockIdx.x * kProbeWaves + wave;
    uint8_t *ring = lds + wave * 2 * kProbeStage;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(buf + gw * span), 0, (int)span, 0x00020000);
    const int n = (int)((span + kProbeStage - 1) / kProbeStage);  // stages of this wave; the last may
                                                                    // run past the span (read nothing)
    uint32_t acc = 0;
    probe_issue(r, ring, lane, 0);
    probe_issue(r, ring + kProbeStage, lane, 1);  // past the end: out of range, reads nothing
    auto step = [&](uint8_t *stage, int k) {
        // stage k has landed once at most the next stage's instructions are outstanding
        __builtin_amdgcn_s_waitcnt((1 << 14) | 0x0f70);  // vmcnt(16)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < kProbeInstr; ++i) {
            const probe_u32x4 v = *(const probe_u32x4 *)(stage + 1024 * i + 16 * lane);
            acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the stage has been read
        asm volatile("" ::: "memory");
        probe_issue(r, stage, lane, k + 2);  // past the end: out of range, reads nothing
    };
    for (int k = 0; k < n; k += 2) {
        step(ring, k);
        if (k + 1 < n) step(ring + kProbeStage, k + 1);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no DMA left writing LDS
    out[gw * 64 + lane] = acc;
}

bool set_probe_attr()
{
    return hipFuncSetAttribute((const void *)read_probe, hipFuncAttributeMaxDynamicSharedMemorySize, kProbeLds) ==
           hipSuccess;
}

}  // namespace

extern "C" {

size_t pn_read_probe_scratch_bytes(void)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return (size_t)cus * kProbeThreads * sizeof(uint32_t);
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
    const uint64_t grid = (uint64_t)cus;
    const uint64_t waves = grid * kProbeWaves;
    if (scratch_bytes < waves * 64 * sizeof(uint32_t)) return PN_ESHAPE;
    uint64_t span = bytes / waves;
    span -= span % 1024;  // whole DMA instructions per wave
    if (span < 1024 || span > 0x7fffffffu) return PN_ESHAPE;
    if (!pn::host::once_per_device(pn::host::kAttrProbe, set_probe_attr)) return PN_ELAUNCH;
    hipLaunchKernelGGL(read_probe, dim3((unsigned)grid), dim3(kProbeThreads), kProbeLds, (hipStream_t)stream,
                       (const uint8_t *)buf, (uint32_t)span, (uint32_t *)scratch);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    *bytes_read = (size_t)(span * waves);
    return PN_OK;
}

}  // extern "C"
