// pn_rotate.hip - blockwise Hadamard rotation of fp16 activations, for AMD
// Instinct MI355X (gfx950).
//
// The model behind the PN format rotates the activations that reach its PN
// weights, at run time ("How Qwen3.8-27B-PN3 uses it"), so a GEMV against
// those weights takes H x instead of x.  The page gives neither the size of
// the transform nor its scaling; the library's reading: H is block-diagonal
// with 1024 x 1024 Sylvester blocks, H[i][j] = (-1)^popcount(i & j), scaled
// by 1/32 (orthonormal), and each output is rounded once to fp16, ties to
// even, an exact zero as +0.  1024 is the largest power of two dividing
// every PN width of the model (5120, 6144, 17408).
//
// One wave rotates one block: lane l holds elements 16 l .. 16 l + 15 in
// fp64, runs the four butterfly stages whose partners are in the same lane,
// then the six whose partners are lanes l ^ 1 .. l ^ 32 (cross-lane
// shuffles).  In fp64 every step is exact: an fp16 value is a multiple of
// 2^-24 below 2^16, so every partial sum of up to 1024 of them is a multiple
// of 2^-24 below 2^26, inside binary64's 53-bit significand.  The only
// rounding is the last one, to fp16, done correctly by way of binary32
// rounded to odd.
//
// The rotation runs once per activation vector, ahead of the GEMV, not in
// the GEMV's x loads: every 16-row tile of a GEMV reads all of x, so a
// rotation fused there would be redone N / 16 times.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "pn_host.h"

using namespace pn::host;

namespace {

constexpr int kBlock = PN_ROTATE_BLOCK;  // elements per Hadamard block
constexpr int kPerLane = kBlock / 64;    // 16
constexpr int kWaves = 4;                // waves per workgroup
static_assert(kBlock == 1024 && kPerLane == 16, "one wave per block, 16 elements a lane");

// binary64 -> fp16, round to nearest even.  The binary32 conversion rounds
// to nearest; turning that into round-to-odd (truncate, then set the last
// bit when inexact) keeps 13 more bits than fp16 has and a sticky bit, so
// the final fp16 rounding of it is the correct rounding of d.
__device__ __forceinline__ uint32_t to_half_rne(double d)
{
    const float f = (float)d;
    uint32_t u = __float_as_uint(f);
    const double back = (double)f;
    if (back != d) {
        if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1u;  // rounded away from zero: step back
        u |= 1u;
    }
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)__uint_as_float(u));
}

__device__ __forceinline__ double half_lo(uint32_t w)
{
    return (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}

__device__ __forceinline__ double half_hi(uint32_t w)
{
    return (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Rotate the block at src into dst (may be the same memory: every lane has
// read its elements before any lane writes).  4-byte aligned pointers.
__device__ __forceinline__ void rotate_block(const uint16_t *src, uint16_t *dst, int lane)
{
    const uint32_t *s = (const uint32_t *)(src + kPerLane * lane);
    double v[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane / 2; ++i) {
        const uint32_t w = s[i];
        v[2 * i] = half_lo(w);
        v[2 * i + 1] = half_hi(w);
    }
    // partners in the lane: element distances 1, 2, 4, 8
#pragma unroll
    for (int h = 1; h < kPerLane; h <<= 1) {
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            if (i & h) continue;
            const double a = v[i], b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
    // partners in lane l ^ d: element distances 16 .. 512.  The lower
    // element of a pair becomes a + b, the upper one a - b.
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const bool upper = (lane & d) != 0;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const double p = __shfl_xor(v[i], d, 64);
            v[i] = upper ? p - v[i] : v[i] + p;
        }
    }
    uint32_t *o = (uint32_t *)(dst + kPerLane * lane);
#pragma unroll
    for (int i = 0; i < kPerLane / 2; ++i)
        o[i] = to_half_rne(v[2 * i] * 0x1p-5 + 0.0) | (to_half_rne(v[2 * i + 1] * 0x1p-5 + 0.0) << 16);
}

// M rows of K elements: wave w takes block w % nbk of row w / nbk.
__global__ __launch_bounds__(64 * kWaves) void rotate_rows(const uint16_t *x, int64_t ldx, uint16_t *out, int64_t ldo,
                                                            int nbk, int total)
{
    const int w = blockIdx.x * kWaves + (int)(threadIdx.x >> 6);
    if (w >= total) return;
    const int64_t m = w / nbk, b = w - m * nbk;
    rotate_block(x + m * ldx + b * kBlock, out + m * ldo + b * kBlock, (int)(threadIdx.x & 63));
}

// A plan's list of blocks (device memory): wave w rotates jobs[w].
__global__ __launch_bounds__(64 * kWaves) void rotate_jobs(const RotJob *jobs, int total)
{
    const int w = blockIdx.x * kWaves + (int)(threadIdx.x >> 6);
    if (w >= total) return;
    const RotJob j = jobs[w];
    rotate_block(j.src, j.dst, (int)(threadIdx.x & 63));
}

}  // namespace

pn_status pn::host::rotate_jobs_launch(const RotJob *jobs, int total, hipStream_t s)
{
    if (total < 1) return PN_OK;
    hipLaunchKernelGGL(rotate_jobs, dim3((unsigned)((total + kWaves - 1) / kWaves)), dim3(64 * kWaves), 0, s, jobs,
                       total);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    g_last_variant = kVarRotate;
    return PN_OK;
}

pn_status pn_rotate(const uint16_t *x, int64_t K, int M, int64_t ldx, uint16_t *out, int64_t ldo, void *stream)
{
    const hipStream_t s = (hipStream_t)stream;
    if (!x || !out) return PN_EINVAL;
    if (K < kBlock || K % kBlock != 0 || M < 1 || ldx < K || ldo < K) return PN_ESHAPE;
    if (!aligned4(x) || !aligned4(out) || (ldx & 1) || (ldo & 1)) return PN_EALIGN;
    const int64_t total = (int64_t)M * (K / kBlock);
    if (total > INT32_MAX - kWaves) return PN_EUNSUPPORTED;
    hipLaunchKernelGGL(rotate_rows, dim3((unsigned)((total + kWaves - 1) / kWaves)), dim3(64 * kWaves), 0, s, x, ldx,
                       out, ldo, (int)(K / kBlock), (int)total);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    g_last_variant = kVarRotate;
    return PN_OK;
}
