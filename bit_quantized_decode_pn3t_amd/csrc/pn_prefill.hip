// pn_prefill.hip - PN GEMM for prefill (any number of activation rows), for
// AMD Instinct MI355X (gfx950), and its C ABI: pn_gemm_prefill and
// pn_gemm_prefill_group.
//
// Y[m, r] = sum_k w[r, k] X[m, k] for m < M, w = d * (n - z) ("Exact decode
// in fp32").  The pages' engine handles prefill by dequantizing PN weights
// for a chunked GEMM ("What the fork adds"); here the weights are decoded
// inside the GEMM, from the packed bytes, and never written out: at prompt
// lengths of hundreds of tokens a GEMM that re-read a decoded fp16 copy
// would move 2 bytes a weight per pass instead of 0.43-0.53.
//
// Products on MFMA (v_mfma_f32_32x32x16_f16): X is the A operand, the
// decoded weights (n - z) - small integers, exact in fp16 - the B operand.
// d * (n - z) is not always exact in fp16 (up to 14 significant bits), so d
// stays out of the operands: each 34-byte block's products go into a fresh
// accumulator, which is then scaled by that block's d in fp32 and added to
// the running sum.
//
// Tiles.  A workgroup of eight waves computes 128 rows of X (M) by 256
// weight rows (N); each wave owns 128 x 32 of it (4 x 1 MFMA tiles), so
// every weight row is decoded by one wave only.  The K loop takes one block
// pair (two 34-byte blocks, 68 bytes, 17 aligned dwords: 160 k for pn3t,
// 128 for pn4t) at a time: the workgroup stages the X tile (128 x 160 or
// 128 fp16) and the 256 weight rows' block pairs in LDS by DMA (X one pair
// ahead in two stages, the weights two pairs ahead in three), and each wave
// decodes its 32 weight rows straight into B operands.
//
// Work.  One launch takes one product or several (up to 8, of either type,
// numbered one after another: a decoder layer's q, k and v, or gate and
// up, whose tiles alone leave part of the device idle).  One workgroup per
// CU, persistent.  The launch's tiles would leave
// the last round of workgroups part empty (272 gate tiles on 256 CUs take
// two rounds of the same length), so the tiles of whole rounds are dealt
// whole (tile t to workgroup t mod G, plain stores) and each of the R
// remaining tiles is shared by `ways` workgroups, each taking a slice of its
// block pairs and adding its sums into Y with fp32 atomics, those tiles'
// rows having been zeroed by a kernel ahead of the launch.  The slices of a
// shared tile are then added in a different order from run to run (within
// the tolerance); tiles dealt whole are stored plainly and come out the
// same every run.
//
// Operand layouts (checked on the GPU: lane l of the 32 x 32 x 16 MFMA):
// A row l % 32, k = 8 (l / 32) + e; B column l % 32, same k; result
// register v holds row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.  So a
// lane's 16 results share one weight row and one scale.
//   pn4t  word j of a block holds codes 8j .. 8j + 7, so k-step s of a block
//         takes word 2s + h in lane half h, and X at 64 b + 16 s + 8 h + e.
//   pn3t  a word holds 10 codes, which do not fall on the 8-code grid; the
//         k order inside a block is permuted instead (a GEMM's sum is
//         order-free if A and B agree): lane half h owns codes 40h .. 40h+39
//         (its words 4h .. 4h+3) and k-step s takes codes 40h + 8s .. +7,
//         the lane's code pairs 4s .. 4s+3; X is read at 80 b + 40 h + 8 s,
//         one aligned 16-byte read like pn4t's.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "pn_device.h"
#include "pn_host.h"

using namespace pn;
using namespace pn::host;

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kPfWaves = 8;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfM = 128;    // X rows per workgroup
constexpr int kPfN = 256;    // weight rows per workgroup
constexpr int kPairDw = 17;  // dwords per block pair
#ifndef PN_PF_MAX_WAYS
#define PN_PF_MAX_WAYS 8
#endif
constexpr int kPfMaxWays = PN_PF_MAX_WAYS;  // workgroups that may share one tile's block pairs
// 32-row X tiles per wave: 4 (each wave decodes its own 32 weight rows and
// multiplies them by all 128 X rows) or 2 (2 x 2 tiles: two waves decode the
// same weight rows).  4 is 3-10 % faster: half the unpack work, twice the X
// operand reads from LDS.
#ifndef PN_PF_WAVE_MT
#define PN_PF_WAVE_MT 4
#endif
constexpr int kMT = PN_PF_WAVE_MT;        // 32-row MFMA tiles of X per wave
constexpr int kNT = 4 / kMT;              // 32-row tiles of weights per wave
constexpr int kWM = kPfM / (32 * kMT);    // waves along M
static_assert(kWM * (kPfN / (32 * kNT)) == kPfWaves, "the waves cover the tile");

template <int TYPE>
struct Pf {
    static constexpr int KS = TYPE == 0 ? 160 : 128;  // k per block pair
    static constexpr int BK = KS / 2;                 // k per block
    static constexpr int STEPS = BK / 16;             // MFMA k-steps per block
    static constexpr int XCH = KS / 8;                // 16-byte chunks of an X row per pair
    static constexpr int XSL = XCH + 1;               // LDS slots per X row (one pad slot)
    static constexpr int XDMA = kPfM * XSL / 64;      // X DMA instructions per stage
    static constexpr int XBYTES = 1024 * XDMA;
    static constexpr int WDMA = kPfN * kPairDw / 64;  // W DMA instructions (4 bytes a lane)
    static constexpr int WBYTES = 256 * WDMA;
    static constexpr int XPER = (XDMA + kPfWaves - 1) / kPfWaves;  // X DMA instructions per wave (at most)
    static constexpr int WPER = (WDMA + kPfWaves - 1) / kPfWaves;
    static constexpr int WSTAGES = 3;  // weight stages: two pairs of lookahead from HBM
    static constexpr int LDS = 2 * XBYTES + WSTAGES * WBYTES;
    // this wave's weight DMA instructions per pair (round-robin over the waves)
    static constexpr int wcount(int wave) { return (WDMA - wave + kPfWaves - 1) / kPfWaves; }
    static_assert(kPfM * XSL % 64 == 0 && kPfN * kPairDw % 64 == 0, "whole DMA instructions");
};

constexpr int kPfLds = Pf<0>::LDS > Pf<1>::LDS ? Pf<0>::LDS : Pf<1>::LDS;
constexpr int kPfGroupMax = 8;  // products per launch (PN_PREFILL_GROUP_MAX)

// One product of a launch.
struct PfProb {
    const uint8_t *W;  // packed rows
    const uint16_t *X;
    float *Y;
    int64_t ldx, ldy;
    int32_t N, M, S, pairs;  // S: row bytes; pairs: block pairs per row
    int32_t tn;              // tiles along N (the product's tile u: N tile u % tn, M tile u / tn)
    int32_t tile0;           // the product's first tile in the launch
    int32_t type;
    int32_t pad;
};

// The launch's products (by value: no device table, nothing allocated) and
// how its tiles are dealt.
struct PfArgs {
    PfProb prob[kPfGroupMax];
    int32_t count;
    int32_t tiles;  // all products' tiles
    int32_t t1;     // tiles [0, t1) dealt whole, a whole number of rounds
    int32_t ways;   // workgroups sharing each of tiles [t1, tiles) (0: none shared)
};

// The product that launch tile t belongs to, read from the launch's
// argument segment with scalar loads (a dynamic index into the by-value
// argument would make the compiler copy the whole array to scratch).
#define PF_KARG __attribute__((address_space(4)))
__device__ __forceinline__ PfProb pf_problem(int t)
{
    const PF_KARG PfArgs *k = (const PF_KARG PfArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    int i = 0;
#pragma unroll
    for (int j = 1; j < kPfGroupMax; ++j)
        if (j < k->count && t >= k->prob[j].tile0) i = j;
    const PF_KARG PfProb &q = k->prob[i];
    PfProb p;
    p.W = q.W;
    p.X = q.X;
    p.Y = q.Y;
    p.ldx = q.ldx;
    p.ldy = q.ldy;
    p.N = q.N;
    p.M = q.M;
    p.S = q.S;
    p.pairs = q.pairs;
    p.tn = q.tn;
    p.tile0 = q.tile0;
    p.type = q.type;
    p.pad = 0;
    return p;
}

__device__ __forceinline__ half8_t cat4(half2_t a, half2_t b, half2_t c, half2_t d)
{
    return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3), __builtin_shufflevector(c, d, 0, 1, 2, 3),
                                   0, 1, 2, 3, 4, 5, 6, 7);
}

// Word j of block b of a staged block pair (17 dwords at p): the first
// block's words are two bytes off the dword grid.
__device__ __forceinline__ uint32_t pair_word(const uint32_t *p, int b, int j)
{
    return b == 0 ? __builtin_amdgcn_alignbit(p[j + 1], p[j], 16) : p[9 + j];
}

__device__ __forceinline__ float pair_scale(const uint32_t *p, int b)
{
    return half_bits_to_float(b == 0 ? p[0] & 0xffffu : p[8] >> 16);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, 0x00020000);
}

// Stage one block pair: X rows m0 .. m0+127 (k of the pair; rows past M read
// zeros), 16 bytes a lane with one pad slot per row, and the block pairs of
// weight rows n0 .. n0+255 (rows past N read zeros), 4 bytes a lane.  The
// instructions are dealt to the waves round-robin; a lane's offsets within
// the tiles are the same for every pair (pf_offsets) and the pair moves the
// scalar offset only.
template <int TYPE>
__device__ __forceinline__ void pf_offsets(uint32_t (&xo)[Pf<TYPE>::XPER], uint32_t (&wo)[Pf<TYPE>::WPER],
                                           uint32_t xrow, uint32_t wrow, int wave, int lane)
{
    using C = Pf<TYPE>;
#pragma unroll
    for (int t = 0; t < C::XPER; ++t) {
        const uint32_t q = 64u * (uint32_t)(wave + kPfWaves * t) + (uint32_t)lane;
        const uint32_t r = q / C::XSL, ch = q - r * C::XSL;
        xo[t] = ch < (uint32_t)C::XCH ? r * xrow + 16u * ch : 0x80000000u;
    }
#pragma unroll
    for (int t = 0; t < C::WPER; ++t) {
        const uint32_t q = 64u * (uint32_t)(wave + kPfWaves * t) + (uint32_t)lane;
        const uint32_t r = q / kPairDw, d = q - r * kPairDw;
        wo[t] = r * wrow + 4u * d;
    }
}

template <int TYPE>
__device__ __forceinline__ void stage_x(uint8_t *st, const __amdgpu_buffer_rsrc_t &xr, const uint32_t (&xo)[Pf<TYPE>::XPER],
                                       int p, int wave)
{
    using C = Pf<TYPE>;
    const int xso = p * C::KS * 2;
#pragma unroll
    for (int t = 0; t < C::XPER; ++t) {
        const int i = wave + kPfWaves * t;
        if (i < C::XDMA)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)(st + 1024 * i), 16, (int)xo[t], xso, 0, 0);
    }
}

template <int TYPE>
__device__ __forceinline__ void stage_w(uint8_t *st, const __amdgpu_buffer_rsrc_t &wr, const uint32_t (&wo)[Pf<TYPE>::WPER],
                                       int p, int wave)
{
    using C = Pf<TYPE>;
    const int wso = p * 68;
#pragma unroll
    for (int t = 0; t < C::WPER; ++t) {
        const int i = wave + kPfWaves * t;
        if (i < C::WDMA)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void *)(st + 256 * i), 4, (int)wo[t], wso, 0, 0);
    }
}

// Wait until at most n of this wave's loads are outstanding (n = 0 or one
// pair's weight DMA count).
template <int TYPE>
__device__ __forceinline__ void pf_wait_vm(bool keep_w, int wave)
{
    using C = Pf<TYPE>;
    static_assert(C::wcount(0) < 16 && C::wcount(kPfWaves - 1) + 1 >= C::wcount(0), "vmcnt immediates");
    if (!keep_w)
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    else if (C::wcount(wave) == C::wcount(0))
        __builtin_amdgcn_s_waitcnt(0x0f70 | C::wcount(0));
    else
        __builtin_amdgcn_s_waitcnt(0x0f70 | C::wcount(kPfWaves - 1));
}

// Block pairs [p0, p1) of tile u of product a (N tile u % tn, M tile u / tn),
// stored (add = false) or added into Y.  Every wave of the workgroup calls
// this with the same arguments.
template <int TYPE>
__device__ __forceinline__ void pf_piece(const PfProb &a, int u, int p0, int p1, bool add, uint8_t *lds, int wave,
                                         int lane)
{
    using C = Pf<TYPE>;
    const int wm = wave % kWM, wn = wave / kWM;
    const int h = lane >> 5, c = lane & 31;
    const uint32_t xrow = (uint32_t)a.ldx * 2u, wrow = (uint32_t)a.S;
    uint32_t xo[C::XPER], wo[C::WPER];
    pf_offsets<TYPE>(xo, wo, xrow, wrow, wave, lane);

    const int n0 = (u % a.tn) * kPfN, m0 = (u / a.tn) * kPfM;
    const int xrows = a.M - m0 < kPfM ? a.M - m0 : kPfM;
    const int wrows = a.N - n0 < kPfN ? a.N - n0 : kPfN;
    const __amdgpu_buffer_rsrc_t xr = rsrc(a.X + (int64_t)m0 * a.ldx, (uint32_t)xrows * xrow);
    const __amdgpu_buffer_rsrc_t wr = rsrc(a.W + (int64_t)n0 * a.S, (uint32_t)wrows * wrow);

    float16_t acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) acc[i][j] = (float16_t){};

    // LDS: two X stages, then WSTAGES weight stages.  Pair j of the piece
    // uses X stage j % 2 and weight stage j % WSTAGES; at its top the wave
    // issues pair j + 1's X and pair j + 2's weights, so a weight DMA has
    // two pairs' compute to land and an X DMA (mostly from L2) one.
    uint8_t *const wbase = lds + 2 * C::XBYTES;
    // every wave is done with the stages of the workgroup's last piece
    __syncthreads();
    stage_x<TYPE>(lds, xr, xo, p0, wave);
    stage_w<TYPE>(wbase, wr, wo, p0, wave);
    asm volatile("" ::: "memory");
    if (p0 + 1 < p1) stage_w<TYPE>(wbase + C::WBYTES, wr, wo, p0 + 1, wave);
    int wcur = 0;  // (p - p0) % WSTAGES
    for (int p = p0; p < p1; ++p) {
        // this wave's loads of pair p have landed (pair p + 1's weights, the
        // youngest, may still be in flight); after the barrier, every wave's
        // have, and every wave is done with pair p - 1's stages
        pf_wait_vm<TYPE>(p + 1 < p1, wave);
        // a bare barrier: __syncthreads() would also wait for the weight
        // DMA still in flight.  The stage's DMA is complete (the waits), and
        // every wave has consumed its reads of the stages being refilled.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int wnext2 = wcur + 2 < C::WSTAGES ? wcur + 2 : wcur + 2 - C::WSTAGES;
        if (p + 1 < p1) stage_x<TYPE>(lds + ((p - p0 + 1) & 1) * C::XBYTES, xr, xo, p + 1, wave);
        // the weight DMA stays the youngest: the next pair's wait counts on it
        asm volatile("" ::: "memory");
        if (p + 2 < p1) stage_w<TYPE>(wbase + wnext2 * C::WBYTES, wr, wo, p + 2, wave);
        const uint16_t *xs = (const uint16_t *)(lds + ((p - p0) & 1) * C::XBYTES);
        const uint32_t *ws = (const uint32_t *)(wbase + wcur * C::WBYTES);
        wcur = wcur + 1 < C::WSTAGES ? wcur + 1 : 0;

#pragma unroll
        for (int b = 0; b < 2; ++b) {
            // decode: the lane's four words of block b, for its row of each N tile
            half2_t u[kNT][4][TYPE == 0 ? 5 : 4];
            float d[kNT];
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const uint32_t *pw = ws + (wn * 32 * kNT + nt * 32 + c) * kPairDw;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    Unpack<TYPE>::run(pair_word(pw, b, TYPE == 0 ? 4 * h + j : h + 2 * j), u[nt][j]);
                d[nt] = pair_scale(pw, b);
            }
            float16_t P[kMT][kNT];  // the block's fresh accumulators
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) P[mt][nt] = (float16_t){};
#pragma unroll
            for (int s = 0; s < C::STEPS; ++s) {
                half8_t B[kNT];
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) {
                    if constexpr (TYPE == 0)  // the lane's code pairs 4s .. 4s+3 (pair i: word i / 5, pair i % 5)
                        B[nt] = cat4(u[nt][(4 * s) / 5][(4 * s) % 5], u[nt][(4 * s + 1) / 5][(4 * s + 1) % 5],
                                     u[nt][(4 * s + 2) / 5][(4 * s + 2) % 5], u[nt][(4 * s + 3) / 5][(4 * s + 3) % 5]);
                    else
                        B[nt] = cat4(u[nt][s][0], u[nt][s][1], u[nt][s][2], u[nt][s][3]);
                }
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) {
                    const uint16_t *px = xs + (wm * 32 * kMT + mt * 32 + c) * (8 * C::XSL);
                    const int k = TYPE == 0 ? 80 * b + 40 * h + 8 * s : 64 * b + 16 * s + 8 * h;
                    const half8_t A = __builtin_bit_cast(half8_t, *(const u32x4 *)(px + k));
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt)
                        P[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B[nt], P[mt][nt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[mt][nt][v] = __builtin_fmaf(d[nt], P[mt][nt][v], acc[mt][nt][v]);
        }
    }

#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const int n = n0 + wn * 32 * kNT + nt * 32 + c;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * 32 * kMT + mt * 32 + 8 * (v / 4) + 4 * h + (v % 4);
                if (m < a.M && n < a.N) {
                    float *y = a.Y + (int64_t)m * a.ldy + n;
                    if (add)
                        __hip_atomic_fetch_add(y, acc[mt][nt][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else
                        *y = acc[mt][nt][v];
                }
            }
        }
}

// Workgroups take the launch's tiles: those of whole rounds one after
// another (tile t to workgroup t mod G), then the R others, workgroup w
// taking slice j = w / R of tile t1 + w % R: its product's block pairs
// [pairs j / ways, pairs (j + 1) / ways).
__global__ __launch_bounds__(kPfThreads) void gemm_prefill(PfArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R = a.tiles - a.t1;
    const bool shares = a.ways > 0 && (int)blockIdx.x < R * a.ways;
    // one call site, so that each type's piece is inlined once
    for (int t = blockIdx.x;; t += gridDim.x) {
        const bool whole = t < a.t1;
        if (!whole && !shares) break;
        // past the whole tiles: this workgroup's slice of a shared tile, once
        const int tt = whole ? t : a.t1 + (int)blockIdx.x % R;
        const int j = whole ? 0 : (int)blockIdx.x / R, ways = whole ? 0 : a.ways;
        const PfProb p = pf_problem(tt);
        const int p0 = ways > 0 ? p.pairs * j / ways : 0, p1 = ways > 0 ? p.pairs * (j + 1) / ways : p.pairs;
        if (p.type == 0)
            pf_piece<0>(p, tt - p.tile0, p0, p1, !whole, lds, wave, lane);
        else
            pf_piece<1>(p, tt - p.tile0, p0, p1, !whole, lds, wave, lane);
        if (!whole) break;
    }
}

// Y = 0 over tiles [t1, tiles) (rows and columns past M and N left alone),
// ahead of a launch whose workgroups add into them (a kernel rather than a
// memset, so that the call can be captured into a graph).  Workgroup (x, y)
// clears rows 4 x .. 4 x + 3 of tile t1 + y.
__global__ __launch_bounds__(256) void zero_tiles(PfArgs a)
{
    const int t = a.t1 + (int)blockIdx.y;
    const PfProb p = pf_problem(t);
    const int u = t - p.tile0;
    const int col = (u % p.tn) * kPfN + (int)threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = (u / p.tn) * kPfM + 4 * (int)blockIdx.x + i;
        if (m < p.M && col < p.N) p.Y[(int64_t)m * p.ldy + col] = 0.0f;
    }
}

bool set_prefill_attr()
{
    return hipFuncSetAttribute((const void *)gemm_prefill, hipFuncAttributeMaxDynamicSharedMemorySize, kPfLds) ==
           hipSuccess;
}

}  // namespace

namespace {

// Validate one product (the checks of pn_gemm_prefill) and fill its record.
pn_status pf_make(pn_type t, const void *W, int64_t N, int64_t K, const void *X, int64_t ldx, int64_t M, float *Y,
                  int64_t ldy, PfProb &p)
{
    pn_status st = check_matrix(t, W, N, K);
    if (st) return st;
    if (!X || !Y) return PN_EINVAL;
    if (M < 1 || ldx < K || ldy < N) return PN_ESHAPE;
    const int64_t nb = K / wpb(t);
    if (nb % 2 != 0) return PN_EUNSUPPORTED;  // whole block pairs only
    if (((uintptr_t)W & 3) || ((uintptr_t)X & 15) || (ldx & 7) || !aligned4(Y)) return PN_EALIGN;
    if (M > INT32_MAX - kPfM || (M + kPfM - 1) / kPfM > 65535) return PN_EUNSUPPORTED;
    if ((uint64_t)kPfM * (uint64_t)ldx * 2u >= 0x80000000ull) return PN_EUNSUPPORTED;  // 32-bit tile offsets
    if (N * M > ((int64_t)1 << 40)) return PN_EUNSUPPORTED;
    if ((uint64_t)kPfN * (uint64_t)nb * 34u >= 0x80000000ull) return PN_EUNSUPPORTED;  // 32-bit row offsets
    const int64_t tn = (N + kPfN - 1) / kPfN;
    if (tn * ((M + kPfM - 1) / kPfM) > INT32_MAX) return PN_EUNSUPPORTED;
    memset(&p, 0, sizeof(p));
    p.W = (const uint8_t *)W;
    p.X = (const uint16_t *)X;
    p.Y = Y;
    p.ldx = ldx;
    p.ldy = ldy;
    p.N = (int32_t)N;
    p.M = (int32_t)M;
    p.S = (int32_t)(nb * 34);
    p.pairs = (int32_t)(nb / 2);
    p.tn = (int32_t)tn;
    p.type = t;
    return PN_OK;
}

int64_t pf_tiles(const PfProb &p) { return (int64_t)p.tn * ((p.M + kPfM - 1) / kPfM); }

// Number the products' tiles one after another, deal them and launch.  One
// workgroup per CU (its LDS stages take 122-138 KiB): the tiles of whole
// rounds are dealt whole, and the R others are each shared by `ways`
// workgroups, as many as fit one round, at most 8 and with at least 4 block
// pairs of every product each: the atomic adds of a shared tile cost about
// as much as computing a few of its pairs (on 256 CUs, 16 gate tiles shared
// 16 ways took 136 us, shared 8 ways less).
pn_status pf_launch(PfArgs &a, hipStream_t s, int variant)
{
    if (!once_per_device(kAttrPrefill, set_prefill_attr)) return PN_ELAUNCH;
    int64_t tiles = 0, min_pairs = INT32_MAX;
    for (int i = 0; i < a.count; ++i) {
        a.prob[i].tile0 = (int32_t)tiles;
        tiles += pf_tiles(a.prob[i]);
        if (tiles > INT32_MAX) return PN_EUNSUPPORTED;
        if (a.prob[i].pairs < min_pairs) min_pairs = a.prob[i].pairs;
    }
    const int64_t G = device_cus();
    a.tiles = (int32_t)tiles;
    a.t1 = (int32_t)(tiles / G * G);
    const int64_t R = tiles - a.t1;
    int64_t ways = R > 0 ? G / R : 1;
    if (ways > kPfMaxWays) ways = kPfMaxWays;
    if (ways > min_pairs / 4) ways = min_pairs / 4;
    if (ways < 2) {  // no tile is shared: the rest are dealt whole too
        a.t1 = (int32_t)tiles;
        ways = 0;
    }
    a.ways = (int32_t)ways;
    const int64_t g2 = R * ways;
    const int64_t grid = a.t1 > 0 ? (G < tiles ? G : tiles) : g2;
    if (g2 > 0) {
        hipLaunchKernelGGL(zero_tiles, dim3(kPfM / 4, (unsigned)(tiles - a.t1)), dim3(kPfN), 0, s, a);
        if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    }
    hipLaunchKernelGGL(gemm_prefill, dim3((unsigned)grid), dim3(kPfThreads), kPfLds, s, a);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    g_last_variant = variant;
    return PN_OK;
}

}  // namespace

pn_status pn_gemm_prefill(pn_type t, const void *W, int64_t N, int64_t K, const uint16_t *X, int64_t ldx, int64_t M,
                          float *Y, int64_t ldy, void *stream)
{
    PfArgs a;
    memset(&a, 0, sizeof(a));
    const pn_status st = pf_make(t, W, N, K, X, ldx, M, Y, ldy, a.prob[0]);
    if (st) return st;
    a.count = 1;
    return pf_launch(a, (hipStream_t)stream, kVarPrefill);
}

pn_status pn_gemm_prefill_group(const pn_gemm_desc *descs, int count, void *stream)
{
    if (!descs || count < 1 || count > kPfGroupMax) return PN_EINVAL;
    PfArgs a;
    memset(&a, 0, sizeof(a));
    for (int i = 0; i < count; ++i) {
        const pn_gemm_desc &e = descs[i];
        const pn_status st = pf_make((pn_type)e.type, e.W, e.N, e.K, e.X, e.ldx, e.M, e.Y, e.ldy, a.prob[i]);
        if (st) return st;
    }
    a.count = count;
    return pf_launch(a, (hipStream_t)stream, kVarPrefillGroup);
}
