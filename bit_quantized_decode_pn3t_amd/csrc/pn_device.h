// pn_device.h - device helpers for the PN decode kernels (gfx950 / CDNA4).
//
// Format (tensorless, "Why a P100-native weight format"): a block is an fp16
// scale d followed by eight 32-bit words; pn3t packs ten 3-bit codes per
// word, pn4t eight 4-bit codes; even codes sit in the low 16 bits and odd
// codes in the high 16 bits at the same offsets ("Codes never straddle the
// two halves of a word"); a weight is d * (n - z) ("Exact decode in fp32").
// Within a half, code pair p sits at bit offset b*p (this library's fixed
// reading of the layout).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pn {

constexpr int kBlockBytes = 34;
constexpr int kWordsPerBlock = 8;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

template <int TYPE> struct Fmt;
template <> struct Fmt<0> {  // pn3t
    static constexpr int C = 10, B = 3, Z = 4, W = 80;
};
template <> struct Fmt<1> {  // pn4t
    static constexpr int C = 8, B = 4, Z = 8, W = 64;
};

// ---------------------------------------------------------------------------
// Code unpacking into exact fp16 pairs.
//
// A masked code pair OR-ed into the mantissa of an fp16 "magic" number 2^e
// reads as (2^e + n) in both halves at once, provided the code's lowest bit
// has weight 1 in that mantissa (e = 10 - offset).  Subtracting (2^e + z) in
// packed fp16 then gives the exact small integers (n_lo - z, n_hi - z): both
// operands are exactly representable and so is their difference.  Pairs
// whose bits reach the exponent field are shifted down first (one shift
// serves two pairs).
//
// pn3t pair offsets 0, 3, 6 use magics 1024, 128, 16; offsets 9 and 12 are
// shifted right by 9 and reuse 1024 and 128.  Bits 15 and 31 are never read.
// pn4t offsets 0 and 4 use 1024 and 64; offsets 8 and 12 are shifted by 8.
// ---------------------------------------------------------------------------
// (a & m) | c as one v_and_or_b32.  gfx9 VOP3 encodings take no literal
// constants, so left to itself the compiler splits this into v_and + v_or
// with literals; here m and c live in registers.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
    return r;
}

template <int TYPE> struct Unpack;

template <> struct Unpack<0> {
    static constexpr int kPairs = 5;
    __device__ __forceinline__ static void run(uint32_t q, half2_t (&t)[5])
    {
        const uint32_t q9 = q >> 9;
        t[0] = as_half2(and_or(q, 0x00070007u, 0x64006400u)) - (half2_t){1028.0f16, 1028.0f16};
        t[1] = as_half2(and_or(q, 0x00380038u, 0x58005800u)) - (half2_t){132.0f16, 132.0f16};
        t[2] = as_half2(and_or(q, 0x01c001c0u, 0x4c004c00u)) - (half2_t){20.0f16, 20.0f16};
        t[3] = as_half2(and_or(q9, 0x00070007u, 0x64006400u)) - (half2_t){1028.0f16, 1028.0f16};
        t[4] = as_half2(and_or(q9, 0x00380038u, 0x58005800u)) - (half2_t){132.0f16, 132.0f16};
    }
};

template <> struct Unpack<1> {
    static constexpr int kPairs = 4;
    __device__ __forceinline__ static void run(uint32_t q, half2_t (&t)[4])
    {
        const uint32_t q8 = q >> 8;
        t[0] = as_half2(and_or(q, 0x000f000fu, 0x64006400u)) - (half2_t){1032.0f16, 1032.0f16};
        t[1] = as_half2(and_or(q, 0x00f000f0u, 0x54005400u)) - (half2_t){72.0f16, 72.0f16};
        t[2] = as_half2(and_or(q8, 0x000f000fu, 0x64006400u)) - (half2_t){1032.0f16, 1032.0f16};
        t[3] = as_half2(and_or(q8, 0x00f000f0u, 0x54005400u)) - (half2_t){72.0f16, 72.0f16};
    }
};

// acc + sum over the word's codes of (n - z) * x, with xp[p] = (x[2p], x[2p+1])
// for the word's code pair p.  Products of fp16 values are exact in fp32;
// v_dot2_f32_f16 accumulates in fp32.
template <int P>
__device__ __forceinline__ float dot_pairs(const half2_t (&t)[P], const uint32_t *xp, float acc)
{
#pragma unroll
    for (int p = 0; p < P; ++p) acc = __builtin_amdgcn_fdot2(t[p], as_half2(xp[p]), acc, false);
    return acc;
}

// Same sum started from zero.  The first product uses the VOP3P encoding with
// an inline-constant zero accumulator (the compiler would otherwise emit a
// v_mov of zero followed by the two-operand v_dot2c form).
template <int P>
__device__ __forceinline__ float dot_pairs0(const half2_t (&t)[P], const uint32_t *xp)
{
    float acc;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(acc) : "v"(t[0]), "v"(xp[0]));
#pragma unroll
    for (int p = 1; p < P; ++p) acc = __builtin_amdgcn_fdot2(t[p], as_half2(xp[p]), acc, false);
    return acc;
}

template <int TYPE>
__device__ __forceinline__ float dot_word(uint32_t q, const uint32_t *xp, float acc)
{
    half2_t t[Unpack<TYPE>::kPairs];
    Unpack<TYPE>::run(q, t);
    return dot_pairs(t, xp, acc);
}

// fp16 bits -> fp32 (exact; fp16 denormals are preserved by the kernels' mode)
__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// ---------------------------------------------------------------------------
// Loads.  Blocks are 34 bytes, so a code word is 4-byte aligned only in every
// other block; gfx950 runs with unaligned global access enabled, and a dword
// load from a 2-aligned address is one instruction.
// ---------------------------------------------------------------------------
#define PN_GLOBAL __attribute__((address_space(1)))
typedef uint32_t __attribute__((aligned(2))) u32_a2_t;

__device__ __forceinline__ uint32_t load_u32_a2(const uint8_t *p)
{
    return *(const PN_GLOBAL u32_a2_t *)p;
}

__device__ __forceinline__ uint32_t load_u16(const uint8_t *p)
{
    return *(const PN_GLOBAL uint16_t *)p;
}

__device__ __forceinline__ uint32_t load_u32(const uint8_t *p)
{
    return *(const PN_GLOBAL uint32_t *)p;
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3:
// 32-bit untyped data).  Loads through it take a per-lane VGPR offset plus a
// scalar offset, and an access past `bytes` returns zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Wave-uniform copies (the value is the same in every lane; this tells the
// compiler so, and keeps it in scalar registers).
__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p)
{
    const uint64_t u = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (T *)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// Wave64 sum: two permlane swaps (gfx950) fold the four 16-lane rows, then
// DPP rotations inside each row.  Every lane receives the total.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));  // row_ror:8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));  // row_ror:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));   // quad_perm 2301
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));   // quad_perm 1032
    return v;
}

}  // namespace pn
