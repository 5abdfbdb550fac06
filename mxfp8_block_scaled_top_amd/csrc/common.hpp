// Device helpers shared by the gfx950 kernels of libmoe_mi355x.
//
// MXFP8 encoding follows the block rule of the BioNeMo MoE recipe page
// (section on MXFP8 and the fused MLP): one scale for every 32 consecutive
// values.  Element format E4M3 (bias 7, 3 mantissa bits, largest finite 448,
// no infinities), scale format E8M0 (power of two, bias 127).  The scale of a
// block is the smallest power of two X with amax <= 448 X, so no element is
// clamped; elements round to nearest, ties to even.  All of it is integer /
// exact arithmetic: the codes do not depend on any floating-point rounding
// mode or on the order of operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kMxBlock = 32;

typedef uint16_t bf16_t;  // bfloat16 bit pattern

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;

// Round to nearest even (gfx950's v_cvt_pk_bf16_f32, two values per
// instruction; denormals kept, overflow to infinity); NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_v));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// E8M0 scale byte of a block from its max magnitude (amax >= 0, finite):
// smallest s with amax <= 448 * 2^s, i.e. 448 = 1.75 * 2^8 compared with the
// significand of amax; S = s + 127 clamped to [0, 254]; amax = 0 gives 0.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
    uint32_t b = __float_as_uint(amax);
    int eb = (int)((b >> 23) & 0xffu);
    int up = (b & 0x7fffffu) > 0x600000u ? 1 : 0;
    int s = eb - 8 + up;
    s = s < 0 ? 0 : (s > 254 ? 254 : s);
    return b == 0u ? 0u : (uint32_t)s;
}

// Exact multiply by 2^(127 - S) for the magnitudes that matter: results at or
// above 2^-126 are exact; smaller ones all encode to zero anyway.
__device__ __forceinline__ float mx_unscale(float v, uint32_t S) {
    return __builtin_ldexpf(v, 127 - (int)S);
}

// E4M3 code of v / 2^(S-127): sign bit kept, magnitude rounded to nearest
// even on the E4M3 grid.  |v| / X <= 448 is guaranteed by the scale choice.
__device__ __forceinline__ uint32_t mx_encode(float v, uint32_t S) {
    uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    float y = mx_unscale(__builtin_fabsf(v), S);
    uint32_t b = __float_as_uint(y);
    uint32_t mag;
    if (b < 0x3c800000u) {
        // below 2^-6: subnormal steps of 2^-9 (exact product), rint = half-even
        mag = (uint32_t)__builtin_rintf(y * 512.0f);
    } else {
        uint32_t e = (b >> 23) - 120u;       // E4M3 exponent field (bias 7)
        uint32_t m = b & 0x7fffffu;
        uint32_t keep = m >> 20;             // top 3 mantissa bits
        uint32_t rest = m & 0xfffffu;
        uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
        mag = ((e << 3) | keep) + up;        // a carry moves into the exponent
    }
    return sign | mag;
}

// Four E4M3 codes of v0..v3 / 2^(S-127), packed little-endian in a word, by
// gfx950's scaled conversion (v_cvt_scalef32_pk_fp8_f32 divides by the given
// power of two and rounds to nearest even, keeping the sign): two values per
// instruction and no separate unscale.  It gives the same bytes as mx_encode
// for every value a block's scale admits (checked exhaustively over all bf16
// inputs and scales, rounding ties and subnormal midpoints), and the same
// bytes as an exact ldexp unscale followed by v_cvt_pk_fp8_f32 for fp32
// inputs with arbitrary low mantissa bits (8.4 M value pairs on the GPU).
typedef __attribute__((ext_vector_type(2))) short s16x2_t;

__device__ __forceinline__ uint32_t mx_encode4(float v0, float v1, float v2, float v3,
                                               uint32_t S) {
    const float scale = __builtin_ldexpf(1.f, (int)S - 127);     // exact, S in [0, 254]
    const s16x2_t z = {0, 0};
    const s16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, v0, v1, scale, false);
    const s16x2_t w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v2, v3, scale, true);
    return __builtin_bit_cast(uint32_t, w);
}

// Value of an E4M3 code times 2^(S-127), exact in fp32.
__device__ __forceinline__ float mx_decode(uint32_t code, uint32_t S) {
    uint32_t e = (code >> 3) & 15u, m = code & 7u;
    float mag = e == 0u ? (float)m * 0.001953125f                // m * 2^-9
                        : __builtin_ldexpf((float)(8u + m), (int)e - 10);
    float v = __builtin_ldexpf(mag, (int)S - 127);
    return (code & 0x80u) ? -v : v;
}

// Row-pair layout of the 8-bit GEMM operands: rows 2p and 2p+1 of a matrix
// with K bytes per row share 128-byte lines, one line per 64 K-bytes, so that
// one K step (64 bytes) of a tile's row pair is one whole line:
//   byte (r, k) at (r >> 1) * p2_stride(K) + (k >> 6) * 128 + (r & 1) * 64 + (k & 63)
// The matrix occupies ceil(R / 2) * p2_stride(K) bytes; bytes of K-steps past
// K (when K is not a multiple of 64) are padding that no kernel reads.
__host__ __device__ inline int64_t p2_stride(int64_t K) { return ((K + 63) / 64) * 128; }
__host__ __device__ inline int64_t p2_off(int64_t r, int64_t k, int64_t ps) {
    return (r >> 1) * ps + (k >> 6) * 128 + (r & 1) * 64 + (k & 63);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
    int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

// A group's size as the kernels use it, from the size the caller gave (lane
// g of a full wave holds group g's): a negative size counts as 0, and sizes
// whose running total passes `rows` are cut at it.  Sizes that are >= 0 and
// sum to rows come through unchanged; any others still keep every group
// inside the rows the buffers hold.  (The running total is taken in 64 bits:
// raw sizes may sum past 2^31.)
__device__ __forceinline__ int clamp_group_size(int n, int64_t rows) {
    const int lane = threadIdx.x & 63;
    const int64_t v = n > 0 ? n : 0;
    int64_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    const int64_t excl = incl - v;
    return (int)((incl < rows ? incl : rows) - (excl < rows ? excl : rows));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
