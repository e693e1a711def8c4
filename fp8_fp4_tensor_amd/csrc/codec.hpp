// codec.hpp -- device-side element codecs and wave reductions for gfx950.
//
// Sources (short labels as in include/fq.h):
//   [MP]  "混合精度训练：fp16 到 fp8" (garden.houmin.site)
//   [CS]  "FP8 Current Scaling：量化、缩放与精度边界" (notes.kuangjux.top)
//   [LP]  "从 BF16 到 FP8/FP4：大语言模型低精度训练与混合精度预训练" (r00kie-liu.github.io)
//
// Arithmetic contract (the library is built with -ffp-contract=off and
// without fast-math, so each of these is one IEEE fp32 operation rounded to
// nearest even; fp32 denormals are preserved, the gfx950 default):
//   - scales are correctly rounded fp32 quotients (Fmax/a and a/Fmax);
//   - the scaled value y = fp32(x * alpha) is one multiply;
//   - y is clamped to +-Fmax with v_med3_f32, so the hardware converters
//     never see an out-of-range value: the encode saturates;
//   - the gfx950 converters (v_cvt_pk_fp8_f32 for OCP E4M3,
//     v_cvt_pk_bf8_f32 for OCP E5M2, v_cvt_scalef32_pk_fp4_f32 with a unit
//     scale for E2M1) round to nearest even and keep the sign of zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fq {

constexpr int kWG = 256;  // threads per workgroup: 4 wave64s

enum : int { kE4M3 = 0, kE5M2 = 1, kE2M1 = 2 };

constexpr float kFLT_MAX = 3.40282346638528859812e+38f;

__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <int FMT>
struct Fmt;
// kMax: largest finite value; kEmax = floor(log2 kMax); kMantBf16: the 7
// mantissa bits of kMax as a bf16 (448 and 57344 are 1.75 * 2^e, 6 is 1.5 * 2^2)
template <>
struct Fmt<kE4M3> {
    static constexpr float kMax = 448.0f;
    static constexpr int kEmax = 8;
    static constexpr uint32_t kMantBf16 = 0x60u;
};
template <>
struct Fmt<kE5M2> {
    static constexpr float kMax = 57344.0f;
    static constexpr int kEmax = 15;
    static constexpr uint32_t kMantBf16 = 0x60u;
};
template <>
struct Fmt<kE2M1> {
    static constexpr float kMax = 6.0f;
    static constexpr int kEmax = 2;
    static constexpr uint32_t kMantBf16 = 0x40u;
};

// ---------------------------------------------------------------- bf16
// bf16 widens to fp32 exactly: its 16 bits are the top half of the fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- cross-lane max
// DPP controls (GFX9 encoding).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over aligned groups of 2, 4, 8 or 16 lanes; every lane of the group
// receives the group max.
__device__ __forceinline__ float max_lanes2(float v) { return fmaxf(v, dpp<kDppXor1>(v)); }
__device__ __forceinline__ float max_lanes4(float v)
{
    v = fmaxf(v, dpp<kDppXor1>(v));
    return fmaxf(v, dpp<kDppXor2>(v));
}
__device__ __forceinline__ float max_lanes16(float v)
{
    v = max_lanes4(v);
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    return fmaxf(v, dpp<kDppMirror>(v));
}
// Max over the whole wave64; every lane receives it.
__device__ __forceinline__ float max_wave(float v)
{
    v = max_lanes16(v);
    v = fmaxf(v, __shfl_xor(v, 16));
    return fmaxf(v, __shfl_xor(v, 32));
}

// This thread's max over amax partials p[0 .. n-1], n <= 4 * kWG: the four
// loads are issued together, so one memory latency covers them.
__device__ __forceinline__ float partials_max(const float* p, int n)
{
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = (int)threadIdx.x + k * kWG;
        v[k] = i < n ? p[i] : 0.0f;
    }
    return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
}

// A workgroup barrier that orders LDS accesses only. __syncthreads() also
// waits for the wave's outstanding global loads and stores (on gfx9 stores
// count in the same counter as loads); this one waits for its LDS operations
// alone, so a tile's global stores stay in flight while the next tile is
// staged. Only for kernels that never read back, within the launch, global
// memory they wrote. Call from uniform control flow.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Max over a 256-thread workgroup; every thread receives it. `lds` holds 4
// floats. Contains __syncthreads(): call from uniform control flow.
__device__ __forceinline__ float max_workgroup(float v, float* lds)
{
    v = max_wave(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();  // lds may still be read by an earlier call
    if ((threadIdx.x & 63) == 0)
        lds[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(lds[0], lds[1]), fmaxf(lds[2], lds[3]));
}

// ---------------------------------------------------------------- scales
// Per-unit scales from an amax a ([CS] "Current Scaling": alpha = Fmax/a
// multiplies before the cast, s = a/Fmax restores; [MP] "FP8 recipe": a
// unit's amax maps to the format's largest value). a = 0 gives 1 and 1; an
// alpha beyond fp32 range is held at FLT_MAX.
__device__ __forceinline__ void tensor_scales(float a, float fmax_v, float& alpha, float& s)
{
    if (a == 0.0f) {
        alpha = 1.0f;
        s = 1.0f;
    } else {
        alpha = fminf(fmax_v / a, kFLT_MAX);
        s = a / fmax_v;
    }
}

// ---------------------------------------------------------------- encode
__device__ __forceinline__ float clampf(float y, float m) { return __builtin_amdgcn_fmed3f(y, -m, m); }

// Two clamped fp32 values -> two FP8 codes written into byte pair HI (0: bytes
// 0,1; 1: bytes 2,3) of `old`; the first value takes the lower byte.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt2(float a, float b, uint32_t old)
{
    if constexpr (FMT == kE4M3)
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
    else
        return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

// Four fp32 values, scaled by alpha, clamped and encoded into one dword
// (value k in byte k).
template <int FMT>
__device__ __forceinline__ uint32_t enc4(float v0, float v1, float v2, float v3, float alpha)
{
    constexpr float M = Fmt<FMT>::kMax;
    const float y0 = clampf(v0 * alpha, M), y1 = clampf(v1 * alpha, M);
    const float y2 = clampf(v2 * alpha, M), y3 = clampf(v3 * alpha, M);
    uint32_t w = cvt2<FMT, false>(y0, y1, 0u);
    return cvt2<FMT, true>(y2, y3, w);
}

// One E4M3 code (low byte) of a non-negative, already-clamped value.
__device__ __forceinline__ uint32_t enc_e4m3_one(float y)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFFu;
}

// E4M3 code -> fp32 (exact).
__device__ __forceinline__ float dec_e4m3(uint32_t code) { return __builtin_amdgcn_cvt_f32_fp8((int)code, 0); }
__device__ __forceinline__ float dec_e5m2(uint32_t code) { return __builtin_amdgcn_cvt_f32_bf8((int)code, 0); }

// Eight fp32 values, each multiplied by r and clamped to +-6, encoded as
// E2M1 nibbles packed into one dword: value k in bits 4k+3..4k.
__device__ __forceinline__ uint32_t enc8_e2m1(const float* v, float r)
{
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clampf(v[0] * r, 6.0f), clampf(v[1] * r, 6.0f), 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clampf(v[2] * r, 6.0f), clampf(v[3] * r, 6.0f), 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clampf(v[4] * r, 6.0f), clampf(v[5] * r, 6.0f), 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clampf(v[6] * r, 6.0f), clampf(v[7] * r, 6.0f), 1.0f, 3);
    return w;
}

// E2M1 nibble -> fp32 (exact).
__device__ __forceinline__ float dec_e2m1(uint32_t nib)
{
    const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    const float m = mag[nib & 7u];
    return (nib & 8u) ? -m : m;
}

// ---------------------------------------------------------------- MX scale
// E8M0 code of a block amax a: 2^(floor(log2 a) - emax) held to
// [2^-127, 2^127], emax = floor(log2 Fmax) of the element format (8 for
// E4M3, 15 for E5M2, 2 for E2M1) ([MP] "MXFP8": a 32-element block shares
// one power-of-two E8M0 scale; [LP] 2.4: MXFP4 likewise with E2M1).
// From the fp32 bits: floor(log2 a) = E - 127 for the exponent field E of a
// normal a, so code = max(E - emax, 0); subnormal a (E = 0) and a = 0 give 0.
template <int FMT = kE4M3>
__device__ __forceinline__ uint32_t mx_code(float a)
{
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu);
    return (uint32_t)max(e - Fmt<FMT>::kEmax, 0);
}
// The fp32 multiplier 2^(127 - code) that scales a block into the element
// range; for code in [0, 253] it is a normal fp32 power of two, so x * it is
// exact unless the product leaves the normal range.
__device__ __forceinline__ float mx_multiplier(uint32_t code) { return __uint_as_float((254u - code) << 23); }
// 2^(code - 127) as fp32 (code 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t code)
{
    return code == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(code << 23);
}

// ---------------------------------------------------------------- tiles
// Tile t of a grid of tiles ntc wide -> its tile row tr and column tc.
// Tensors hold at most 2^36 elements, so tile indices and counts stay below
// 2^32 and one 32-bit division does (a 64-bit one costs about a hundred
// scalar instructions per tile).
__device__ __forceinline__ void tile_coords(int64_t t, int64_t ntc, int64_t& tr, int64_t& tc)
{
    const uint32_t q = (uint32_t)t / (uint32_t)ntc;
    tr = q;
    tc = t - (int64_t)q * ntc;
}

// ---------------------------------------------------------------- memory
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld16_stream(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }
__device__ __forceinline__ void st8_stream(void* p, u32x2 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p)); }
__device__ __forceinline__ void st4_stream(void* p, uint32_t v) { __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p)); }

// Input element types: fp32 (float) or bf16 (its bits, uint16_t).
// kE = elements per 16-byte load.
template <typename T>
struct In;
template <>
struct In<float> {
    static constexpr int kE = 4;
    __device__ static __forceinline__ void unpack(u32x4 v, float* f)
    {
        f[0] = __uint_as_float(v[0]);
        f[1] = __uint_as_float(v[1]);
        f[2] = __uint_as_float(v[2]);
        f[3] = __uint_as_float(v[3]);
    }
    __device__ static __forceinline__ float load1(const float* x, int64_t i) { return x[i]; }
    // max |x| over the four values of a load
    __device__ static __forceinline__ float absmax16(u32x4 v)
    {
        return fmaxf(fmaxf(fabsf(__uint_as_float(v[0])), fabsf(__uint_as_float(v[1]))),
                     fmaxf(fabsf(__uint_as_float(v[2])), fabsf(__uint_as_float(v[3]))));
    }
};
template <>
struct In<uint16_t> {
    static constexpr int kE = 8;
    __device__ static __forceinline__ void unpack(u32x4 v, float* f)
    {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = bf16_lo(v[k]);
            f[2 * k + 1] = bf16_hi(v[k]);
        }
    }
    __device__ static __forceinline__ float load1(const uint16_t* x, int64_t i)
    {
        return __uint_as_float((uint32_t)x[i] << 16);
    }
    // max |x| over the eight values of a load, on the bits: for finite bf16
    // the magnitude bits (sign cleared) order exactly as the magnitudes, so
    // a 16-bit integer max (two lanes per dword) is the float max. No value
    // is unpacked, so nothing from this pass stays live in registers.
    __device__ static __forceinline__ float absmax16(u32x4 v)
    {
        typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
        u16x2 m = __builtin_bit_cast(u16x2, v[0] & 0x7fff7fffu);
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v[1] & 0x7fff7fffu));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v[2] & 0x7fff7fffu));
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v[3] & 0x7fff7fffu));
        return __uint_as_float((uint32_t)(m[0] > m[1] ? m[0] : m[1]) << 16);
    }
};

// max |f[k]| over E values
template <int E>
__device__ __forceinline__ float absmax(const float* f)
{
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < E; ++k)
        m = fmaxf(m, fabsf(f[k]));
    return m;
}

// Max over aligned groups of N lanes (N in 1, 2, 4, 8, 16, 32, 64).
template <int N>
__device__ __forceinline__ float max_lanes(float v)
{
    if constexpr (N >= 2)
        v = fmaxf(v, dpp<kDppXor1>(v));
    if constexpr (N >= 4)
        v = fmaxf(v, dpp<kDppXor2>(v));
    if constexpr (N >= 8)
        v = fmaxf(v, dpp<kDppHalfMirror>(v));
    if constexpr (N >= 16)
        v = fmaxf(v, dpp<kDppMirror>(v));
    if constexpr (N >= 32)
        v = fmaxf(v, __shfl_xor(v, 16));
    if constexpr (N >= 64)
        v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// E scaled values -> E FP8 codes (E = 4: one dword; E = 8: two dwords).
template <int FMT, int E>
struct Enc8;
template <int FMT>
struct Enc8<FMT, 4> {
    __device__ static __forceinline__ void store(uint8_t* q, const float* f, float alpha)
    {
        st4_stream(q, enc4<FMT>(f[0], f[1], f[2], f[3], alpha));
    }
};
template <int FMT>
struct Enc8<FMT, 8> {
    __device__ static __forceinline__ void store(uint8_t* q, const float* f, float alpha)
    {
        u32x2 w;
        w[0] = enc4<FMT>(f[0], f[1], f[2], f[3], alpha);
        w[1] = enc4<FMT>(f[4], f[5], f[6], f[7], alpha);
        st8_stream(q, w);
    }
};

// One scaled value -> its FP8 code.
template <int FMT>
__device__ __forceinline__ uint8_t enc1(float v, float alpha)
{
    return (uint8_t)(cvt2<FMT, false>(clampf(v * alpha, Fmt<FMT>::kMax), 0.0f, 0u) & 0xFFu);
}

// ---------------------------------------------------------------- stochastic rounding
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): the published multipliers and Weyl constants.
// Each round's two 32 x 32 -> 64-bit products are one v_mad_u64_u32 each,
// and each three-way xor one v_bitop3_b32 (truth table 0x96 = a ^ b ^ c).
constexpr uint32_t kPhM0 = 0xD2511F53u, kPhM1 = 0xCD9E8D57u;
constexpr uint32_t kPhW0 = 0x9E3779B9u, kPhW1 = 0xBB67AE85u;

struct Philox4 {
    uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1)
{
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint64_t p0 = (uint64_t)kPhM0 * c0, p1 = (uint64_t)kPhM1 * c2;
        c0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        c1 = (uint32_t)p1;
        c2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c3 = (uint32_t)p0;
        k0 += kPhW0;
        k1 += kPhW1;
    }
    return Philox4{{c0, c1, c2, c3}};
}

// The random bits of elements 8h .. 8h+7 of a plane: one call with counter
// (h, s) as 32-bit words and key = seed, s = 2 * offset + plane.
__device__ __forceinline__ Philox4 sr_group(uint64_t h, uint64_t s, uint64_t seed)
{
    return philox4x32_10((uint32_t)h, (uint32_t)(h >> 32), (uint32_t)s, (uint32_t)(s >> 32), (uint32_t)seed,
                         (uint32_t)(seed >> 32));
}

// Stochastic rounding of one clamped fp32 value y to E4M3 / E5M2 with the
// 16 random bits u16 (bits 15..0): gfx950's v_cvt_scalef32_sr_fp8_f32 /
// _bf8_f32 at unit scale add the bits of their random word below the last
// kept bit and truncate, so a word whose bits 31..16 are u16 (15..0 zero)
// rounds up iff u16 + g * 2^16 >= 2^16 (g the position between the two
// neighbours), the add-and-truncate rounding with 16 random bits. Only
// byte 0 of the result is used.
template <int FMT>
__device__ __forceinline__ uint32_t sr8_byte0(float y, uint32_t u16)
{
    if constexpr (FMT == kE4M3)
        return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0, y, u16 << 16, 1.0f, 0);
    else
        return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_bf8_f32(0, y, u16 << 16, 1.0f, 0);
}

// Byte 0 of each of four words -> one dword, word k in byte k.
__device__ __forceinline__ uint32_t gather_byte0(uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3)
{
    // v_perm_b32(a, b, sel): selector byte i picks byte sel_i of {a:b} (0..3 from b, 4..7 from a), 0x0c gives 0
    return __builtin_amdgcn_perm(t1, t0, 0x0c0c0400u) | __builtin_amdgcn_perm(t3, t2, 0x04000c0cu);
}

}  // namespace fq
