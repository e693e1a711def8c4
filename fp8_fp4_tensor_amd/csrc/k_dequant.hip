// k_dequant.hip -- dequantization back to fp32 or bf16: the code's value
// times the scale of its tensor or block, one fp32 multiply rounded to
// nearest even (and, for bf16 output, one rounding of that fp32 to bf16).
//
// Sources: [CS] "FP8 Current Scaling：量化、缩放与精度边界"
// (notes.kuangjux.top), section "Current Scaling" (restored value = q * s)
// and section "实现接口与精度边界" (a quantized tensor supports dequantize);
// [MP] "混合精度训练：fp16 到 fp8" (garden.houmin.site), section "MXFP8"
// (value = element x block scale; E4M3 or E5M2 elements) and section
// "NVFP4"; [LP] "从 BF16 到 FP8/FP4" section 2.4 (MXFP4).
//
// Bandwidth layout: a thread step is 16 elements (16 code bytes, or 8 packed
// FP4 bytes) read with one vector load and written as 64 (fp32) or 32 (bf16)
// contiguous bytes. Per-tensor codes are treated as a flat array; block
// recipes walk rows (a workgroup per row, threads across it), so every
// 16-element step lies inside one block and takes one scale, with no
// division per element. Codes decode exactly with the gfx950 converters.
#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace fq {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kGrid = 8192;

enum : int { kDqE4M3 = 0, kDqE5M2 = 1, kDqFp4 = 2 };

// 16 codes (one dword per four FP8 codes, or two FP4 nibbles per byte) -> 16 floats
template <int CODE>
__device__ __forceinline__ void decode16(const uint32_t* w, float* f)
{
    if constexpr (CODE == kDqFp4) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 0);
            const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 1);
            const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 2);
            const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 3);
            f[8 * d] = v0[0];
            f[8 * d + 1] = v0[1];
            f[8 * d + 2] = v1[0];
            f[8 * d + 3] = v1[1];
            f[8 * d + 4] = v2[0];
            f[8 * d + 5] = v2[1];
            f[8 * d + 6] = v3[0];
            f[8 * d + 7] = v3[1];
        }
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            f32x2 lo, hi;
            if constexpr (CODE == kDqE4M3) {
                lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], false);
                hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], true);
            } else {
                lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w[d], false);
                hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w[d], true);
            }
            f[4 * d] = lo[0];
            f[4 * d + 1] = lo[1];
            f[4 * d + 2] = hi[0];
            f[4 * d + 3] = hi[1];
        }
    }
}

// 16 codes of a step: FP8 codes are 16 bytes, FP4 codes 8 bytes
template <int CODE>
__device__ __forceinline__ void load_codes(const uint8_t* q, int64_t step, uint32_t* w)
{
    if constexpr (CODE == kDqFp4) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(q + step * 8));
        w[0] = v[0];
        w[1] = v[1];
    } else {
        const u32x4 v = ld16_stream(q + step * 16);
        w[0] = v[0];
        w[1] = v[1];
        w[2] = v[2];
        w[3] = v[3];
    }
}

// 16 values times sc -> y[step*16 .. +16), fp32 or bf16
template <bool BF16>
__device__ __forceinline__ void store16(void* y, int64_t step, const float* f, float sc)
{
    if constexpr (BF16) {
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            bf16x2 b;
            b[0] = (__bf16)(f[2 * k] * sc);
            b[1] = (__bf16)(f[2 * k + 1] * sc);
            h[k] = __builtin_bit_cast(uint32_t, b);
        }
        uint8_t* p = reinterpret_cast<uint8_t*>(y) + step * 32;
        st16_stream(p, u32x4{h[0], h[1], h[2], h[3]});
        st16_stream(p + 16, u32x4{h[4], h[5], h[6], h[7]});
    } else {
        uint8_t* p = reinterpret_cast<uint8_t*>(y) + step * 64;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            st16_stream(p + 16 * k, u32x4{__float_as_uint(f[4 * k] * sc), __float_as_uint(f[4 * k + 1] * sc),
                                          __float_as_uint(f[4 * k + 2] * sc), __float_as_uint(f[4 * k + 3] * sc)});
    }
}

template <bool BF16>
__device__ __forceinline__ void store1(void* y, int64_t i, float v)
{
    if constexpr (BF16)
        reinterpret_cast<__bf16*>(y)[i] = (__bf16)v;
    else
        reinterpret_cast<float*>(y)[i] = v;
}

// Per-tensor: flat codes, one scale.
template <int CODE, bool BF16>
__global__ __launch_bounds__(kWG) void k_dq_tensor(const uint8_t* __restrict__ q, int64_t n, const float* s,
                                                   void* __restrict__ y)
{
    const float sc = *s;
    const int64_t nsteps = n / 16;
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < nsteps; i += (int64_t)gridDim.x * kWG) {
        uint32_t w[4];
        float f[16];
        load_codes<CODE>(q, i, w);
        decode16<CODE>(w, f);
        store16<BF16>(y, i, f, sc);
    }
    for (int64_t i = nsteps * 16 + (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) {
        const float v = CODE == kDqE4M3 ? dec_e4m3(q[i]) : dec_e5m2(q[i]);
        store1<BF16>(y, i, v * sc);
    }
}

// Block scales (fp32, MX E8M0, NVFP4 E4M3 x S): a workgroup per row.
// SKIND: 0 fp32 scale plane, 1 E8M0 codes, 2 E4M3 codes times the tensor scale.
template <int CODE, int SKIND, bool BF16>
__global__ __launch_bounds__(kWG) void k_dq_rows(const uint8_t* __restrict__ q, const void* __restrict__ scales,
                                                 const float* S, int64_t R, int64_t C, int br, int bc,
                                                 void* __restrict__ y)
{
    const int64_t steps_per_row = C / 16, nbc = C / bc;
    const float Sv = SKIND == 2 ? *S : 1.0f;
    for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
        const int64_t srow = (r / br) * nbc;
        for (int64_t j = threadIdx.x; j < steps_per_row; j += kWG) {
            const int64_t step = r * steps_per_row + j;
            const int64_t si = srow + (16 * j) / bc;
            float sc;
            if constexpr (SKIND == 0)
                sc = reinterpret_cast<const float*>(scales)[si];
            else if constexpr (SKIND == 1)
                sc = e8m0_value(reinterpret_cast<const uint8_t*>(scales)[si]);
            else
                sc = dec_e4m3(reinterpret_cast<const uint8_t*>(scales)[si]) * Sv;
            uint32_t w[4];
            float f[16];
            load_codes<CODE>(q, step, w);
            decode16<CODE>(w, f);
            store16<BF16>(y, step, f, sc);
        }
    }
}

int grid_for(int64_t n) { return (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, kWG), kGrid)); }

template <int CODE, int SKIND>
void rows_t(const uint8_t* q, const void* s, const float* S, int64_t R, int64_t C, int br, int bc, void* y, int bf,
            hipStream_t stream)
{
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(R, kGrid));
    if (bf)
        k_dq_rows<CODE, SKIND, true><<<grid, kWG, 0, stream>>>(q, s, S, R, C, br, bc, y);
    else
        k_dq_rows<CODE, SKIND, false><<<grid, kWG, 0, stream>>>(q, s, S, R, C, br, bc, y);
}

}  // namespace

hipError_t launch_dequant_tensor(const uint8_t* q, int fmt, int64_t n, const float* s, void* y, int bf,
                                 hipStream_t stream)
{
    const int grid = grid_for(n / 16 + 1);
    if (fmt == kE4M3) {
        if (bf)
            k_dq_tensor<kDqE4M3, true><<<grid, kWG, 0, stream>>>(q, n, s, y);
        else
            k_dq_tensor<kDqE4M3, false><<<grid, kWG, 0, stream>>>(q, n, s, y);
    } else {
        if (bf)
            k_dq_tensor<kDqE5M2, true><<<grid, kWG, 0, stream>>>(q, n, s, y);
        else
            k_dq_tensor<kDqE5M2, false><<<grid, kWG, 0, stream>>>(q, n, s, y);
    }
    return hipGetLastError();
}

hipError_t launch_dequant_block(const uint8_t* q, const float* s, int64_t R, int64_t C, int br, int bc, void* y,
                                int bf, hipStream_t stream)
{
    rows_t<kDqE4M3, 0>(q, s, nullptr, R, C, br, bc, y, bf, stream);
    return hipGetLastError();
}

hipError_t launch_dequant_mx(const uint8_t* q, const uint8_t* e, int fmt, int64_t R, int64_t C, void* y, int bf,
                             hipStream_t stream)
{
    if (fmt == kE2M1)
        rows_t<kDqFp4, 1>(q, e, nullptr, R, C, 1, 32, y, bf, stream);
    else if (fmt == kE5M2)
        rows_t<kDqE5M2, 1>(q, e, nullptr, R, C, 1, 32, y, bf, stream);
    else
        rows_t<kDqE4M3, 1>(q, e, nullptr, R, C, 1, 32, y, bf, stream);
    return hipGetLastError();
}

hipError_t launch_dequant_nvfp4(const uint8_t* p, const uint8_t* codes, const float* S, int64_t R, int64_t C, int br,
                                int bc, void* y, int bf, hipStream_t stream)
{
    rows_t<kDqFp4, 2>(p, codes, S, R, C, br, bc, y, bf, stream);
    return hipGetLastError();
}

}  // namespace fq
