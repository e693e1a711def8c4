// k_dequant.hip -- dequantization back to fp32: the code's value times the
// scale of its tensor or block, one fp32 multiply rounded to nearest even.
//
// Sources: [CS] "FP8 Current Scaling：量化、缩放与精度边界"
// (notes.kuangjux.top), section "Current Scaling" (restored value = q * s)
// and section "实现接口与精度边界" (a quantized tensor supports dequantize);
// [MP] "混合精度训练：fp16 到 fp8" (garden.houmin.site), section "MXFP8"
// (value = element x block scale).
//
// These kernels check results and restore values; they are simple
// grid-stride loops with one element per thread step.
#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace fq {
namespace {

constexpr int kGrid = 2048;

template <int FMT>
__global__ __launch_bounds__(kWG) void k_dq_tensor(const uint8_t* __restrict__ q, int64_t n, const float* s,
                                                   float* __restrict__ y)
{
    const float sc = *s;
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) {
        const float v = FMT == kE4M3 ? dec_e4m3(q[i]) : dec_e5m2(q[i]);
        y[i] = v * sc;
    }
}

__global__ __launch_bounds__(kWG) void k_dq_block(const uint8_t* __restrict__ q, const float* __restrict__ s,
                                                  int64_t R, int64_t C, int br, int bc, float* __restrict__ y)
{
    const int64_t n = R * C, nbc = C / bc;
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) {
        const int64_t r = i / C, c = i % C;
        y[i] = dec_e4m3(q[i]) * s[(r / br) * nbc + c / bc];
    }
}

__global__ __launch_bounds__(kWG) void k_dq_mx(const uint8_t* __restrict__ q, const uint8_t* __restrict__ e,
                                               int64_t R, int64_t C, float* __restrict__ y)
{
    const int64_t n = R * C;
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) {
        const int64_t r = i / C, c = i % C;
        y[i] = dec_e4m3(q[i]) * e8m0_value(e[r * (C / 32) + c / 32]);
    }
}

__global__ __launch_bounds__(kWG) void k_dq_nvfp4(const uint8_t* __restrict__ p, const uint8_t* __restrict__ codes,
                                                  const float* S, int64_t R, int64_t C, int br, int bc,
                                                  float* __restrict__ y)
{
    const float Sv = *S;
    const int64_t n = R * C, nbc = C / bc;
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) {
        const int64_t r = i / C, c = i % C;
        const uint32_t byte = p[r * (C / 2) + c / 2];
        const uint32_t nib = (c & 1) ? (byte >> 4) : (byte & 0xFu);
        const float d = dec_e4m3(codes[(r / br) * nbc + c / bc]) * Sv;
        y[i] = dec_e2m1(nib) * d;
    }
}

int grid_for(int64_t n) { return (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, kWG), kGrid)); }

}  // namespace

hipError_t launch_dequant_tensor(const uint8_t* q, int fmt, int64_t n, const float* s, float* y,
                                 hipStream_t stream)
{
    if (fmt == kE4M3)
        k_dq_tensor<kE4M3><<<grid_for(n), kWG, 0, stream>>>(q, n, s, y);
    else
        k_dq_tensor<kE5M2><<<grid_for(n), kWG, 0, stream>>>(q, n, s, y);
    return hipGetLastError();
}

hipError_t launch_dequant_block(const uint8_t* q, const float* s, int64_t R, int64_t C, int br, int bc, float* y,
                                hipStream_t stream)
{
    k_dq_block<<<grid_for(R * C), kWG, 0, stream>>>(q, s, R, C, br, bc, y);
    return hipGetLastError();
}

hipError_t launch_dequant_mx(const uint8_t* q, const uint8_t* e, int64_t R, int64_t C, float* y, hipStream_t stream)
{
    k_dq_mx<<<grid_for(R * C), kWG, 0, stream>>>(q, e, R, C, y);
    return hipGetLastError();
}

hipError_t launch_dequant_nvfp4(const uint8_t* p, const uint8_t* codes, const float* S, int64_t R, int64_t C,
                                int br, int bc, float* y, hipStream_t stream)
{
    k_dq_nvfp4<<<grid_for(R * C), kWG, 0, stream>>>(p, codes, S, R, C, br, bc, y);
    return hipGetLastError();
}

}  // namespace fq
