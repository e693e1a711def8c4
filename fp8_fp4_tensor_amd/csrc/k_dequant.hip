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
// Bandwidth layout: a lane chunk is the elements of 16 output bytes (8 for
// bf16, 4 for fp32), so each store instruction of a wave writes 1 KiB of
// contiguous output; lanes keep several chunks' loads in flight. Per-tensor
// codes are treated as a flat array; block recipes give a workgroup a row,
// and every chunk lies inside one block and takes one scale, with no
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

// A lane chunk is G elements whose output is exactly 16 bytes: G = 8 for
// bf16 output, 4 for fp32. Consecutive lanes take consecutive chunks, so a
// wave's store instruction writes 1 KiB of contiguous output (whole lines;
// streaming stores of lines a lane only partly covers each became
// partial-line writes and ran 2-4x slower). Chunks lie inside one block.
template <bool BF16>
constexpr int chunk_elems() { return BF16 ? 8 : 4; }
constexpr int kChunks = 4;  // chunks per lane with loads in flight

// G codes starting at element e (FP8: G bytes; FP4: G/2 bytes), zero-extended into w
template <int CODE, int G>
__device__ __forceinline__ void load_chunk(const uint8_t* q, int64_t e, uint32_t* w)
{
    if constexpr (CODE == kDqFp4) {
        if constexpr (G == 8)
            w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(q + e / 2));
        else
            w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(q + e / 2));
    } else {
        if constexpr (G == 8) {
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(q + e));
            w[0] = v[0];
            w[1] = v[1];
        } else {
            w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(q + e));
        }
    }
}

// G codes -> G floats, exact (gfx950 converters; FP4 byte_sel must be a constant)
template <int CODE, int G>
__device__ __forceinline__ void decode_chunk(const uint32_t* w, float* f)
{
    if constexpr (CODE == kDqFp4) {
        f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[0], 1.0f, 0);
        f[0] = v[0];
        f[1] = v[1];
        v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[0], 1.0f, 1);
        f[2] = v[0];
        f[3] = v[1];
        if constexpr (G == 8) {
            v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[0], 1.0f, 2);
            f[4] = v[0];
            f[5] = v[1];
            v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[0], 1.0f, 3);
            f[6] = v[0];
            f[7] = v[1];
        }
    } else {
#pragma unroll
        for (int d = 0; d < G / 4; ++d) {
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

// G values times sc -> 16 bytes of y at element e (bf16: one RTNE rounding of the fp32 product)
template <bool BF16>
__device__ __forceinline__ void store_chunk(void* y, int64_t e, const float* f, float sc)
{
    if constexpr (BF16) {
        uint32_t h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            bf16x2 b;
            b[0] = (__bf16)(f[2 * k] * sc);
            b[1] = (__bf16)(f[2 * k + 1] * sc);
            h[k] = __builtin_bit_cast(uint32_t, b);
        }
        st16_stream(reinterpret_cast<uint8_t*>(y) + e * 2, u32x4{h[0], h[1], h[2], h[3]});
    } else {
        st16_stream(reinterpret_cast<uint8_t*>(y) + e * 4,
                    u32x4{__float_as_uint(f[0] * sc), __float_as_uint(f[1] * sc), __float_as_uint(f[2] * sc),
                          __float_as_uint(f[3] * sc)});
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

// Per-tensor: flat codes, one scale; kTensorChunks chunks per lane per
// round, the round's loads issued before any decode.
constexpr int kTensorChunks = 8;

template <int CODE, bool BF16>
__global__ __launch_bounds__(kWG) void k_dq_tensor(const uint8_t* __restrict__ q, int64_t n, const float* s,
                                                   void* __restrict__ y)
{
    constexpr int G = chunk_elems<BF16>(), kChunks = kTensorChunks;
    const float sc = *s;
    const int64_t nch = n / G, nthreads = (int64_t)gridDim.x * kWG;
    const int64_t t = (int64_t)blockIdx.x * kWG + threadIdx.x;
    for (int64_t base = t; base < nch; base += nthreads * kChunks) {
        uint32_t w[kChunks][2];
#pragma unroll
        for (int k = 0; k < kChunks; ++k)
            if (base + k * nthreads < nch)
                load_chunk<CODE, G>(q, (base + k * nthreads) * G, w[k]);
#pragma unroll
        for (int k = 0; k < kChunks; ++k) {
            const int64_t i = base + k * nthreads;
            if (i < nch) {
                float f[G];
                decode_chunk<CODE, G>(w[k], f);
                store_chunk<BF16>(y, i * G, f, sc);
            }
        }
    }
    for (int64_t i = nch * G + t; i < n; i += nthreads) {
        const float v = CODE == kDqE4M3 ? dec_e4m3(q[i]) : dec_e5m2(q[i]);
        store1<BF16>(y, i, v * sc);
    }
}

// Block scales (fp32, MX E8M0, NVFP4 E4M3 x S): a workgroup per row, lanes
// across it in chunks; a chunk lies inside one block (C % 16 == 0, blocks 16,
// 32 or 128 wide), so it takes one scale.
// SKIND: 0 fp32 scale plane, 1 E8M0 codes, 2 E4M3 codes times the tensor scale.
// Block sizes are powers of two, passed as shifts (no integer division).
template <int CODE, int SKIND, bool BF16>
__global__ __launch_bounds__(kWG) void k_dq_rows(const uint8_t* __restrict__ q, const void* __restrict__ scales,
                                                 const float* S, int64_t R, int64_t C, int br_shift, int bc_shift,
                                                 void* __restrict__ y)
{
    constexpr int G = chunk_elems<BF16>();
    const int64_t cpr = C / G, nbc = C >> bc_shift;
    const float Sv = SKIND == 2 ? *S : 1.0f;
    for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
        const int64_t srow = (r >> br_shift) * nbc;
        for (int64_t j0 = threadIdx.x; j0 < cpr; j0 += kWG * kChunks) {
            uint32_t w[kChunks][2];
            float sc[kChunks];
#pragma unroll
            for (int k = 0; k < kChunks; ++k) {
                const int64_t j = j0 + k * kWG;
                if (j < cpr) {
                    load_chunk<CODE, G>(q, r * C + j * G, w[k]);
                    const int64_t si = srow + ((j * G) >> bc_shift);
                    if constexpr (SKIND == 0)
                        sc[k] = reinterpret_cast<const float*>(scales)[si];
                    else if constexpr (SKIND == 1)
                        sc[k] = e8m0_value(reinterpret_cast<const uint8_t*>(scales)[si]);
                    else
                        sc[k] = dec_e4m3(reinterpret_cast<const uint8_t*>(scales)[si]) * Sv;
                }
            }
#pragma unroll
            for (int k = 0; k < kChunks; ++k) {
                const int64_t j = j0 + k * kWG;
                if (j < cpr) {
                    float f[G];
                    decode_chunk<CODE, G>(w[k], f);
                    store_chunk<BF16>(y, r * C + j * G, f, sc[k]);
                }
            }
        }
    }
}

int grid_for(int64_t n) { return (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, kWG), kGrid)); }

template <int CODE, int SKIND>
void rows_t(const uint8_t* q, const void* s, const float* S, int64_t R, int64_t C, int br, int bc, void* y, int bf,
            hipStream_t stream)
{
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(R, kGrid));
    const int brs = __builtin_ctz((unsigned)br), bcs = __builtin_ctz((unsigned)bc);  // powers of two
    if (bf)
        k_dq_rows<CODE, SKIND, true><<<grid, kWG, 0, stream>>>(q, s, S, R, C, brs, bcs, y);
    else
        k_dq_rows<CODE, SKIND, false><<<grid, kWG, 0, stream>>>(q, s, S, R, C, brs, bcs, y);
}

}  // namespace

hipError_t launch_dequant_tensor(const uint8_t* q, int fmt, int64_t n, const float* s, void* y, int bf,
                                 hipStream_t stream)
{
    // a grid that gives every lane kTensorChunks chunks of G elements (8192 x
    // 4096 to bf16: 23.1 -> 22.2 us per cold call against 4 chunks of half
    // the intended count)
    const int grid = grid_for(cdiv(n / (bf ? chunk_elems<true>() : chunk_elems<false>()), kTensorChunks) + 1);
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
