// k_mxfp4.hip -- MXFP4: E2M1 elements (two per byte) in 32-element blocks
// that share one E8M0 power-of-two scale; rowwise 1x32 along the rows and
// colwise 32x1 down the columns, stored transposed.
//
// Sources: [LP] "从 BF16 到 FP8/FP4" section 2.4 (MXFP4: 32-element blocks
// with a UE8M0 scale, compared with NVFP4's 16-element E4M3-scaled blocks);
// [MP] "混合精度训练：fp16 到 fp8" section "MXFP8" (the MX block structure:
// value = element x shared power-of-two scale) and section "NVFP4" (the
// float4_e2m1fn_x2 layout: element 2k in bits 3..0, 2k+1 in bits 7..4).
// Block scale 2^e, e = floor(log2 amax) - 2 (2 = floor(log2 6)), held to the
// E8M0 range; q = Q_E2M1(x * 2^-e): the multiply by a power of two is exact,
// then clamp to +-6 and round to nearest even (v_cvt_scalef32_pk_fp4_f32 at
// unit scale).
//
// These kernels serve fp32 inputs; bf16 inputs take the tile kernel
// k_mxfp4_bf16 (k_mx.hip), which makes both planes from one read.
//   k_mxfp4_row  flat: a 1x32 block is eight lanes of fp32, three DPP steps;
//                each lane writes its packed codes.
//   k_mxfp4_col  a 32-row x 256-column slab in LDS; one thread per column
//                owns one 32x1 block and writes its 16 packed bytes of X^T.
#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace fq {
namespace {

constexpr int kLoads = 4;
constexpr int kMaxGrid = 16384;
constexpr int64_t kMaxSlabGrid = int64_t(1) << 16;  // 2^24 work-items at most

// E values times m -> E/2 packed bytes
template <int E>
__device__ __forceinline__ void fp4_store(uint8_t* p, const float* f, float m)
{
    if constexpr (E == 8) {
        st4_stream(p, enc8_e2m1(f, m));
    } else {
        uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, clampf(f[0] * m, 6.0f), clampf(f[1] * m, 6.0f),
                                                              1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clampf(f[2] * m, 6.0f), clampf(f[3] * m, 6.0f), 1.0f, 1);
        *reinterpret_cast<uint16_t*>(p) = (uint16_t)w;
    }
}

template <typename T>
__global__ __launch_bounds__(kWG) void k_mxfp4_row(const T* __restrict__ x, int64_t n, uint8_t* __restrict__ p,
                                                   uint8_t* __restrict__ codes)
{
    constexpr int E = In<T>::kE, U = 64 * E, LPB = 32 / E;
    const int lane = threadIdx.x & 63;
    const int64_t nunits = cdiv(n, U);
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t u0 = wave * kLoads; u0 < nunits; u0 += nwaves * kLoads) {
        u32x4 v[kLoads];
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t e = (u0 + j) * U + lane * E;
            v[j] = (u0 + j < nunits && e < n) ? ld16_stream(x + e) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            if (u0 + j >= nunits)
                break;
            const int64_t e = (u0 + j) * U + lane * E;
            float f[E];
            In<T>::unpack(v[j], f);
            const uint32_t code = mx_code<kE2M1>(max_lanes<LPB>(absmax<E>(f)));
            if (e < n) {
                fp4_store<E>(p + e / 2, f, mx_multiplier(code));
                if ((lane & (LPB - 1)) == 0)
                    codes[e / 32] = (uint8_t)code;
            }
        }
    }
}

// Colwise: 32x1 blocks of X, i.e. 1x32 blocks of X^T [C, R].
template <typename T>
__global__ __launch_bounds__(kWG) void k_mxfp4_col(const T* __restrict__ x, int64_t R, int64_t C,
                                                   uint8_t* __restrict__ pt, uint8_t* __restrict__ ct)
{
    constexpr int TC = 256, E = In<T>::kE, LPR = TC / E, RPR = kWG / LPR;
    __shared__ __align__(16) T tile[32][TC];
    const int64_t ntc = cdiv(C, TC), nslabs = (R / 32) * ntc;
    const int cc = (threadIdx.x % LPR) * E;
    // workgroups stride over the 32 x 256 slabs (the grid is capped)
    for (int64_t t = blockIdx.x; t < nslabs; t += gridDim.x) {
        const int64_t r0 = (t / ntc) * 32, c0 = (t % ntc) * TC;
        __syncthreads();  // the previous slab's LDS reads are done
        for (int rr = threadIdx.x / LPR; rr < 32; rr += RPR) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (c0 + cc < C)
                v = ld16_stream(x + (r0 + rr) * C + c0 + cc);
            *reinterpret_cast<u32x4*>(&tile[rr][cc]) = v;
        }
        __syncthreads();
        const int c = threadIdx.x;
        if (c0 + c >= C)
            continue;
        float f[32];
#pragma unroll
        for (int k = 0; k < 32; ++k)
            f[k] = In<T>::load1(&tile[0][0], (int64_t)k * TC + c);
        const uint32_t code = mx_code<kE2M1>(absmax<32>(f));
        const float m = mx_multiplier(code);
        u32x4 w;
        w[0] = enc8_e2m1(f, m);
        w[1] = enc8_e2m1(f + 8, m);
        w[2] = enc8_e2m1(f + 16, m);
        w[3] = enc8_e2m1(f + 24, m);
        // row c0 + c of X^T: R/2 bytes, a multiple of 16 (R % 32 == 0); an
        // ordinary store, so a line's 16-byte pieces meet in L2
        *reinterpret_cast<u32x4*>(pt + (c0 + c) * (R / 2) + r0 / 2) = w;
        ct[(c0 + c) * (R / 32) + r0 / 32] = (uint8_t)code;
    }
}

template <typename T>
void launch_t(const void* xv, int64_t R, int64_t C, uint8_t* p, uint8_t* codes, uint8_t* pt, uint8_t* codest,
              hipStream_t stream)
{
    const T* x = (const T*)xv;
    constexpr int E = In<T>::kE;
    if (p) {
        const int64_t n = R * C;
        const int64_t per_wg = (int64_t)kWG * E * kLoads;
        const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, per_wg), kMaxGrid));
        k_mxfp4_row<T><<<grid, kWG, 0, stream>>>(x, n, p, codes);
    }
    if (pt) {
        const int64_t grid = std::min<int64_t>((R / 32) * cdiv(C, 256), kMaxSlabGrid);
        k_mxfp4_col<T><<<(unsigned)grid, kWG, 0, stream>>>(x, R, C, pt, codest);
    }
}

}  // namespace

hipError_t launch_mxfp4(const void* x, int in_bf16, int64_t R, int64_t C, uint8_t* q, uint8_t* e, uint8_t* qt,
                        uint8_t* et, hipStream_t stream)
{
    if (R * C == 0)
        return hipSuccess;
    if (in_bf16)
        return launch_mxfp4_bf16((const uint16_t*)x, R, C, q, e, qt, et, stream);
    launch_t<float>(x, R, C, q, e, qt, et, stream);
    return hipGetLastError();
}

}  // namespace fq
