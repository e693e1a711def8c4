// k_mx.hip -- MXFP8: E4M3 elements in 32-element blocks that share one E8M0
// (power-of-two) scale, rowwise (1x32 along a row) and colwise (32x1 down a
// column, stored transposed), both from a single read of the input.
//
// Source: [MP] "混合精度训练：fp16 到 fp8" (garden.houmin.site), section
// "MXFP8" (32-element blocks, one E8M0 scale each, value = element x scale;
// E8M0 is the exponent field of an fp32), "FP8 recipe" item 5 (E4M3, 1x32
// for inputs, gradients and weights) and "MXFP8 recipe" (rowwise and colwise
// copies of each tensor, 1x32 and 32x1).
// Block scale: 2^e with e = floor(log2 amax) - 8 (8 = floor(log2 448)),
// held to the E8M0 range; q = Q_E4M3(x * 2^-e), exact multiply, saturating.
//
// One workgroup per 128x128 tile. Rowwise: each lane holds 16 bytes of a
// row, a quad of lanes is one 1x32 block (bf16), reduced with two DPP steps;
// codes and E8M0 scales are written straight from registers. Colwise: the
// tile's raw inputs go to LDS in the same pass; then each thread owns one
// column and 64 rows (two 32x1 blocks), reads them back (lanes of a wave
// read consecutive columns of one row: no bank conflicts), and writes each
// block's 32 codes as 32 contiguous bytes of the transposed plane.
#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace fq {
namespace {

template <typename T>
constexpr int tile_pitch()
{
    return sizeof(T) == 2 ? 128 + 8 : 128;  // bf16 rows padded by 16 bytes; fp32 fits 64 KiB unpadded
}

template <typename T>
__global__ __launch_bounds__(kWG) void k_mx(const T* __restrict__ x, int64_t R, int64_t C,
                                            uint8_t* __restrict__ q, uint8_t* __restrict__ e,
                                            uint8_t* __restrict__ qt, uint8_t* __restrict__ et)
{
    constexpr int E = In<T>::kE, LPR = 128 / E, RPR = kWG / LPR, ROUNDS = 128 / RPR, LPB = 32 / E;
    constexpr int P = tile_pitch<T>();
    extern __shared__ __align__(16) unsigned char smem[];
    T* tile = reinterpret_cast<T*>(smem);
    const int lane = threadIdx.x & 63;
    const int64_t ntc = cdiv(C, 128);
    const int64_t r0 = (int64_t)(blockIdx.x / ntc) * 128, c0 = (int64_t)(blockIdx.x % ntc) * 128;
    const int cc = (threadIdx.x % LPR) * E, rr0 = threadIdx.x / LPR;
    const bool col_in = c0 + cc < C;
    u32x4 v[ROUNDS];
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
        const int64_t r = r0 + rr0 + k * RPR;
        v[k] = (col_in && r < R) ? ld16_stream(x + r * C + c0 + cc) : u32x4{0u, 0u, 0u, 0u};
    }
    const int64_t nbc = C / 32;
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
        const int rr = rr0 + k * RPR;
        if (qt)
            *reinterpret_cast<u32x4*>(tile + rr * P + cc) = v[k];
        if (q) {
            float f[E];
            In<T>::unpack(v[k], f);
            const float a = max_lanes<LPB>(absmax<E>(f));
            const uint32_t code = mx_code(a);
            const float mult = mx_multiplier(code);
            if (col_in && r0 + rr < R) {
                Enc8<kE4M3, E>::store(q + (r0 + rr) * C + c0 + cc, f, mult);
                if ((lane & (LPB - 1)) == 0)
                    e[(r0 + rr) * nbc + (c0 + cc) / 32] = (uint8_t)code;
            }
        }
    }
    if (!qt)
        return;
    __syncthreads();
    const int c = threadIdx.x & 127, h = threadIdx.x >> 7;
    if (c0 + c >= C)
        return;
    const int64_t nbr = R / 32;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int rb = 64 * h + 32 * b;
        if (r0 + rb >= R)
            break;
        float f[32];
#pragma unroll
        for (int k = 0; k < 32; ++k)
            f[k] = In<T>::load1(tile, (int64_t)(rb + k) * P + c);
        const uint32_t code = mx_code(absmax<32>(f));
        const float mult = mx_multiplier(code);
        u32x4 w0, w1;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            w0[d] = enc4<kE4M3>(f[4 * d], f[4 * d + 1], f[4 * d + 2], f[4 * d + 3], mult);
            w1[d] = enc4<kE4M3>(f[16 + 4 * d], f[17 + 4 * d], f[18 + 4 * d], f[19 + 4 * d], mult);
        }
        uint8_t* out = qt + (c0 + c) * R + r0 + rb;
        st16_stream(out, w0);
        st16_stream(out + 16, w1);
        et[(c0 + c) * nbr + (r0 + rb) / 32] = (uint8_t)code;
    }
}

}  // namespace

hipError_t launch_mx(const void* x, int in_bf16, int64_t R, int64_t C, uint8_t* q, uint8_t* e, uint8_t* qt,
                     uint8_t* et, hipStream_t stream)
{
    const unsigned grid = (unsigned)(cdiv(C, 128) * cdiv(R, 128));
    if (in_bf16) {
        const size_t lds = qt ? 128 * tile_pitch<uint16_t>() * 2 : 0;
        k_mx<uint16_t><<<grid, kWG, lds, stream>>>((const uint16_t*)x, R, C, q, e, qt, et);
    } else {
        const size_t lds = qt ? 128 * tile_pitch<float>() * 4 : 0;
        k_mx<float><<<grid, kWG, lds, stream>>>((const float*)x, R, C, q, e, qt, et);
    }
    return hipGetLastError();
}

}  // namespace fq
