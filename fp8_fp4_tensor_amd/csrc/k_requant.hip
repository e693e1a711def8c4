// k_requant.hip -- the colwise copy of a quantized tensor from its rowwise
// copy alone, without the high-precision source ([MP] "混合精度训练：fp16 到
// fp8" (garden.houmin.site), section "FP8 通信": an FP8 expert-parallel
// dispatch sends only the rowwise FP8 data, and the backward pass needs the
// colwise copy, so the received data is de-quantized and re-quantized in the
// other direction; the scales must be powers of two for this double
// quantization to match a single one up to special values such as
// subnormals). With power-of-two scales the restored values dec(q) * scale
// are exact in fp32.
//
//   k_mx_requant      MXFP8: 1x32 rowwise blocks -> 32x1 colwise blocks.
//   k_block_requant   blockwise E4M3 with power-of-two tile scales: 1x128
//                     rowwise tiles -> 128x1 colwise tiles.
//
// Both walk 128x128 tiles of codes with a resident grid, the next tile's
// loads in flight while the current one is requantized, and write X^T as
// whole 128-byte lines through a transposed LDS tile; a tile's stores drain
// while the next tile is staged and requantized.
#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace fq {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Byte offset of 16-byte chunk ch (0..7) of row `row` in an LDS tile of
// transposed codes (128-byte rows): chunks XOR-swizzled by (row / 2) % 8, so
// the eight rows two apart that eight lanes write at once hit distinct banks.
__device__ __forceinline__ int tr_off(int row, int ch) { return row * 128 + ((ch ^ ((row >> 1) & 7)) << 4); }

// The colwise MXFP8 copy from the rowwise copy alone ([MP] "FP8 通信": the
// EP backward step de-quantizes the rowwise FP8 data and re-quantizes it in
// the other direction). Per 128x128 tile: the rowwise codes (16 KiB) and the
// tile rows' scales (as fp32) go to LDS; each thread takes a column pair and 32
// rows, restores the values exactly (dec(q) * 2^(code-127) is exact in fp32
// for power-of-two scales), quantizes each 32x1 column block with the MX
// rule, and the transposed codes leave through an LDS tile as whole lines.
// HBM traffic is one code byte in and one out per element, plus scales.
//
// FULL: R and C are multiples of 128, so every load and store is
// unconditional. The first tile is peeled off the loop, so that the loop is
// entered, like each of its iterations, with the next tile's loads followed
// by this tile's stores in flight; the compiler then waits for the loads
// alone before staging a tile, and with LDS-only barriers a tile's stores
// drain while the next one is requantized.
template <bool FULL>
__global__ __launch_bounds__(kWG) void k_mx_requant(const uint8_t* __restrict__ q, const uint8_t* __restrict__ e,
                                                    int64_t R, int64_t C, uint8_t* __restrict__ qt,
                                                    uint8_t* __restrict__ et)
{
    constexpr int QP = 128 + 16;  // pitch of the code tile (bytes)
    constexpr int SP = 128 + 4;   // pitch of the scale table (floats): its four rows start in distinct banks
    __shared__ __align__(16) uint8_t qtile[128 * QP];
    __shared__ __align__(16) float escale[4 * SP];  // [column block][tile row]: the row scales as fp32
    __shared__ __align__(16) uint8_t otile[128 * 128];
    __shared__ __align__(16) uint8_t ocode[128 * 4];
    const int64_t ntc = cdiv(C, 128), ntiles = ntc * cdiv(R, 128);
    const int64_t nbc = C / 32, nbr = R / 32;
    // a tile's codes and E8M0 codes are loaded into registers one tile
    // early, so they fly while the previous tile is requantized
    u32x4 v[4];
    uint32_t ew = 0;
    auto load_tile = [&](int64_t t) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * 128, c0 = tc * 128;
        if (FULL) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = k * kWG + threadIdx.x, row = i >> 3, seg = (i & 7) * 16;
                v[k] = ld16_stream(q + (r0 + row) * C + c0 + seg);
            }
            // four E8M0 codes of a tile row: 4-byte aligned (nbc % 4 == 0)
            if (threadIdx.x < 128)
                ew = *reinterpret_cast<const uint32_t*>(e + (r0 + threadIdx.x) * nbc + c0 / 32);
        } else {
            const int64_t nrows_in = min((int64_t)128, R - r0), ncols_in = min((int64_t)128, C - c0);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = k * kWG + threadIdx.x, row = i >> 3, seg = (i & 7) * 16;
                v[k] = (row < nrows_in && seg < ncols_in) ? ld16_stream(q + (r0 + row) * C + c0 + seg)
                                                          : u32x4{0u, 0u, 0u, 0u};
            }
            ew = 0;
            if (threadIdx.x < nrows_in)
                for (int j = 0; j < ncols_in / 32; ++j)
                    ew |= (uint32_t)e[(r0 + threadIdx.x) * nbc + c0 / 32 + j] << (8 * j);
        }
    };
    // Tile t, whose loads are in v and ew. LDS hazards between consecutive
    // tiles: the staging writes of tile t+1 follow the second barrier of
    // tile t (after every read of qtile and escale), and its otile / ocode
    // writes follow its own first barrier (after every read of tile t's).
    auto step = [&](int64_t t) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * 128, c0 = tc * 128;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = k * kWG + threadIdx.x, row = i >> 3, seg = (i & 7) * 16;
            *reinterpret_cast<u32x4*>(qtile + row * QP + seg) = v[k];
        }
        if (threadIdx.x < 128) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                escale[j * SP + threadIdx.x] = e8m0_value((ew >> (8 * j)) & 0xFFu);
        }
        lds_barrier();
        if (t + gridDim.x < ntiles)
            load_tile(t + gridDim.x);
        const int pc = threadIdx.x & 63, rb = threadIdx.x >> 6;
        const int cb = (2 * pc) >> 5;  // the 32-column block of both columns
        float f0[32], f1[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const int row = 32 * rb + k;
            const uint32_t two = *reinterpret_cast<const uint16_t*>(qtile + row * QP + 2 * pc);
            const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)two, false);
            const float sc = escale[cb * SP + row];
            f0[k] = d[0] * sc;
            f1[k] = d[1] * sc;
        }
        const uint32_t code0 = mx_code(absmax<32>(f0)), code1 = mx_code(absmax<32>(f1));
        const float m0 = mx_multiplier(code0), m1 = mx_multiplier(code1);
        u32x4 w[4];
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            w[d >> 2][d & 3] = enc4<kE4M3>(f0[4 * d], f0[4 * d + 1], f0[4 * d + 2], f0[4 * d + 3], m0);
            w[2 + (d >> 2)][d & 3] = enc4<kE4M3>(f1[4 * d], f1[4 * d + 1], f1[4 * d + 2], f1[4 * d + 3], m1);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            *reinterpret_cast<u32x4*>(otile + tr_off(2 * pc + j, 2 * rb)) = w[2 * j];
            *reinterpret_cast<u32x4*>(otile + tr_off(2 * pc + j, 2 * rb + 1)) = w[2 * j + 1];
        }
        ocode[(2 * pc) * 4 + rb] = (uint8_t)code0;
        ocode[(2 * pc + 1) * 4 + rb] = (uint8_t)code1;
        lds_barrier();
        if (FULL) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = k * kWG + threadIdx.x, row = i >> 3, seg = (i & 7) * 16;
                st16_stream(qt + (c0 + row) * R + r0 + seg,
                            *reinterpret_cast<const u32x4*>(otile + tr_off(row, seg >> 4)));
            }
            // four E8M0 codes of an X^T tile row: 4-byte aligned (nbr % 4 == 0)
            if (threadIdx.x < 128)
                *reinterpret_cast<uint32_t*>(et + (c0 + threadIdx.x) * nbr + r0 / 32) =
                    *reinterpret_cast<const uint32_t*>(ocode + threadIdx.x * 4);
        } else {
            const int64_t nrows_in = min((int64_t)128, R - r0), ncols_in = min((int64_t)128, C - c0);
            const int64_t nrows = ncols_in, nbytes = nrows_in;  // rows and bytes of the X^T tile
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = k * kWG + threadIdx.x, row = i >> 3, seg = (i & 7) * 16;
                if (row < nrows && seg < nbytes)
                    st16_stream(qt + (c0 + row) * R + r0 + seg,
                                *reinterpret_cast<const u32x4*>(otile + tr_off(row, seg >> 4)));
            }
            if (threadIdx.x < nrows) {
                const int row = threadIdx.x;
                uint8_t* dst = et + (c0 + row) * nbr + r0 / 32;
                for (int j = 0; j < nbytes / 32; ++j)
                    dst[j] = ocode[row * 4 + j];
            }
        }
    };
    int64_t t = blockIdx.x;
    if (t >= ntiles)
        return;
    load_tile(t);
    step(t);
    for (t += gridDim.x; t < ntiles; t += gridDim.x)
        step(t);
}

// Requantize blockwise 1x128 (power-of-two scales) in the other direction.
// A 128x128 tile of rowwise codes and its 128 row scales are staged in LDS
// (the next tile's loads already in flight into registers). Thread (p, rb)
// restores columns 2p, 2p+1 over rows 32rb..32rb+31 exactly in fp32 (an
// E4M3 value times a power of two); the four waves' column maxima meet in
// LDS to give each 128x1 block its E8M0-rule scale; the re-encoded codes go
// through a transposed LDS tile and out as whole 128-byte lines of X^T, and
// each X^T row's tile scale as one fp32. R and C are multiples of 128. The
// first tile is peeled and the barriers order LDS only, as in k_mx_requant.
__global__ __launch_bounds__(kWG) void k_block_requant(const uint8_t* __restrict__ q, const float* __restrict__ s,
                                                       int64_t R, int64_t C, uint8_t* __restrict__ qt,
                                                       float* __restrict__ st)
{
    constexpr int QP = 128 + 16;  // pitch of the staged code tile (bytes)
    __shared__ __align__(16) uint8_t qtile[128 * QP];
    __shared__ __align__(16) uint8_t otile[128 * 128];
    __shared__ float stile[128];
    __shared__ float pmax[4][128];
    const int64_t ntc = C / 128, ntiles = ntc * (R / 128), nsr = R / 128;
    u32x4 v[4];
    float sv = 0.0f;
    auto load_tile = [&](int64_t t) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * 128, c0 = tc * 128;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = k * kWG + threadIdx.x, row = i >> 3, seg = (i & 7) * 16;
            v[k] = ld16_stream(q + (r0 + row) * C + c0 + seg);
        }
        if (threadIdx.x < 128)
            sv = s[(r0 + threadIdx.x) * ntc + c0 / 128];
    };
    // LDS hazards between consecutive tiles: qtile / stile writes of tile
    // t+1 follow the third barrier of tile t, pmax writes follow its first
    // barrier, otile writes its second.
    auto step = [&](int64_t t) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * 128, c0 = tc * 128;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = k * kWG + threadIdx.x, row = i >> 3, seg = (i & 7) * 16;
            *reinterpret_cast<u32x4*>(qtile + row * QP + seg) = v[k];
        }
        if (threadIdx.x < 128)
            stile[threadIdx.x] = sv;
        lds_barrier();
        if (t + gridDim.x < ntiles)
            load_tile(t + gridDim.x);
        const int pc = threadIdx.x & 63, rb = threadIdx.x >> 6;
        float f0[32], f1[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const int row = 32 * rb + k;
            const uint32_t two = *reinterpret_cast<const uint16_t*>(qtile + row * QP + 2 * pc);
            const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)two, false);
            const float sc = stile[row];
            f0[k] = d[0] * sc;
            f1[k] = d[1] * sc;
        }
        pmax[rb][2 * pc] = absmax<32>(f0);
        pmax[rb][2 * pc + 1] = absmax<32>(f1);
        lds_barrier();
        const float a0 = fmaxf(fmaxf(pmax[0][2 * pc], pmax[1][2 * pc]), fmaxf(pmax[2][2 * pc], pmax[3][2 * pc]));
        const float a1 = fmaxf(fmaxf(pmax[0][2 * pc + 1], pmax[1][2 * pc + 1]),
                               fmaxf(pmax[2][2 * pc + 1], pmax[3][2 * pc + 1]));
        const uint32_t code0 = mx_code<kE4M3>(a0), code1 = mx_code<kE4M3>(a1);
        const float m0 = mx_multiplier(code0), m1 = mx_multiplier(code1);
        u32x4 w[4];
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            w[d >> 2][d & 3] = enc4<kE4M3>(f0[4 * d], f0[4 * d + 1], f0[4 * d + 2], f0[4 * d + 3], m0);
            w[2 + (d >> 2)][d & 3] = enc4<kE4M3>(f1[4 * d], f1[4 * d + 1], f1[4 * d + 2], f1[4 * d + 3], m1);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            *reinterpret_cast<u32x4*>(otile + tr_off(2 * pc + j, 2 * rb)) = w[2 * j];
            *reinterpret_cast<u32x4*>(otile + tr_off(2 * pc + j, 2 * rb + 1)) = w[2 * j + 1];
        }
        if (rb == 0) {
            st[(c0 + 2 * pc) * nsr + r0 / 128] = e8m0_value(code0);
            st[(c0 + 2 * pc + 1) * nsr + r0 / 128] = e8m0_value(code1);
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = k * kWG + threadIdx.x, row = i >> 3, seg = (i & 7) * 16;
            st16_stream(qt + (c0 + row) * R + r0 + seg, *reinterpret_cast<const u32x4*>(otile + tr_off(row, seg >> 4)));
        }
    };
    int64_t t = blockIdx.x;
    if (t >= ntiles)
        return;
    load_tile(t);
    step(t);
    for (t += gridDim.x; t < ntiles; t += gridDim.x)
        step(t);
}

}  // namespace

hipError_t launch_mx_requant(const uint8_t* q, const uint8_t* e, int64_t R, int64_t C, uint8_t* qt, uint8_t* et,
                             hipStream_t stream)
{
    const int64_t ntiles = cdiv(C, 128) * cdiv(R, 128);
    if (R % 128 == 0 && C % 128 == 0) {
        static ResidentGrid cache;
        const int64_t grid = std::min<int64_t>(ntiles, cache.get(k_mx_requant<true>, kWG, 0));
        k_mx_requant<true><<<(unsigned)grid, kWG, 0, stream>>>(q, e, R, C, qt, et);
    } else {
        static ResidentGrid cache;
        const int64_t grid = std::min<int64_t>(ntiles, cache.get(k_mx_requant<false>, kWG, 0));
        k_mx_requant<false><<<(unsigned)grid, kWG, 0, stream>>>(q, e, R, C, qt, et);
    }
    return hipGetLastError();
}

hipError_t launch_block_requant(const uint8_t* q, const float* s, int64_t R, int64_t C, uint8_t* qt, float* st,
                                hipStream_t stream)
{
    const int64_t ntiles = (C / 128) * (R / 128);
    static ResidentGrid cache;
    const int64_t grid = std::min<int64_t>(ntiles, cache.get(k_block_requant, kWG, 0));
    k_block_requant<<<(unsigned)grid, kWG, 0, stream>>>(q, s, R, C, qt, st);
    return hipGetLastError();
}

}  // namespace fq
