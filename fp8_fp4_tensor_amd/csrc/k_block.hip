// k_block.hip -- blockwise E4M3 quantization with an fp32 scale per tile:
// 1x128 tiles for activations and gradients, 128x128 tiles for weights.
//
// Source: [MP] "混合精度训练：fp16 到 fp8" (garden.houmin.site), section
// "FP8 recipe" item 4 and section "Blockwise scaling" (the DeepSeek-V3-like
// recipe: pure E4M3, 1x128 and 128x128 tiles, fp32 scaling factors, and the
// three GEMMs that read X^T with 1x128 tiles and W^T with 128x128 tiles).
// Each tile is quantized like a tensor under current scaling:
// a_B = max|x|, alpha_B = 448/a_B, q = Q(fp32(alpha_B x)), s_B = a_B/448.
// With power-of-two scales (the section's MXFP8 emulation, a tile as MX
// blocks sharing one E8M0 scale): s_B = 2^(floor(log2 a_B) - 8), alpha_B =
// 1/s_B, both exact powers of two, so alpha_B x is exact.
//
//   k_block_1x128      rows are contiguous, so 1x128 tiles are consecutive
//                      128-element runs of the flat tensor: one tile is 16
//                      lanes x 16 bytes of bf16 (32 lanes for fp32), and the
//                      tile max is a 4-step DPP reduction inside a row of
//                      lanes. A lane keeps four loads (four tiles of its
//                      lane group) in flight; lane i of each quad does the
//                      scale division for load i and the quad shares the
//                      results by DPP, a quarter of the division work. One
//                      read, no LDS.
//   k_block_1x128_rowcol  the colwise copy (1x128 tiles of X^T, i.e. 128-row
//                      runs down each column) and, when asked, the rowwise
//                      one from the same read: a 128x128 tile per workgroup,
//                      rowwise from registers as k_block_1x128, colwise from
//                      the tile staged in LDS (swizzled), four lanes sharing a
//                      column (DPP max) and writing its 128 codes, one line
//                      of X^T.
//   k_block_128x128    one workgroup per tile, kept in registers between the
//                      tile max and the cast; the colwise copy is the byte
//                      transpose of the same codes, through LDS.
#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace fq {
namespace {

constexpr int kLoads = 4;
constexpr int kMaxGrid = 16384;
constexpr int kBlock128Tiles = 2;  // 128x128 tiles per workgroup, side by side

// LDS column offset of the codes of row r: 8-byte units XOR-swizzled by the
// row's 16-row group, so reads of one column over rows 16 apart hit distinct banks.
__device__ __forceinline__ int code_swizzle(int r) { return 8 * ((r >> 4) & 7); }

// Tile multiplier and stored scale from the tile amax.
template <bool POW2>
__device__ __forceinline__ void tile_scales(float a, float& alpha, float& s)
{
    if constexpr (POW2) {
        const uint32_t code = mx_code<kE4M3>(a);
        alpha = mx_multiplier(code);
        s = e8m0_value(code);
    } else {
        tensor_scales(a, 448.0f, alpha, s);
    }
}

template <typename T, bool POW2>
__global__ __launch_bounds__(kWG) void k_block_1x128(const T* __restrict__ x, int64_t n, uint8_t* __restrict__ q,
                                                     float* __restrict__ s_out)
{
    constexpr int E = In<T>::kE, U = 64 * E, LPB = 128 / E;
    const int lane = threadIdx.x & 63;
    const int64_t nunits = cdiv(n, U);
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    static_assert(kLoads == 4 && LPB >= 4, "a quad of lanes shares the scale arithmetic of the four loads");
    const int jsel = lane & 3;
    for (int64_t u0 = wave * kLoads; u0 < nunits; u0 += nwaves * kLoads) {
        u32x4 v[kLoads];
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t e = (u0 + j) * U + lane * E;
            v[j] = (u0 + j < nunits && e < n) ? ld16_stream(x + e) : u32x4{0u, 0u, 0u, 0u};
        }
        // the tile maxima of the four loads; lane i of each quad then takes
        // the scale arithmetic of load i, and the quad shares the results
        float a[kLoads];
#pragma unroll
        for (int j = 0; j < kLoads; ++j)
            a[j] = max_lanes<LPB>(In<T>::absmax16(v[j]));
        const float asel = jsel == 0 ? a[0] : jsel == 1 ? a[1] : jsel == 2 ? a[2] : a[3];
        float alpha_sel, s_sel;
        tile_scales<POW2>(asel, alpha_sel, s_sel);
        float alpha[kLoads];
        alpha[0] = dpp<0x00>(alpha_sel);
        alpha[1] = dpp<0x55>(alpha_sel);
        alpha[2] = dpp<0xAA>(alpha_sel);
        alpha[3] = dpp<0xFF>(alpha_sel);
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            if (u0 + j >= nunits)
                break;
            const int64_t e = (u0 + j) * U + lane * E;
            float f[E];
            In<T>::unpack(v[j], f);
            if (e < n) {
                Enc8<kE4M3, E>::store(q + e, f, alpha[j]);
                if ((lane & (LPB - 1)) == j)
                    s_out[e / 128] = s_sel;
            }
        }
    }
}

// The colwise copy of 1x128 tiles and, with ROW, the rowwise copy from the
// same read: a 128x128 tile of X per workgroup. The LPR lanes that load a
// tile row hold one 1x128 tile of X: the rowwise codes and scale come
// straight from registers, as in k_block_1x128 (a row's max by DPP; lane j
// of a row does the scale arithmetic of round j and the others read it with
// a lane permute). The tile is staged in LDS with its 16-byte chunks
// XOR-swizzled by 32-row group, and after one barrier (LDS only, so the
// rowwise stores drain meanwhile) quads of lanes take the colwise tiles (128
// rows of one column: a 1x128 tile of X^T), 64 columns per pass: lane q of a
// quad reads rows 32q .. 32q + 31 of its column (distinct banks), the quad's
// max is two DPP steps, and each lane writes 32 contiguous bytes of the
// 128-byte line of X^T (ordinary stores: the four pieces meet in L2).
// R % 128 == 0, C % 128 == 0; LDS: 128 rows x 128 elements.
template <typename T, bool POW2, bool ROW = true>
__global__ __launch_bounds__(kWG) void k_block_1x128_rowcol(const T* __restrict__ x, int64_t R, int64_t C,
                                                            uint8_t* __restrict__ q, float* __restrict__ s_out,
                                                            uint8_t* __restrict__ qt, float* __restrict__ st)
{
    constexpr int TC = 128, E = In<T>::kE, CPR = TC / E, SW = 16 / E;  // chunks per row; swizzle step
    constexpr int LPR = CPR, RPR = kWG / LPR, ROUNDS = 128 / RPR;      // lanes per row, rows per round
    static_assert(ROUNDS <= LPR, "each round's scale is computed by a lane of the row");
    extern __shared__ __align__(16) unsigned char smem[];
    T (*tile)[TC] = reinterpret_cast<T (*)[TC]>(smem);
    const int64_t ntc = C / TC;
    const int64_t r0 = (int64_t)(blockIdx.x / ntc) * 128, c0 = (int64_t)(blockIdx.x % ntc) * TC;
    const int lane = threadIdx.x & 63;
    const int j = threadIdx.x % LPR, rr0 = threadIdx.x / LPR;  // this lane's chunk of its rows; first row
    u32x4 v[ROUNDS];
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k)
        v[k] = ld16_stream(x + (r0 + rr0 + k * RPR) * C + c0 + j * E);
    // stage for the colwise pass: chunk j of row r at chunk j ^ (SW * ((r >> 5) & 3))
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
        const int r = rr0 + k * RPR;
        *reinterpret_cast<u32x4*>(&tile[r][(j ^ (SW * ((r >> 5) & 3))) * E]) = v[k];
    }
    // rowwise: round k's row max in every lane of the row; lane j computes
    // the scales of round j % ROUNDS and lends them to the row's other lanes
    if constexpr (ROW) {
    float a[ROUNDS];
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k)
        a[k] = max_lanes<LPR>(In<T>::absmax16(v[k]));
    float asel = a[0];
#pragma unroll
    for (int k = 1; k < ROUNDS; ++k)
        asel = (j % ROUNDS) == k ? a[k] : asel;
    float alpha_sel, s_sel;
    tile_scales<POW2>(asel, alpha_sel, s_sel);
    const int base = lane & ~(LPR - 1);
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
        const float alpha = __shfl(alpha_sel, base + k);
        const int64_t row = r0 + rr0 + k * RPR;
        float f[E];
        In<T>::unpack(v[k], f);
        Enc8<kE4M3, E>::store(q + row * C + c0 + j * E, f, alpha);
        if (j == k)
            s_out[row * ntc + c0 / 128] = s_sel;
    }
    }
    lds_barrier();
    // colwise: thread t takes column c = (t >> 2) + 64h and rows 32cq .. 32cq + 31
    const int cq = threadIdx.x & 3;
#pragma unroll
    for (int h = 0; h < TC / 64; ++h) {
        const int c = (threadIdx.x >> 2) + 64 * h;
        const int col = ((c / E) ^ (SW * cq)) * E + (c % E);  // column c's place in rows 32cq .. 32cq + 31
        float f[32];
#pragma unroll
        for (int k = 0; k < 32; ++k)
            f[k] = In<T>::load1(&tile[32 * cq + k][0], col);
        const float am = max_lanes4(absmax<32>(f));
        float alpha, s;
        tile_scales<POW2>(am, alpha, s);
        u32x4 w0, w1;
        w0[0] = enc4<kE4M3>(f[0], f[1], f[2], f[3], alpha);
        w0[1] = enc4<kE4M3>(f[4], f[5], f[6], f[7], alpha);
        w0[2] = enc4<kE4M3>(f[8], f[9], f[10], f[11], alpha);
        w0[3] = enc4<kE4M3>(f[12], f[13], f[14], f[15], alpha);
        w1[0] = enc4<kE4M3>(f[16], f[17], f[18], f[19], alpha);
        w1[1] = enc4<kE4M3>(f[20], f[21], f[22], f[23], alpha);
        w1[2] = enc4<kE4M3>(f[24], f[25], f[26], f[27], alpha);
        w1[3] = enc4<kE4M3>(f[28], f[29], f[30], f[31], alpha);
        uint8_t* out = qt + (c0 + c) * R + r0 + 32 * cq;
        *reinterpret_cast<u32x4*>(out) = w0;
        *reinterpret_cast<u32x4*>(out + 16) = w1;
        if (cq == 0)
            st[(c0 + c) * (R / 128) + r0 / 128] = s;
    }
}

// 128x128 tiles; a workgroup takes NT horizontally adjacent tiles (the rows
// it reads and writes are then NT * 256 and NT * 128 contiguous bytes), kept
// in registers between the tile maxima and the cast. q/s rowwise (may be
// null), qt/st colwise (may be null): the colwise copy is the byte transpose
// of the same codes, through LDS.
template <typename T, bool POW2, int NT>
__global__ __launch_bounds__(kWG) void k_block_128x128(const T* __restrict__ x, int64_t R, int64_t C,
                                                       uint8_t* __restrict__ q, float* __restrict__ s_out,
                                                       uint8_t* __restrict__ qt, float* __restrict__ st)
{
    constexpr int E = In<T>::kE, W = 128 * NT, LPR = W / E, RPR = kWG / LPR, ROUNDS = 128 / RPR;
    constexpr int LPT = 128 / E, NG = kWG / LPT;  // lanes per tile row; lane groups per workgroup
    __shared__ float red[NG];
    __shared__ __align__(16) uint8_t codes[128][W + 16];
    const int64_t ntc = C / 128, ntr = R / 128, nwc = cdiv(ntc, NT);
    const int64_t tr = blockIdx.x / nwc, tw = blockIdx.x % nwc;
    const int64_t r0 = tr * 128, c0 = tw * W;
    const int cc = (threadIdx.x % LPR) * E, rr0 = threadIdx.x / LPR;
    const int j = cc / 128;                  // this thread's tile in the workgroup
    const bool tin = tw * NT + j < ntc;      // that tile exists (the last workgroup of a row may hold fewer)
    u32x4 v[ROUNDS];
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k)
        v[k] = tin ? ld16_stream(x + (r0 + rr0 + k * RPR) * C + c0 + cc) : u32x4{0u, 0u, 0u, 0u};
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
        float f[E];
        In<T>::unpack(v[k], f);
        m = fmaxf(m, absmax<E>(f));
    }
    // tile maxima: lanes of one tile row segment (LPT lanes), then the NG / NT
    // groups of the same tile (group g holds tile g % NT)
    m = max_lanes<LPT>(m);
    if (threadIdx.x % LPT == 0)
        red[threadIdx.x / LPT] = m;
    __syncthreads();
    float a = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; g += NT)
        a = fmaxf(a, red[g + j]);
    float alpha, s;
    tile_scales<POW2>(a, alpha, s);
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
        float f[E];
        In<T>::unpack(v[k], f);
        const int rr = rr0 + k * RPR;
        if constexpr (E == 8) {
            u32x2 w;
            w[0] = enc4<kE4M3>(f[0], f[1], f[2], f[3], alpha);
            w[1] = enc4<kE4M3>(f[4], f[5], f[6], f[7], alpha);
            if (q && tin)
                st8_stream(q + (r0 + rr) * C + c0 + cc, w);
            if (qt)
                *reinterpret_cast<u32x2*>(&codes[rr][cc ^ code_swizzle(rr)]) = w;
        } else {
            const uint32_t w = enc4<kE4M3>(f[0], f[1], f[2], f[3], alpha);
            if (q && tin)
                st4_stream(q + (r0 + rr) * C + c0 + cc, w);
            if (qt)
                *reinterpret_cast<uint32_t*>(&codes[rr][cc ^ code_swizzle(rr)]) = w;
        }
    }
    if (tin && rr0 == 0 && cc % 128 == 0) {
        const int64_t tc = tw * NT + j;
        if (s_out)
            s_out[tr * ntc + tc] = s;
        if (st)
            st[tc * ntr + tr] = s;
    }
    if (qt) {
        __syncthreads();
        // colwise: X^T rows c0 .. c0 + W - 1, 128 bytes each (rows r0 .. r0 + 127
        // of the codes). Eight lanes per X^T row, lane k taking codes rows
        // 16k .. 16k + 15, so each store instruction writes eight whole lines;
        // the swizzle puts the eight lanes' byte reads in distinct banks.
        const int k = threadIdx.x & 7;
        for (int c = threadIdx.x >> 3; c < W; c += kWG / 8) {
            u32x4 w;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t word = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int r = 16 * k + 4 * d + b;
                    word |= (uint32_t)codes[r][c ^ code_swizzle(r)] << (8 * b);
                }
                w[d] = word;
            }
            if (c0 + c < C)
                st16_stream(qt + (c0 + c) * R + r0 + 16 * k, w);
        }
    }
}

}  // namespace

hipError_t launch_block_1x128(const void* x, int in_bf16, int pow2, int64_t R, int64_t C, uint8_t* q, float* s,
                              hipStream_t stream)
{
    const int64_t n = R * C;
    const int E = in_bf16 ? 8 : 4;
    const int64_t per_wg = (int64_t)kWG * E * kLoads;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, per_wg), kMaxGrid));
    const uint16_t* xb = (const uint16_t*)x;
    const float* xf = (const float*)x;
    if (in_bf16 && pow2)
        k_block_1x128<uint16_t, true><<<grid, kWG, 0, stream>>>(xb, n, q, s);
    else if (in_bf16)
        k_block_1x128<uint16_t, false><<<grid, kWG, 0, stream>>>(xb, n, q, s);
    else if (pow2)
        k_block_1x128<float, true><<<grid, kWG, 0, stream>>>(xf, n, q, s);
    else
        k_block_1x128<float, false><<<grid, kWG, 0, stream>>>(xf, n, q, s);
    return hipGetLastError();
}

template <typename T, bool POW2>
static void block_1x128_rowcol_t(const T* x, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qt, float* st,
                                 hipStream_t stream)
{
    const unsigned grid = (unsigned)((R / 128) * (C / 128));
    const size_t lds = 128 * 128 * sizeof(T);
    if (q)
        k_block_1x128_rowcol<T, POW2, true><<<grid, kWG, lds, stream>>>(x, R, C, q, s, qt, st);
    else
        k_block_1x128_rowcol<T, POW2, false><<<grid, kWG, lds, stream>>>(x, R, C, q, s, qt, st);
}

hipError_t launch_block_1x128_rowcol(const void* x, int in_bf16, int pow2, int64_t R, int64_t C, uint8_t* q,
                                     float* s, uint8_t* qt, float* st, hipStream_t stream)
{
    const uint16_t* xb = (const uint16_t*)x;
    const float* xf = (const float*)x;
    if (in_bf16 && pow2)
        block_1x128_rowcol_t<uint16_t, true>(xb, R, C, q, s, qt, st, stream);
    else if (in_bf16)
        block_1x128_rowcol_t<uint16_t, false>(xb, R, C, q, s, qt, st, stream);
    else if (pow2)
        block_1x128_rowcol_t<float, true>(xf, R, C, q, s, qt, st, stream);
    else
        block_1x128_rowcol_t<float, false>(xf, R, C, q, s, qt, st, stream);
    return hipGetLastError();
}

template <typename T, bool POW2>
void block_128x128_t(const T* x, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qt, float* st,
                     hipStream_t stream)
{
    constexpr int NT = kBlock128Tiles;
    const unsigned grid = (unsigned)(cdiv(C / 128, NT) * (R / 128));
    k_block_128x128<T, POW2, NT><<<grid, kWG, 0, stream>>>(x, R, C, q, s, qt, st);
}

hipError_t launch_block_128x128(const void* x, int in_bf16, int pow2, int64_t R, int64_t C, uint8_t* q, float* s,
                                uint8_t* qt, float* st, hipStream_t stream)
{
    const uint16_t* xb = (const uint16_t*)x;
    const float* xf = (const float*)x;
    if (in_bf16 && pow2)
        block_128x128_t<uint16_t, true>(xb, R, C, q, s, qt, st, stream);
    else if (in_bf16)
        block_128x128_t<uint16_t, false>(xb, R, C, q, s, qt, st, stream);
    else if (pow2)
        block_128x128_t<float, true>(xf, R, C, q, s, qt, st, stream);
    else
        block_128x128_t<float, false>(xf, R, C, q, s, qt, st, stream);
    return hipGetLastError();
}

}  // namespace fq
