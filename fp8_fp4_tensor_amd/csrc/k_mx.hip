// k_mx.hip -- MX: E4M3 (MXFP8) or E5M2 elements in 32-element blocks that
// share one E8M0 (power-of-two) scale, rowwise (1x32 along a row) and colwise
// (32x1 down a column, stored transposed), both from a single read of the
// input. MXFP4 (E2M1 elements) from bf16 takes the same region walk
// (k_mxfp4_bf16, below); fp32 MXFP4 input takes k_mxfp4.hip.
//
// Source: [MP] "混合精度训练：fp16 到 fp8" (garden.houmin.site), section
// "MXFP8" (32-element blocks, one E8M0 scale each, value = element x scale;
// E8M0 is the exponent field of an fp32), "FP8 recipe" item 5 (E4M3, 1x32
// for inputs, gradients and weights) and "MXFP8 recipe" (rowwise and colwise
// copies of each tensor, 1x32 and 32x1).
// Block scale: 2^e with e = floor(log2 amax) - emax (8 = floor(log2 448) for
// E4M3, 15 = floor(log2 57344) for E5M2), held to the E8M0 range;
// q = Q(x * 2^-e), exact multiply, saturating.
//
// One workgroup per 128x128 tile (bf16 input: two tiles side by side per
// 512-thread workgroup, kMxTiles). Rowwise: each lane holds 16 bytes of a
// row, a quad of lanes is one 1x32 block (bf16), reduced with two DPP steps;
// codes and E8M0 scales are written straight from registers. Colwise: the
// tile's raw inputs go to LDS in the same pass; then each thread owns one
// column pair and 32 rows (two 32x1 blocks), reads them back (lanes of a
// wave read consecutive columns of one row: no bank conflicts) and puts its codes
// into a second LDS tile laid out as X^T; that tile is written out with
// eight lanes per 128-byte row of X^T, so every store instruction writes
// whole lines instead of one 16-byte piece of 64 different lines.
#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace fq {
namespace {

constexpr int kOP = 128;  // pitch of the LDS tile of transposed codes
static_assert(128 * kOP + 128 * 4 <= 128 * 128 * 2, "the code tile must fit in the input tile it reuses");
// bf16 MX tile walk: 128x128 tiles per workgroup, side by side (a 128-row x
// 256-column region, 512 threads): rows are read as 512-byte segments and
// the rowwise E8M0 codes of a row leave as 8 contiguous bytes
constexpr int kMxTiles = 2;
// the region walk's grid: one region per workgroup up to this many regions,
// beyond it each workgroup strides over several (a tall, narrow tensor would
// otherwise pass 2^32 work-items)
constexpr int64_t kMaxRegionGrid = 16384;
static_assert(kMxTiles * 128 * kOP + kMxTiles * 128 * 4 <= 128 * (128 * kMxTiles + 8) * 2,
              "the transposed code tile must fit in the input region it reuses");

// Byte offset of 16-byte chunk ch (0..7) of row `row` in the tile of
// transposed codes: 128-byte rows, chunks XOR-swizzled by (row / 2) % 8, so
// the eight rows two apart that eight lanes write at once hit distinct banks
// (a row's eight chunks, read by eight lanes, stay distinct too).
__device__ __forceinline__ int otile_off(int row, int ch) { return row * kOP + ((ch ^ ((row >> 1) & 7)) << 4); }

template <typename T>
constexpr int tile_pitch()
{
    return sizeof(T) == 2 ? 128 + 8 : 128;  // bf16 rows padded by 16 bytes; fp32 unpadded (64 KiB)
}

// Loads of one tile row band for this thread: ROUNDS x 16 bytes.
template <typename T, int ROUNDS>
__device__ __forceinline__ void mx_load_tile(const T* __restrict__ x, int64_t R, int64_t C, int64_t r0, int64_t c0,
                                             int cc, int rr0, int rpr, u32x4* v)
{
    const bool col_in = c0 + cc < C;
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
        const int64_t r = r0 + rr0 + k * rpr;
        v[k] = (col_in && r < R) ? ld16_stream(x + r * C + c0 + cc) : u32x4{0u, 0u, 0u, 0u};
    }
}

// Persistent: workgroup g takes tiles g, g + G, ..., with G the number of
// workgroups the device holds at once, so no tail of late workgroups forms;
// the resident workgroups of a CU overlap each other's loads and compute.
template <typename T, int FMT>
__global__ __launch_bounds__(kWG) void k_mx(const T* __restrict__ x, int64_t R, int64_t C,
                                            uint8_t* __restrict__ q, uint8_t* __restrict__ e,
                                            uint8_t* __restrict__ qt, uint8_t* __restrict__ et)
{
    constexpr int E = In<T>::kE, LPR = 128 / E, RPR = kWG / LPR, ROUNDS = 128 / RPR, LPB = 32 / E;
    constexpr int P = tile_pitch<T>();
    extern __shared__ __align__(16) unsigned char smem[];
    T* tile = reinterpret_cast<T*>(smem);
    const int lane = threadIdx.x & 63;
    const int64_t ntc = cdiv(C, 128), ntiles = ntc * cdiv(R, 128);
    const int cc = (threadIdx.x % LPR) * E, rr0 = threadIdx.x / LPR;
    const int64_t nbc = C / 32, nbr = R / 32;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * 128, c0 = tc * 128;
        u32x4 v[ROUNDS];
        mx_load_tile<T, ROUNDS>(x, R, C, r0, c0, cc, rr0, RPR, v);
        const bool col_in = c0 + cc < C;
        // whole 4-code words: the tile spans 128 columns and rows of codes are 4-byte aligned
        const bool full_row_codes = c0 + 128 <= C && (nbc & 3) == 0;
        if (qt)
            __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
        for (int k = 0; k < ROUNDS; ++k) {
            const int rr = rr0 + k * RPR;
            if (qt)
                *reinterpret_cast<u32x4*>(tile + rr * P + cc) = v[k];
            if (q) {
                float f[E];
                In<T>::unpack(v[k], f);
                const float a = max_lanes<LPB>(absmax<E>(f));
                const uint32_t code = mx_code<FMT>(a);
                const float mult = mx_multiplier(code);
                // the row's four block codes, gathered into its first lane
                const int rbase = lane & ~(LPR - 1);
                const uint32_t word = (uint32_t)__shfl((int)code, rbase) |
                                      ((uint32_t)__shfl((int)code, rbase + LPB) << 8) |
                                      ((uint32_t)__shfl((int)code, rbase + 2 * LPB) << 16) |
                                      ((uint32_t)__shfl((int)code, rbase + 3 * LPB) << 24);
                if (col_in && r0 + rr < R) {
                    Enc8<FMT, E>::store(q + (r0 + rr) * C + c0 + cc, f, mult);
                    if (full_row_codes) {
                        if (lane == rbase)
                            *reinterpret_cast<uint32_t*>(e + (r0 + rr) * nbc + c0 / 32) = word;
                    } else if ((lane & (LPB - 1)) == 0) {
                        e[(r0 + rr) * nbc + (c0 + cc) / 32] = (uint8_t)code;
                    }
                }
            }
        }
        if (!qt)
            continue;
        __syncthreads();
        // colwise: thread (p, rb) quantizes rows 32rb..32rb+31 of tile columns
        // 2p and 2p+1 (two 32x1 blocks); a wave reads one LDS row of 128
        // columns per instruction. After a barrier the codes go to an LDS
        // tile laid out as X^T, which reuses the input tile's memory.
        const int pc = threadIdx.x & 63, rb = threadIdx.x >> 6;
        u32x4 w[4];
        uint32_t codes2[2];
        if constexpr (sizeof(T) == 2) {
            // keep the 32 packed bf16 pairs (32 registers) and widen on use
            uint32_t pr[32];
#pragma unroll
            for (int k = 0; k < 32; ++k)
                pr[k] = *reinterpret_cast<const uint32_t*>(tile + (int64_t)(32 * rb + k) * P + 2 * pc);
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                a0 = fmaxf(a0, fabsf(bf16_lo(pr[k])));
                a1 = fmaxf(a1, fabsf(bf16_hi(pr[k])));
            }
            codes2[0] = mx_code<FMT>(a0);
            codes2[1] = mx_code<FMT>(a1);
            const float m0 = mx_multiplier(codes2[0]), m1 = mx_multiplier(codes2[1]);
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                w[d >> 2][d & 3] = enc4<FMT>(bf16_lo(pr[4 * d]), bf16_lo(pr[4 * d + 1]), bf16_lo(pr[4 * d + 2]),
                                               bf16_lo(pr[4 * d + 3]), m0);
                w[2 + (d >> 2)][d & 3] = enc4<FMT>(bf16_hi(pr[4 * d]), bf16_hi(pr[4 * d + 1]),
                                                     bf16_hi(pr[4 * d + 2]), bf16_hi(pr[4 * d + 3]), m1);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float f[32];
#pragma unroll
                for (int k = 0; k < 32; ++k)
                    f[k] = In<T>::load1(tile, (int64_t)(32 * rb + k) * P + 2 * pc + j);
                codes2[j] = mx_code<FMT>(absmax<32>(f));
                const float m = mx_multiplier(codes2[j]);
#pragma unroll
                for (int d = 0; d < 8; ++d)
                    w[2 * j + (d >> 2)][d & 3] = enc4<FMT>(f[4 * d], f[4 * d + 1], f[4 * d + 2], f[4 * d + 3], m);
            }
        }
        __syncthreads();
        uint8_t* otile = smem;              // [128][kOP] codes of X^T
        uint8_t* ocode = smem + 128 * kOP;  // [128][4] E8M0 codes of X^T
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            *reinterpret_cast<u32x4*>(otile + otile_off(2 * pc + j, 2 * rb)) = w[2 * j];
            *reinterpret_cast<u32x4*>(otile + otile_off(2 * pc + j, 2 * rb + 1)) = w[2 * j + 1];
            ocode[(2 * pc + j) * 4 + rb] = (uint8_t)codes2[j];
        }
        __syncthreads();
        // write X^T rows c0..c0+127, bytes r0..r0+127 of each: eight lanes per
        // 128-byte row, so each store instruction writes eight whole lines.
        const int64_t nrows = min((int64_t)128, C - c0), nbytes = min((int64_t)128, R - r0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = k * kWG + threadIdx.x;
            const int row = i >> 3, seg = (i & 7) * 16;
            if (row < nrows && seg < nbytes)
                st16_stream(qt + (c0 + row) * R + r0 + seg,
                            *reinterpret_cast<const u32x4*>(otile + otile_off(row, seg >> 4)));
        }
        if (threadIdx.x < nrows) {
            const int row = threadIdx.x;
            uint8_t* dst = et + (c0 + row) * nbr + r0 / 32;
            if (nbytes == 128 && (nbr & 3) == 0) {
                *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(ocode + row * 4);
            } else {
                for (int j = 0; j < nbytes / 32; ++j)
                    dst[j] = ocode[row * 4 + j];
            }
        }
    }
}

// ---------------------------------------------------------------- bf16 fast path
// The same MX computation for bf16 inputs, on packed bf16 pairs, with the
// gfx950 converters that take bf16 and a power-of-two scale directly
// (v_cvt_scalef32_pk_fp8_bf16 / _bf8_bf16: two elements, each divided by the
// scale and rounded to nearest even; E5M2 elements go through the same
// steps with its own emax and limit). It equals Q_E4M3(x * 2^-e) for every finite bf16
// x and every E8M0 code, as long as |x * 2^-e| <= 448; beyond that it gives
// NaN instead of saturating. A block's scaled values stay below 512, so the
// magnitudes are first clamped, as bf16 bit patterns, to the pattern of
// 448 * 2^e (a normal bf16 for every code): that clamp is exact, and the
// clamped elements then convert to exactly 448. The block amax is an integer
// max of the magnitude bits (exact for finite bf16). Per element this costs
// about a third of the VALU work of widening, multiplying and clamping in
// fp32.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
// bf16 pattern of Fmax * 2^(code - 127): exponent field code + emax, the
// mantissa of Fmax (448 * 2^e: code + 8, 1.75; 57344 * 2^e: code + 15, 1.75)
template <int FMT>
__device__ __forceinline__ uint32_t mx_limit_bf16(uint32_t code)
{
    return ((code + (uint32_t)Fmt<FMT>::kEmax) << 7) | Fmt<FMT>::kMantBf16;
}
// E8M0 code from the bf16 magnitude bits of a block amax
template <int FMT>
__device__ __forceinline__ uint32_t mx_code_bf16(uint32_t mag)
{
    return (uint32_t)max((int)((mag >> 7) & 0xFFu) - Fmt<FMT>::kEmax, 0);
}
// clamp both magnitudes of a pair to lim2 (limit in each half, below
// 0x8000), keep the signs
__device__ __forceinline__ uint32_t clamp_pair(uint32_t w, uint32_t lim2)
{
    return pk_min16(w & 0x7fff7fffu, lim2) | (w & 0x80008000u);
}
// two clamped bf16 pairs -> four E4M3 (or E5M2) codes (pair a in bytes 0-1, b in 2-3)
template <int FMT>
__device__ __forceinline__ uint32_t cvt4_scaled(uint32_t a, uint32_t b, float scale)
{
    s16x2 r = {0, 0};
    if constexpr (FMT == kE4M3) {
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, a), scale, false);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, b), scale, true);
    } else {
        r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(bf16x2, a), scale, false);
        r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(bf16x2, b), scale, true);
    }
    return __builtin_bit_cast(uint32_t, r);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int FMT>
__global__ __launch_bounds__(kMxTiles * kWG) void k_mx_bf16(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                 uint8_t* __restrict__ q, uint8_t* __restrict__ e,
                                                 uint8_t* __restrict__ qt, uint8_t* __restrict__ et)
{
    // kMxTiles 128x128 tiles side by side: TW columns, 16 lanes x 8 bf16 per
    // tile row; LDS pitch P in bf16
    constexpr int W = kMxTiles, NT = W * kWG, TW = 128 * W, ROUNDS = 8, P = TW + 8;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
    const int lane = threadIdx.x & 63;
    const int64_t ntc = cdiv(C, TW), ntiles = ntc * cdiv(R, 128);
    const int cc = (threadIdx.x & (16 * W - 1)) * 8, rr0 = threadIdx.x / (16 * W);
    const int64_t nbc = C / 32, nbr = R / 32;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * 128, c0 = tc * TW;
        const bool col_in = c0 + cc < C;
        u32x4 v[ROUNDS];
        {
            const uint16_t* src = x + (r0 + rr0) * C + c0 + cc;
            const int64_t step = 16 * C;
#pragma unroll
            for (int k = 0; k < ROUNDS; ++k) {
                v[k] = (col_in && r0 + rr0 + 16 * k < R) ? ld16_stream(src) : u32x4{0u, 0u, 0u, 0u};
                src += step;
            }
        }
        // whole u32 E8M0 words for this lane's 128-column tile
        const bool full_row_codes = c0 + (cc & ~127) + 128 <= C && (nbc & 3) == 0;
        if (qt)
            lds_barrier();  // the previous region's LDS reads are done (LDS-only barriers
                            // throughout: the rowwise stores drain during the colwise half)
        {
            uint8_t* dst = q ? q + (r0 + rr0) * C + c0 + cc : nullptr;
            uint8_t* edst = q ? e + (r0 + rr0) * nbc + c0 / 32 : nullptr;
#pragma unroll
            for (int k = 0; k < ROUNDS; ++k) {
                const int rr = rr0 + 16 * k;
                if (qt)
                    *reinterpret_cast<u32x4*>(tile + rr * P + cc) = v[k];
                if (q) {
                    uint32_t m = pk_max16(pk_max16(v[k][0] & 0x7fff7fffu, v[k][1] & 0x7fff7fffu),
                                          pk_max16(v[k][2] & 0x7fff7fffu, v[k][3] & 0x7fff7fffu));
                    m = max(m & 0xFFFFu, m >> 16);
                    m = max(m, dppu<kDppXor1>(m));
                    m = max(m, dppu<kDppXor2>(m));  // the 1x32 block: a quad of lanes
                    const uint32_t code = mx_code_bf16<FMT>(m);
                    const uint32_t lim = mx_limit_bf16<FMT>(code), lim2 = lim | (lim << 16);
                    const float scale = e8m0_value(code);
                    u32x2 w;
                    w[0] = cvt4_scaled<FMT>(clamp_pair(v[k][0], lim2), clamp_pair(v[k][1], lim2), scale);
                    w[1] = cvt4_scaled<FMT>(clamp_pair(v[k][2], lim2), clamp_pair(v[k][3], lim2), scale);
                    // a tile row's four block codes into its first lane (DPP row_shl 4, 8, 12)
                    const int rbase = lane & ~15;
                    const uint32_t word = code | (dppu<0x104>(code) << 8) | (dppu<0x108>(code) << 16) |
                                          (dppu<0x10C>(code) << 24);
                    if (col_in && r0 + rr < R) {
                        st8_stream(dst, w);
                        if (full_row_codes) {
                            if (lane == rbase)
                                *reinterpret_cast<uint32_t*>(edst + (cc & ~127) / 32) = word;
                        } else if ((lane & 3) == 0) {
                            edst[cc / 32] = (uint8_t)code;
                        }
                    }
                }
                if (q) {
                    dst += 16 * C;
                    edst += 16 * nbc;
                }
            }
        }
        if (!qt)
            continue;
        lds_barrier();
        // colwise: thread (p, rb) takes tile columns 2p, 2p+1, rows 32rb..+31
        const int pc = threadIdx.x & (64 * W - 1), rb = threadIdx.x / (64 * W);
        u32x4 w[4];
        uint32_t code0, code1;
        {
            uint32_t pr[32];
#pragma unroll
            for (int k = 0; k < 32; ++k)
                pr[k] = *reinterpret_cast<const uint32_t*>(tile + (32 * rb + k) * P + 2 * pc);
            uint32_t m = 0;
#pragma unroll
            for (int k = 0; k < 32; ++k)
                m = pk_max16(m, pr[k] & 0x7fff7fffu);
            code0 = mx_code_bf16<FMT>(m & 0xFFFFu);
            code1 = mx_code_bf16<FMT>(m >> 16);
            const uint32_t lim2 = mx_limit_bf16<FMT>(code0) | (mx_limit_bf16<FMT>(code1) << 16);
            const float s0 = e8m0_value(code0), s1 = e8m0_value(code1);
#pragma unroll
            for (int k = 0; k < 32; ++k)
                pr[k] = clamp_pair(pr[k], lim2);
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                // rows 4d..4d+3 of column 2p (low halves) and of column 2p+1 (high halves)
                const uint32_t a0 = __builtin_amdgcn_perm(pr[4 * d + 1], pr[4 * d], 0x05040100u);
                const uint32_t b0 = __builtin_amdgcn_perm(pr[4 * d + 3], pr[4 * d + 2], 0x05040100u);
                const uint32_t a1 = __builtin_amdgcn_perm(pr[4 * d + 1], pr[4 * d], 0x07060302u);
                const uint32_t b1 = __builtin_amdgcn_perm(pr[4 * d + 3], pr[4 * d + 2], 0x07060302u);
                w[d >> 2][d & 3] = cvt4_scaled<FMT>(a0, b0, s0);
                w[2 + (d >> 2)][d & 3] = cvt4_scaled<FMT>(a1, b1, s1);
            }
        }
        lds_barrier();
        uint8_t* otile = smem;             // [TW][kOP] codes of X^T
        uint8_t* ocode = smem + TW * kOP;  // [TW][4] E8M0 codes of X^T
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            *reinterpret_cast<u32x4*>(otile + otile_off(2 * pc + j, 2 * rb)) = w[2 * j];
            *reinterpret_cast<u32x4*>(otile + otile_off(2 * pc + j, 2 * rb + 1)) = w[2 * j + 1];
        }
        ocode[(2 * pc) * 4 + rb] = (uint8_t)code0;
        ocode[(2 * pc + 1) * 4 + rb] = (uint8_t)code1;
        lds_barrier();
        const int64_t nrows = min((int64_t)TW, C - c0), nbytes = min((int64_t)128, R - r0);
        {
            const int row0 = threadIdx.x >> 3, seg = (threadIdx.x & 7) * 16;
            uint8_t* dst = qt + (c0 + row0) * R + r0 + seg;
            const int64_t step = (NT / 8) * R;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int row = row0 + (NT / 8) * k;
                if (row < nrows && seg < nbytes)
                    st16_stream(dst, *reinterpret_cast<const u32x4*>(otile + otile_off(row, seg >> 4)));
                dst += step;
            }
        }
        if (threadIdx.x < nrows) {
            const int row = threadIdx.x;
            uint8_t* dst = et + (c0 + row) * nbr + r0 / 32;
            if (nbytes == 128 && (nbr & 3) == 0) {
                *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(ocode + row * 4);
            } else {
                for (int j = 0; j < nbytes / 32; ++j)
                    dst[j] = ocode[row * 4 + j];
            }
        }
    }
}

// ---------------------------------------------------------------- rowwise only, flat
// MX rowwise copy alone from bf16: the tensor is streamed as a flat array
// (C % 32 == 0, so a 1x32 block is 32 consecutive elements: a quad of
// lanes), each wave reading 1 KiB per load instruction with four loads in
// flight per lane; the same packed-bf16 amax, clamp and scaled converter as
// k_mx_bf16. Block codes are byte stores (ordinary: a wave's 16 codes meet in L2).
template <int FMT>
__global__ __launch_bounds__(kWG) void k_mx_row_bf16(const uint16_t* __restrict__ x, int64_t n,
                                                     uint8_t* __restrict__ q, uint8_t* __restrict__ e)
{
    constexpr int kL = 4;
    const int lane = threadIdx.x & 63;
    const int64_t nunits = cdiv(n, 512);
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), nwaves = (int64_t)gridDim.x * 4;
    for (int64_t u0 = wave * kL; u0 < nunits; u0 += nwaves * kL) {
        u32x4 v[kL];
#pragma unroll
        for (int j = 0; j < kL; ++j) {
            const int64_t el = (u0 + j) * 512 + lane * 8;
            v[j] = (u0 + j < nunits && el < n) ? ld16_stream(x + el) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kL; ++j) {
            if (u0 + j >= nunits)
                break;
            const int64_t el = (u0 + j) * 512 + lane * 8;
            uint32_t m = pk_max16(pk_max16(v[j][0] & 0x7fff7fffu, v[j][1] & 0x7fff7fffu),
                                  pk_max16(v[j][2] & 0x7fff7fffu, v[j][3] & 0x7fff7fffu));
            m = max(m & 0xFFFFu, m >> 16);
            m = max(m, dppu<kDppXor1>(m));
            m = max(m, dppu<kDppXor2>(m));  // the 1x32 block: a quad of lanes
            const uint32_t code = mx_code_bf16<FMT>(m);
            const uint32_t lim = mx_limit_bf16<FMT>(code), lim2 = lim | (lim << 16);
            const float scale = e8m0_value(code);
            u32x2 w;
            w[0] = cvt4_scaled<FMT>(clamp_pair(v[j][0], lim2), clamp_pair(v[j][1], lim2), scale);
            w[1] = cvt4_scaled<FMT>(clamp_pair(v[j][2], lim2), clamp_pair(v[j][3], lim2), scale);
            if (el < n) {
                st8_stream(q + el, w);
                if ((lane & 3) == 0)
                    e[el / 32] = (uint8_t)code;
            }
        }
    }
}

// ---------------------------------------------------------------- MXFP4 from bf16
// MXFP4 (E2M1 elements, two per byte) with the region walk of k_mx_bf16:
// both planes from one read of a 128-row x 256-column region per 512-thread
// workgroup. Magnitudes are clamped as bf16 patterns to 6 * 2^e (exact),
// then v_cvt_scalef32_pk_fp4_bf16 divides each pair by the power-of-two
// scale and rounds to nearest even. A row of X gets 128 bytes of codes per
// region (one line, from 32 lanes); a row of X^T gets 64 bytes (128 rows of
// 4-bit codes), written by four lanes.
constexpr int kOP4 = 64 + 16;  // pitch of the LDS tile of transposed FP4 codes

// four clamped bf16 pairs (elements 2i, 2i+1 in pair i) -> one dword of E2M1, element k in bits 4k..4k+3
__device__ __forceinline__ uint32_t cvt8_fp4_scaled(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3, float scale)
{
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, p0), scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, p1), scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, p2), scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, p3), scale, 3);
    return w;
}

__global__ __launch_bounds__(kMxTiles * kWG) void k_mxfp4_bf16(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ e,
                                                            uint8_t* __restrict__ qt, uint8_t* __restrict__ et)
{
    constexpr int W = kMxTiles, NT = W * kWG, TW = 128 * W, ROUNDS = 8, P = TW + 8;
    static_assert(TW * kOP4 + TW * 4 <= 128 * P * 2, "the code tile must fit in the input region it reuses");
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
    const int lane = threadIdx.x & 63;
    const int64_t ntc = cdiv(C, TW), ntiles = ntc * cdiv(R, 128);
    const int cc = (threadIdx.x & (16 * W - 1)) * 8, rr0 = threadIdx.x / (16 * W);
    const int64_t nbc = C / 32, nbr = R / 32;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * 128, c0 = tc * TW;
        const bool col_in = c0 + cc < C;
        u32x4 v[ROUNDS];
        {
            const uint16_t* src = x + (r0 + rr0) * C + c0 + cc;
            const int64_t step = 16 * C;
#pragma unroll
            for (int k = 0; k < ROUNDS; ++k) {
                v[k] = (col_in && r0 + rr0 + 16 * k < R) ? ld16_stream(src) : u32x4{0u, 0u, 0u, 0u};
                src += step;
            }
        }
        // whole u32 E8M0 words for this lane's 128-column tile
        const bool full_row_codes = c0 + (cc & ~127) + 128 <= C && (nbc & 3) == 0;
        if (qt)
            lds_barrier();  // the previous region's LDS reads are done
        {
            uint8_t* dst = q ? q + (r0 + rr0) * (C / 2) + (c0 + cc) / 2 : nullptr;
            uint8_t* edst = q ? e + (r0 + rr0) * nbc + c0 / 32 : nullptr;
#pragma unroll
            for (int k = 0; k < ROUNDS; ++k) {
                const int rr = rr0 + 16 * k;
                if (qt)
                    *reinterpret_cast<u32x4*>(tile + rr * P + cc) = v[k];
                if (q) {
                    uint32_t m = pk_max16(pk_max16(v[k][0] & 0x7fff7fffu, v[k][1] & 0x7fff7fffu),
                                          pk_max16(v[k][2] & 0x7fff7fffu, v[k][3] & 0x7fff7fffu));
                    m = max(m & 0xFFFFu, m >> 16);
                    m = max(m, dppu<kDppXor1>(m));
                    m = max(m, dppu<kDppXor2>(m));  // the 1x32 block: a quad of lanes
                    const uint32_t code = mx_code_bf16<kE2M1>(m);
                    const uint32_t lim = mx_limit_bf16<kE2M1>(code), lim2 = lim | (lim << 16);
                    const uint32_t w = cvt8_fp4_scaled(clamp_pair(v[k][0], lim2), clamp_pair(v[k][1], lim2),
                                                       clamp_pair(v[k][2], lim2), clamp_pair(v[k][3], lim2),
                                                       e8m0_value(code));
                    const int rbase = lane & ~15;
                    const uint32_t word = code | (dppu<0x104>(code) << 8) | (dppu<0x108>(code) << 16) |
                                          (dppu<0x10C>(code) << 24);
                    if (col_in && r0 + rr < R) {
                        st4_stream(dst, w);
                        if (full_row_codes) {
                            if (lane == rbase)
                                *reinterpret_cast<uint32_t*>(edst + (cc & ~127) / 32) = word;
                        } else if ((lane & 3) == 0) {
                            edst[cc / 32] = (uint8_t)code;
                        }
                    }
                    dst += 16 * (C / 2);
                    edst += 16 * nbc;
                }
            }
        }
        if (!qt)
            continue;
        lds_barrier();
        // colwise: thread (p, rb) takes region columns 2p, 2p+1, rows 32rb..+31
        const int pc = threadIdx.x & (64 * W - 1), rb = threadIdx.x / (64 * W);
        u32x4 w0, w1;
        uint32_t code0, code1;
        {
            uint32_t pr[32];
#pragma unroll
            for (int k = 0; k < 32; ++k)
                pr[k] = *reinterpret_cast<const uint32_t*>(tile + (32 * rb + k) * P + 2 * pc);
            uint32_t m = 0;
#pragma unroll
            for (int k = 0; k < 32; ++k)
                m = pk_max16(m, pr[k] & 0x7fff7fffu);
            code0 = mx_code_bf16<kE2M1>(m & 0xFFFFu);
            code1 = mx_code_bf16<kE2M1>(m >> 16);
            const uint32_t lim2 = mx_limit_bf16<kE2M1>(code0) | (mx_limit_bf16<kE2M1>(code1) << 16);
            const float s0 = e8m0_value(code0), s1 = e8m0_value(code1);
#pragma unroll
            for (int k = 0; k < 32; ++k)
                pr[k] = clamp_pair(pr[k], lim2);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                // rows 8d..8d+7: column 2p from the low halves, column 2p+1 from the high halves
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lo[i] = __builtin_amdgcn_perm(pr[8 * d + 2 * i + 1], pr[8 * d + 2 * i], 0x05040100u);
                    hi[i] = __builtin_amdgcn_perm(pr[8 * d + 2 * i + 1], pr[8 * d + 2 * i], 0x07060302u);
                }
                w0[d] = cvt8_fp4_scaled(lo[0], lo[1], lo[2], lo[3], s0);
                w1[d] = cvt8_fp4_scaled(hi[0], hi[1], hi[2], hi[3], s1);
            }
        }
        lds_barrier();
        uint8_t* otile = smem;              // [TW][kOP4] FP4 codes of X^T (64 bytes per row)
        uint8_t* ocode = smem + TW * kOP4;  // [TW][4] E8M0 codes of X^T
        *reinterpret_cast<u32x4*>(otile + (2 * pc) * kOP4 + 16 * rb) = w0;
        *reinterpret_cast<u32x4*>(otile + (2 * pc + 1) * kOP4 + 16 * rb) = w1;
        ocode[(2 * pc) * 4 + rb] = (uint8_t)code0;
        ocode[(2 * pc + 1) * 4 + rb] = (uint8_t)code1;
        lds_barrier();
        const int64_t nrows = min((int64_t)TW, C - c0), nbytes = min((int64_t)128, R - r0) / 2;
        {
            // 64 bytes of each X^T row per region: ordinary stores, so the two
            // halves of a line (from vertically adjacent regions) can meet in L2
            const int row0 = threadIdx.x >> 2, seg = (threadIdx.x & 3) * 16;
            uint8_t* dst = qt + (c0 + row0) * (R / 2) + r0 / 2 + seg;
            const int64_t step = (NT / 4) * (R / 2);
#pragma unroll
            for (int k = 0; k < TW / (NT / 4); ++k) {
                const int row = row0 + (NT / 4) * k;
                if (row < nrows && seg < nbytes)
                    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(otile + row * kOP4 + seg);
                dst += step;
            }
        }
        if (threadIdx.x < nrows) {
            const int row = threadIdx.x;
            uint8_t* dst = et + (c0 + row) * nbr + r0 / 32;
            if (nbytes == 64 && (nbr & 3) == 0) {
                *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(ocode + row * 4);
            } else {
                for (int j = 0; j < nbytes / 16; ++j)
                    dst[j] = ocode[row * 4 + j];
            }
        }
    }
}

}  // namespace

template <int FMT>
void launch_mx_t(const void* x, int in_bf16, int64_t R, int64_t C, uint8_t* q, uint8_t* e, uint8_t* qt,
                 uint8_t* et, hipStream_t stream)
{
    const int64_t ntiles = cdiv(C, 128) * cdiv(R, 128);
    if (in_bf16 && !qt) {
        const int64_t n = R * C;
        const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, (int64_t)kWG * 8 * 4), 16384));
        k_mx_row_bf16<FMT><<<grid, kWG, 0, stream>>>((const uint16_t*)x, n, q, e);
        return;
    }
    if (in_bf16) {
        // one region per workgroup: the hardware starts each workgroup as
        // another finishes (54.5 against 56.8 us per kernel at 8192x8192 for
        // a resident grid striding over the regions)
        const size_t lds = qt ? 128 * (128 * kMxTiles + 8) * 2 : 0;
        const int64_t nregions = cdiv(C, 128 * kMxTiles) * cdiv(R, 128);
        const unsigned grid = (unsigned)std::min<int64_t>(nregions, kMaxRegionGrid);
        k_mx_bf16<FMT><<<grid, kMxTiles * kWG, lds, stream>>>((const uint16_t*)x, R, C, q, e, qt, et);
    } else {
        const size_t lds = qt ? 128 * tile_pitch<float>() * 4 : 0;
        static ResidentGrid cache;
        const int64_t grid = std::min<int64_t>(ntiles, cache.get(k_mx<float, FMT>, kWG, lds));
        k_mx<float, FMT><<<(unsigned)grid, kWG, lds, stream>>>((const float*)x, R, C, q, e, qt, et);
    }
}

hipError_t launch_mxfp4_bf16(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, uint8_t* e, uint8_t* qt,
                             uint8_t* et, hipStream_t stream)
{
    // one region per workgroup, as for MXFP8
    const size_t lds = qt ? 128 * (128 * kMxTiles + 8) * 2 : 0;
    const int64_t nregions = cdiv(C, 128 * kMxTiles) * cdiv(R, 128);
    const unsigned grid = (unsigned)std::min<int64_t>(nregions, kMaxRegionGrid);
    k_mxfp4_bf16<<<grid, kMxTiles * kWG, lds, stream>>>(x, R, C, q, e, qt, et);
    return hipGetLastError();
}

hipError_t launch_mx(const void* x, int in_bf16, int fmt, int64_t R, int64_t C, uint8_t* q, uint8_t* e,
                     uint8_t* qt, uint8_t* et, hipStream_t stream)
{
    if (fmt == kE5M2)
        launch_mx_t<kE5M2>(x, in_bf16, R, C, q, e, qt, et, stream);
    else
        launch_mx_t<kE4M3>(x, in_bf16, R, C, q, e, qt, et, stream);
    return hipGetLastError();
}

}  // namespace fq
