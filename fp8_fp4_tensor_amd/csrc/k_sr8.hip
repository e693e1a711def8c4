// k_sr8.hip -- stochastic rounding of the elements to E4M3 or E5M2 for the
// per-tensor, blockwise 1x128 and MX recipes.
//
// Sources: [MP] "混合精度训练：fp16 到 fp8" (garden.houmin.site), section
// "FP8 数据格式" (rounding: round-to-nearest-even by default, stochastic
// rounding as an option that helps training stability), "FP8 recipe" items
// 3-5 (per-tensor current scaling, 1x128 tiles for inputs and gradients, MX
// 1x32 blocks) and "MXFP8 recipe"; [LP] "从 BF16 到 FP8/FP4" section 2.4
// item 5 (stochastic rounding on gradients). The scales are those of the
// round-to-nearest recipes; only the element rounding changes: an element's
// scaled value y = fp32(x * alpha) (MX: x * 2^-e, exact), clamped to
// +-Fmax, rounds up iff u + g * 2^16 >= 2^16, with u its 16 random bits and
// g its position between the two neighbouring codes.
//
// Random bits: element e of an output plane (its index in that plane's
// row-major order; the colwise plane is X^T) takes bits 16*(j%2)..+15 of
// word j/2, j = e % 8, of one Philox4x32-10 call with key = seed and counter
// (e / 8, 2 * offset + plane), plane 0 rowwise, 1 colwise -- the mapping of
// the NVFP4 stochastic rounding. Each plane draws its own bits, so with
// stochastic rounding the colwise copy of a per-tensor recipe is the recipe
// applied to X^T, not the transposed rowwise bytes.
//
//   k_sr8_row  flat over the tensor: a lane holds 16 bytes per unit (8 bf16
//              or 4 fp32 elements, one Philox group or half of one), two
//              units per step; 1x128 and 1x32 block maxima by DPP across the
//              lanes of a block.
//   k_sr8_col  a 128-row x 64-column tile of X staged in LDS as fp32 (rows
//              XOR-swizzled by 32-row quarter); thread (c, q) takes column
//              c, rows 32q..32q+31: one MX block, a quarter of a 1x128 block
//              (the four quarters of a column are a quad of lanes: DPP max),
//              and writes 32 consecutive bytes of row c of X^T. For
//              per-tensor and MX calls with both planes it also writes the
//              rowwise plane from the same tile (thread (r, h): 32 columns
//              of row r), so the input is read once. With 16-byte rows a
//              resident grid takes the tiles in turn, each workgroup
//              issuing the next tile's loads once the current one is in
//              LDS (the rounding is long enough to hide them); otherwise
//              one tile per workgroup, or several beyond 16384 tiles.
#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace fq {
namespace {

enum { kSrTensor = 0, kSrBlock128 = 1, kSrMx32 = 2 };

constexpr int kRowMaxGrid = 16384, kRowTensorMaxGrid = 2048, kRowLoads = 2;
constexpr int kColRows = 128, kColCols = 64;
// k_sr8_col: one tile per workgroup up to this many tiles, beyond it each
// workgroup strides over several (a tall, narrow tensor would otherwise pass
// 2^32 work-items)
constexpr int64_t kColMaxGrid = 16384;

// alpha, s and the amax of a per-tensor cast from its scale source
// (every workgroup re-reduces the amax partials). Uniform control flow.
template <int FMT>
__device__ __forceinline__ void tensor_scale_from(const ScaleSrc& src, float* lds, float& alpha, float& s, float& a)
{
    if (src.amax_in) {
        a = *src.amax_in;
    } else {
        const float m = partials_max(src.partials, src.n_partials);
        a = max_workgroup(m, lds);
    }
    tensor_scales(a, Fmt<FMT>::kMax, alpha, s);
}

// Multiplier and stored scale of a 1x128 block (E4M3) from its amax:
// alpha = 448 / a and s = a / 448, or the power of two 2^-(floor(log2 a) - 8)
// and its inverse.
template <bool POW2>
__device__ __forceinline__ void block_scale(float a, float& mult, float& s)
{
    if constexpr (POW2) {
        const uint32_t code = mx_code<kE4M3>(a);
        mult = mx_multiplier(code);
        s = e8m0_value(code);
    } else {
        tensor_scales(a, 448.0f, mult, s);
    }
}

// Four scaled values (clamped here) with their 16-bit randoms -> one dword of codes.
template <int FMT>
__device__ __forceinline__ uint32_t sr4(const float* y, float mult, uint32_t w0, uint32_t w1)
{
    constexpr float M = Fmt<FMT>::kMax;
    return gather_byte0(sr8_byte0<FMT>(clampf(y[0] * mult, M), w0 & 0xFFFFu),
                        sr8_byte0<FMT>(clampf(y[1] * mult, M), w0 >> 16),
                        sr8_byte0<FMT>(clampf(y[2] * mult, M), w1 & 0xFFFFu),
                        sr8_byte0<FMT>(clampf(y[3] * mult, M), w1 >> 16));
}

// The 16 random bits of element e of a plane (one Philox call).
__device__ __forceinline__ uint32_t sr_bits_of(int64_t e, uint64_t s, uint64_t seed)
{
    const Philox4 ph = sr_group((uint64_t)e >> 3, s, seed);
    const int j = (int)(e & 7);
    const uint32_t w = j < 2 ? ph.w[0] : j < 4 ? ph.w[1] : j < 6 ? ph.w[2] : ph.w[3];
    return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Rowwise plane: n elements flat; per-tensor (src), 1x128 or 1x32 blocks
// (n a multiple of the block length, so a block lies in one 16-byte unit
// group and never straddles the end). A wave takes L consecutive units per
// step, their loads issued together. s_out / amax_out: per-tensor only.
template <typename T, int FMT, int KIND, bool POW2, int L>
__global__ __launch_bounds__(kWG) void k_sr8_row(const T* __restrict__ x, int64_t n, ScaleSrc src, uint64_t seed,
                                                 uint64_t stream_s, uint8_t* __restrict__ q, void* __restrict__ sc,
                                                 float* s_out, float* amax_out)
{
    __shared__ float lds[4];
    constexpr int E = In<T>::kE, U = 64 * E;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), nwaves = (int64_t)gridDim.x * 4;
    float alpha = 1.0f;
    if constexpr (KIND == kSrTensor) {
        float s, a;
        tensor_scale_from<FMT>(src, lds, alpha, s, a);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            if (s_out)
                *s_out = s;
            if (amax_out)
                *amax_out = a;
        }
    }
    // per-tensor: whole units here, the ragged tail below; blocks: every unit,
    // lanes past the end idle (a block is never cut by the end)
    const int64_t nunits = KIND == kSrTensor ? n / U : cdiv(n, U);
    for (int64_t u0 = wave * L; u0 < nunits; u0 += nwaves * L) {
        u32x4 v[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const int64_t e = (u0 + j) * U + lane * E;
            v[j] = (u0 + j < nunits && e < n) ? ld16_stream(x + e) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (u0 + j >= nunits)
                break;
            const int64_t e = (u0 + j) * U + lane * E;
            const bool in = e < n;
            float mult = alpha;
            if constexpr (KIND == kSrBlock128) {
                constexpr int LPB = 128 / E;
                float s;
                block_scale<POW2>(max_lanes<LPB>(In<T>::absmax16(v[j])), mult, s);
                if (in && (lane & (LPB - 1)) == 0)
                    reinterpret_cast<float*>(sc)[e / 128] = s;
            } else if constexpr (KIND == kSrMx32) {
                constexpr int LPB = 32 / E;
                const uint32_t code = mx_code<FMT>(max_lanes<LPB>(In<T>::absmax16(v[j])));
                mult = mx_multiplier(code);
                if (in && (lane & (LPB - 1)) == 0)
                    reinterpret_cast<uint8_t*>(sc)[e / 32] = (uint8_t)code;
            }
            if (!in)
                continue;
            float f[E];
            In<T>::unpack(v[j], f);
            const Philox4 ph = sr_group((uint64_t)e >> 3, stream_s, seed);
            if constexpr (E == 8) {
                u32x2 w;
                w[0] = sr4<FMT>(f, mult, ph.w[0], ph.w[1]);
                w[1] = sr4<FMT>(f + 4, mult, ph.w[2], ph.w[3]);
                st8_stream(q + e, w);
            } else {
                const bool upper = (e & 4) != 0;  // elements 4..7 of the group
                st4_stream(q + e, sr4<FMT>(f, mult, upper ? ph.w[2] : ph.w[0], upper ? ph.w[3] : ph.w[1]));
            }
        }
    }
    if constexpr (KIND == kSrTensor) {
        for (int64_t i = nunits * U + (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG)
            q[i] = (uint8_t)sr8_byte0<FMT>(clampf(In<T>::load1(x, i) * alpha, Fmt<FMT>::kMax),
                                           sr_bits_of(i, stream_s, seed));
    }
}

// LDS offset (floats) of element (r, c) of the 128 x 64 tile: 32-row quarter
// q of a row XOR-swizzles the column by 16 q, so the four quarters a quad of
// lanes reads at once fall in different banks.
// 32 consecutive elements of a plane (element index e0, n of them valid)
// from fp32 values y times mult: with n == 32 and e0 a multiple of 16, four
// Philox groups and two 16-byte stores; otherwise element by element.
template <int FMT>
__device__ __forceinline__ void sr_run32(const float* y, float mult, uint8_t* dst, int64_t e0, int64_t n,
                                         bool aligned16, uint64_t stream_s, uint64_t seed)
{
    if (aligned16 && n == 32) {
        u32x4 w[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const Philox4 ph = sr_group((uint64_t)(e0 >> 3) + g, stream_s, seed);
            w[g >> 1][2 * (g & 1)] = sr4<FMT>(y + 8 * g, mult, ph.w[0], ph.w[1]);
            w[g >> 1][2 * (g & 1) + 1] = sr4<FMT>(y + 8 * g + 4, mult, ph.w[2], ph.w[3]);
        }
        *reinterpret_cast<u32x4*>(dst) = w[0];
        *reinterpret_cast<u32x4*>(dst + 16) = w[1];
    } else {
        for (int k = 0; k < 32 && k < n; ++k)
            dst[k] = (uint8_t)sr8_byte0<FMT>(clampf(y[k] * mult, Fmt<FMT>::kMax), sr_bits_of(e0 + k, stream_s, seed));
    }
}

// The pitch P is kColCols, or kColCols + 4 floats when the tile's rows are
// also read along the row (16-byte reads, rows of a wave 272 bytes apart).
template <int P>
__device__ __forceinline__ int col_tile_off(int r, int c) { return r * P + (c ^ (((r >> 5) & 3) << 4)); }

// Colwise plane (X^T): per-tensor (src), 1x128 blocks (R % 128 == 0) or 1x32
// blocks (R % 32 == 0) down the columns of X. VEC: rows of X are 16-byte
// aligned and 16-byte multiples (C % (16 / sizeof(T)) == 0). ROW (per-tensor
// and MX): the rowwise plane too, from the same staged tile: thread (r, h)
// rounds columns 32h .. 32h+31 of tile row r (one MX block) with the rowwise
// random bits (stream_row).
// At most 128 registers, so that four workgroups fit on a CU as the LDS tile allows.
template <typename T, int FMT, int KIND, bool POW2, bool VEC, bool ROW>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4))) void k_sr8_col(const T* __restrict__ x, int64_t R, int64_t C, ScaleSrc src,
                                                 uint64_t seed, uint64_t stream_s, uint8_t* __restrict__ qt,
                                                 void* __restrict__ sct, float* s_out, float* amax_out,
                                                 uint64_t stream_row, uint8_t* __restrict__ q, void* __restrict__ sq)
{
    static_assert(!ROW || KIND != kSrBlock128, "a 1x128 block is wider than the tile");
    constexpr int P = ROW ? kColCols + 4 : kColCols;
    __shared__ __align__(16) float tile[kColRows * P];
    __shared__ float lds[4];
    const int64_t ntc = cdiv(C, kColCols), ntiles = ntc * cdiv(R, kColRows);
    float alpha = 1.0f;
    if constexpr (KIND == kSrTensor) {
        float s, a;
        tensor_scale_from<FMT>(src, lds, alpha, s, a);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            if (s_out)
                *s_out = s;
            if (amax_out)
                *amax_out = a;
        }
    }
    // VEC: 16-byte loads, the next tile's issued into registers once this
    // one is in LDS, so they are in flight while this tile is rounded
    constexpr int E = In<T>::kE, SEGS = kColCols / E, NLV = kColRows * SEGS / kWG;
    u32x4 v[NLV];
    auto load_vec = [&](int64_t t) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * kColRows, c0 = tc * kColCols;
#pragma unroll
        for (int k = 0; k < NLV; ++k) {
            const int i = k * kWG + (int)threadIdx.x, row = i / SEGS, col = (i % SEGS) * E;
            const bool in = r0 + row < R && c0 + col < C;
            v[k] = in ? ld16_stream(x + (r0 + row) * C + c0 + col) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    int64_t t = blockIdx.x;
    if constexpr (VEC) {
        if (t < ntiles)
            load_vec(t);
    }
    for (; t < ntiles; t += gridDim.x) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * kColRows, c0 = tc * kColCols;
        // stage the tile as fp32 (zeros outside the tensor)
        if constexpr (VEC) {
#pragma unroll
            for (int k = 0; k < NLV; ++k) {
                const int i = k * kWG + (int)threadIdx.x, row = i / SEGS, col = (i % SEGS) * E;
                float f[E];
                In<T>::unpack(v[k], f);
#pragma unroll
                for (int j = 0; j < E; j += 4)
                    *reinterpret_cast<float4*>(tile + col_tile_off<P>(row, col + j)) =
                        make_float4(f[j], f[j + 1], f[j + 2], f[j + 3]);
            }
        } else {
            constexpr int NL = kColRows * kColCols / kWG;
#pragma unroll 8
            for (int k = 0; k < NL; ++k) {
                const int i = k * kWG + (int)threadIdx.x, row = i / kColCols, col = i % kColCols;
                const bool in = r0 + row < R && c0 + col < C;
                tile[col_tile_off<P>(row, col)] = in ? In<T>::load1(x, (r0 + row) * C + c0 + col) : 0.0f;
            }
        }
        lds_barrier();  // LDS only: the previous tile's stores and the loads below stay in flight
        if constexpr (VEC) {
            if (t + gridDim.x < ntiles)
                load_vec(t + gridDim.x);
        }
        const int c = (int)threadIdx.x >> 2, qr = (int)threadIdx.x & 3;
        float y[32];
#pragma unroll
        for (int k = 0; k < 32; ++k)
            y[k] = tile[col_tile_off<P>(32 * qr + k, c)];
        float mult = alpha;
        const bool col_in = c0 + c < C;
        if constexpr (KIND == kSrBlock128) {
            float s;
            block_scale<POW2>(max_lanes4(absmax<32>(y)), mult, s);
            if (col_in && qr == 0)
                reinterpret_cast<float*>(sct)[(c0 + c) * (R / 128) + r0 / 128] = s;
        } else if constexpr (KIND == kSrMx32) {
            const uint32_t code = mx_code<FMT>(absmax<32>(y));
            mult = mx_multiplier(code);
            if (col_in && r0 + 32 * qr < R)
                reinterpret_cast<uint8_t*>(sct)[(c0 + c) * (R / 32) + r0 / 32 + qr] = (uint8_t)code;
        }
        if (col_in)
            sr_run32<FMT>(y, mult, qt + (c0 + c) * R + r0 + 32 * qr, (c0 + c) * R + r0 + 32 * qr,
                          min((int64_t)32, R - r0 - 32 * qr), (R & 15) == 0, stream_s, seed);
        if constexpr (ROW) {
            const int row = (int)threadIdx.x >> 1, h = (int)threadIdx.x & 1;
            const int64_t gr = r0 + row, gc = c0 + 32 * h;
            if (gr < R && gc < C) {
                float z[32];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float4 v = *reinterpret_cast<const float4*>(tile + col_tile_off<P>(row, 32 * h + 4 * k));
                    z[4 * k] = v.x;
                    z[4 * k + 1] = v.y;
                    z[4 * k + 2] = v.z;
                    z[4 * k + 3] = v.w;
                }
                float rmult = alpha;
                if constexpr (KIND == kSrMx32) {
                    const uint32_t code = mx_code<FMT>(absmax<32>(z));
                    rmult = mx_multiplier(code);
                    reinterpret_cast<uint8_t*>(sq)[gr * (C / 32) + gc / 32] = (uint8_t)code;
                }
                sr_run32<FMT>(z, rmult, q + gr * C + gc, gr * C + gc, min((int64_t)32, C - gc), (C & 15) == 0,
                              stream_row, seed);
            }
        }
        lds_barrier();  // the tile's LDS reads are done before the next tile is staged
    }
}

template <typename T, int FMT, int KIND, bool POW2, bool ROW>
void launch_col(const T* x, int64_t R, int64_t C, ScaleSrc src, SrArgs sr, uint8_t* qt, void* sqt, float* s_out,
                float* amax_out, uint8_t* q, void* sq, hipStream_t stream)
{
    const int64_t ntiles = cdiv(R, kColRows) * cdiv(C, kColCols);
    if (C % In<T>::kE == 0) {
        // a resident grid: each workgroup rounds several tiles, loading the next during each
        static ResidentGrid cache;
        const unsigned grid = (unsigned)std::min<int64_t>(
            ntiles, std::min<int64_t>(kColMaxGrid, cache.get(k_sr8_col<T, FMT, KIND, POW2, true, ROW>, kWG, 0)));
        k_sr8_col<T, FMT, KIND, POW2, true, ROW><<<grid, kWG, 0, stream>>>(
            x, R, C, src, sr.seed, 2 * sr.offset + 1, qt, sqt, s_out, amax_out, 2 * sr.offset, q, sq);
    } else {
        const unsigned grid = (unsigned)std::min<int64_t>(ntiles, kColMaxGrid);
        k_sr8_col<T, FMT, KIND, POW2, false, ROW><<<grid, kWG, 0, stream>>>(
            x, R, C, src, sr.seed, 2 * sr.offset + 1, qt, sqt, s_out, amax_out, 2 * sr.offset, q, sq);
    }
}

template <typename T, int FMT, int KIND, bool POW2>
void launch_t(const void* xv, int64_t R, int64_t C, ScaleSrc src, SrArgs sr, uint8_t* q, void* sq, uint8_t* qt,
              void* sqt, float* s_out, float* amax_out, hipStream_t stream)
{
    const T* x = reinterpret_cast<const T*>(xv);
    const int64_t n = R * C;
    // both planes of per-tensor and MX calls: one kernel, one read
    if constexpr (KIND != kSrBlock128) {
        if (q && qt && n > 0) {
            launch_col<T, FMT, KIND, POW2, true>(x, R, C, src, sr, qt, sqt, s_out, amax_out, q, sq, stream);
            return;
        }
    }
    // an empty per-tensor call still writes s and the amax (1 and 0)
    if (q || (n == 0 && KIND == kSrTensor)) {
        // per-tensor: at most 2048 workgroups, since each re-reduces the amax partials
        const int64_t per = (int64_t)kWG * In<T>::kE * kRowLoads;
        const int64_t cap = KIND == kSrTensor ? kRowTensorMaxGrid : kRowMaxGrid;
        const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, per), cap));
        k_sr8_row<T, FMT, KIND, POW2, kRowLoads><<<grid, kWG, 0, stream>>>(x, n, src, sr.seed, 2 * sr.offset, q, sq,
                                                                           s_out, amax_out);
    }
    if (qt && n > 0)  // s and the amax are written once, by the rowwise pass if there is one
        launch_col<T, FMT, KIND, POW2, false>(x, R, C, src, sr, qt, sqt, q ? nullptr : s_out,
                                              q ? nullptr : amax_out, nullptr, nullptr, stream);
}

template <typename T, int KIND, bool POW2>
void launch_fmt(int fmt, const void* x, int64_t R, int64_t C, ScaleSrc src, SrArgs sr, uint8_t* q, void* sq,
                uint8_t* qt, void* sqt, float* s_out, float* amax_out, hipStream_t stream)
{
    if (fmt == kE4M3)
        launch_t<T, kE4M3, KIND, POW2>(x, R, C, src, sr, q, sq, qt, sqt, s_out, amax_out, stream);
    else
        launch_t<T, kE5M2, KIND, POW2>(x, R, C, src, sr, q, sq, qt, sqt, s_out, amax_out, stream);
}

template <typename T>
void launch_kind(int kind, int pow2, int fmt, const void* x, int64_t R, int64_t C, ScaleSrc src, SrArgs sr,
                 uint8_t* q, void* sq, uint8_t* qt, void* sqt, float* s_out, float* amax_out, hipStream_t stream)
{
    if (kind == kSrTensor)
        launch_fmt<T, kSrTensor, false>(fmt, x, R, C, src, sr, q, sq, qt, sqt, s_out, amax_out, stream);
    else if (kind == kSrBlock128 && pow2)
        launch_t<T, kE4M3, kSrBlock128, true>(x, R, C, src, sr, q, sq, qt, sqt, s_out, amax_out, stream);
    else if (kind == kSrBlock128)
        launch_t<T, kE4M3, kSrBlock128, false>(x, R, C, src, sr, q, sq, qt, sqt, s_out, amax_out, stream);
    else
        launch_fmt<T, kSrMx32, false>(fmt, x, R, C, src, sr, q, sq, qt, sqt, s_out, amax_out, stream);
}

}  // namespace

hipError_t launch_sr8(const void* x, int in_bf16, int fmt, int kind, int pow2, int64_t R, int64_t C, ScaleSrc src,
                      SrArgs sr, uint8_t* q, void* sq, uint8_t* qt, void* sqt, float* s_out, float* amax_out,
                      hipStream_t stream)
{
    if (in_bf16)
        launch_kind<uint16_t>(kind, pow2, fmt, x, R, C, src, sr, q, sq, qt, sqt, s_out, amax_out, stream);
    else
        launch_kind<float>(kind, pow2, fmt, x, R, C, src, sr, q, sq, qt, sqt, s_out, amax_out, stream);
    return hipGetLastError();
}

}  // namespace fq
