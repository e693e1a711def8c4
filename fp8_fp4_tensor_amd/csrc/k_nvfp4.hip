// k_nvfp4.hip -- NVFP4: E2M1 elements packed two per byte, 1x16 or 16x16
// blocks with an E4M3 block scale, plus one fp32 tensor-level scale.
//
// Sources: [MP] "混合精度训练：fp16 到 fp8" (garden.houmin.site), section
// "FP8 recipe" item 6 (1x16 blocks, E4M3 scales, one extra fp32 global
// scale that makes up for E4M3's narrow range) and section "NVFP4" (the
// float4_e2m1fn_x2 layout: two values per byte, 16 values); [LP] "从 BF16 到
// FP8/FP4" section 2.4 (E2M1 elements, 16-element blocks with an E4M3 scale
// and an FP32 tensor scale; 16x16 blocks for weights, 1x16 for activations
// and gradients; round to nearest even).
//
// The two scale levels follow the per-tensor rule applied to the block
// scales themselves: with A the tensor amax, the block decode scales a_B/6
// form a tensor whose amax is A/6; it is quantized to E4M3 with current
// scaling, alpha_s = 448/fp32(A/6), S = fp32(A/6)/448 (S is stored):
//   c_B = Q_E4M3(fp32(fp32(a_B/6) * alpha_s)),  d_B = fp32(dec(c_B) * S),
//   r_B = 1/d_B (0 if d_B = 0),  q = Q_E2M1(fp32(x * r_B)).
// Two divisions per block (a_B/6 and 1/d_B), none per element.
//
// The amax pass (k_amax_partial) runs first; each workgroup of the block
// pass re-reduces its partials to get A.
//   k_nvfp4_1x16   flat: a 1x16 block is two lanes of bf16 (four of fp32),
//                  one DPP step; each lane writes one packed dword.
//   k_nvfp4_16x16  each lane owns E columns of a 16-row strip (16 loads), so
//                  a 16x16 block is again two lanes; one DPP step.
//   k_nvfp4_colt   colwise 1x16 copy (blocks of 16 rows of one column): a
//                  128 x 64 tile in LDS, four lanes per column, each X^T row
//                  written as 64-byte segments (optionally with SR and RHT).
//   k_nvfp4_col    colwise 16x16 copy: a 32-row slab in LDS, one thread per
//                  column; the same blocks as rowwise (max also across 16
//                  neighbouring lanes), so the nibbles are the rowwise ones
//                  transposed.
//   k_rht_amax_partial, k_nvfp4_col<..., RHT>  the random Hadamard transform
//                  of weight-gradient inputs ([LP] 2.4 item 3): 16-row chunks
//                  of each column transformed in registers in both passes.
//   k_nvfp4_1x16_sr  stochastic rounding of the elements ([MP] "NVFP4"; [LP]
//                  2.4 item 5): a lane owns a whole 1x16 block, which is two
//                  Philox4x32-10 calls (8 x 16 random bits each); the colwise
//                  kernel takes the same path per 16-row block.
#include <algorithm>
#include <type_traits>

#include "codec.hpp"
#include "launch.hpp"

namespace fq {
namespace {

constexpr int kLoads = 4;
// Rowwise 1x16 pass 2: fewer, longer-lived workgroups, so the per-workgroup
// set-up (tensor scale from the partials, the multiplier table) is paid less
// often: at 8192x14336 both passes take 82 us with 4096 workgroups,
// 89 us with 14336 (one per four 1 KiB units per wave), 85 us with 2048.
// The same cap serves the stochastic-rounding kernel (101 us against
// 110 us with 16384 workgroups of 256 blocks).
constexpr int kMaxGrid1x16 = 4096;
// Colwise 1x16 (k_nvfp4_colt): workgroups stride over 128 x 64 tiles, the
// set-up paid once per workgroup.
constexpr int kMaxGridColt = 2048;
// 16x16 strips and colwise slabs: one per workgroup up to 2^16 of them
// (every transformer-linear shape here), beyond that workgroups stride over
// them, so a grid stays far below 2^32 work-items
constexpr int64_t kMaxSlabGrid = int64_t(1) << 16;

// fp32(a / 6) for a >= 0, correctly rounded: q = a * RN(1/6), the residual
// a - 6q (exact), one correction step. An exhaustive check over every fp32
// a >= 2^-125 finds it equal to the division; below that (quotients in the
// subnormal range, where the residual is no longer exact) the division runs.
__device__ __forceinline__ float div6(float a)
{
    if (__builtin_expect(a >= 0x1p-125f, 1)) {
        constexpr float zh = 0x1.555556p-3f;  // RN(1/6)
        const float q = a * zh;
        return __builtin_fmaf(__builtin_fmaf(-q, 6.0f, a), zh, q);
    }
    return a / 6.0f;
}

// Tensor-level scale from the amax source, and the table of element
// multipliers r(c) = 1 / (dec(c) * S) for every block scale code c (a code
// is at most 0x7E: b * alpha_s is clamped to [0, 448]), so a block's
// multiplier is a lookup instead of a division. Uniform control flow; ends
// with a workgroup barrier.
__device__ __forceinline__ void nvfp4_tensor(const ScaleSrc& src, float* lds, float* rtab, float& alpha_s, float& S,
                                             float& A)
{
    if (src.amax_in) {
        A = *src.amax_in;
    } else {
        const float m = partials_max(src.partials, src.n_partials);
        A = max_workgroup(m, lds);
    }
    tensor_scales(A / 6.0f, 448.0f, alpha_s, S);
    if (threadIdx.x < 128) {
        const float d = dec_e4m3(threadIdx.x) * S;
        rtab[threadIdx.x] = (d == 0.0f) ? 0.0f : fminf(1.0f / d, kFLT_MAX);
    }
    __syncthreads();
}

// Block scale code and element multiplier from a block amax:
// b = a/6, c = Q_E4M3(b * alpha_s), r = 1 / (dec(c) * S) (0 when that is 0).
// For finite inputs c is a non-negative code, at most 0x7E; a NaN product
// (non-finite input) would clamp to -448 and give 0xFE, so the table index
// keeps the low seven bits and stays inside the table whatever the input.
__device__ __forceinline__ void nvfp4_block(float a, float alpha_s, const float* rtab, uint32_t& code, float& r)
{
    const float b = div6(a);
    code = enc_e4m3_one(clampf(b * alpha_s, 448.0f));
    r = rtab[code & 0x7Fu];
}

// E values times r -> E/2 packed bytes (E = 8: a dword; E = 4: 16 bits).
template <int E>
struct Fp4Store;
template <>
struct Fp4Store<8> {
    __device__ static __forceinline__ void store(uint8_t* p, const float* f, float r)
    {
        st4_stream(p, enc8_e2m1(f, r));
    }
};
template <>
struct Fp4Store<4> {
    __device__ static __forceinline__ void store(uint8_t* p, const float* f, float r)
    {
        uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, clampf(f[0] * r, 6.0f), clampf(f[1] * r, 6.0f),
                                                              1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clampf(f[2] * r, 6.0f), clampf(f[3] * r, 6.0f), 1.0f, 1);
        *reinterpret_cast<uint16_t*>(p) = (uint16_t)w;
    }
};

// ---------------------------------------------------------------- stochastic rounding
// Stochastic rounding to E2M1 with gfx950's v_cvt_scalef32_sr_pk_fp4_f32 at
// unit scale. For its first value the converter adds bits 31..10 of its
// random word below the last kept bit and truncates (saturating at 6, sign
// kept); with a word whose bits 31..16 are u and 15..0 zero this is exactly
// "round up iff u + g * 2^16 >= 2^16". Its second value would read bits
// 30..9 of the same word, so each element gets a call of its own, with 0 as
// the second value: bits 3..0 of the result are the element's code and bits
// 7..4 are 0 (code 0 for any random word). Only byte 0 of a result is
// defined: the compiler does not carry the other bytes of the destination
// through this builtin.
__device__ __forceinline__ uint32_t sr_byte0(float y, uint32_t word_hi16)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, f32x2{y, 0.0f}, word_hi16, 1.0f, 0);
}

// 8 values (times r, stochastically rounded with one group's random bits:
// element 2k takes bits 15..0 of word k, element 2k+1 bits 31..16) -> one
// dword of packed E2M1, element j in bits 4j..4j+3. Byte 0 of
// lo | hi << 4 is the pair's byte (the other bytes are undefined); v_perm
// gathers the four byte 0s.
__device__ __forceinline__ uint32_t enc8_e2m1_sr(const float* f, float r, const Philox4& ph)
{
    uint32_t t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        t[k] = sr_byte0(f[2 * k] * r, ph.w[k] << 16) | (sr_byte0(f[2 * k + 1] * r, ph.w[k] & 0xFFFF0000u) << 4);
    // v_perm_b32(a, b, sel): selector byte i picks byte sel_i of {a:b} (0..3 from b, 4..7 from a), 0x0c gives 0
    const uint32_t lo = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(t[3], t[2], 0x04000c0cu);
    return lo | hi;
}

// ---------------------------------------------------------------- random Hadamard transform
// ([LP] 2.4 item 3) y = (1/4) H16 diag(s) x on 16 values in registers: the
// sign flips (exact), the fast Walsh-Hadamard butterfly in fp32 with stages
// h = 1, 2, 4, 8 (pair (i, i+h), bit h of i clear -> (a + b, a - b): the
// same additions, in the same order, as the transform's definition), and
// the exact factor 1/4. 64 additions for 16 values.
__device__ __forceinline__ void rht16(float* f, uint32_t signs)
{
#pragma unroll
    for (int i = 0; i < 16; ++i)
        f[i] = ((signs >> i) & 1u) ? -f[i] : f[i];
#pragma unroll
    for (int h = 1; h < 16; h *= 2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (!(i & h)) {
                const float a = f[i], b = f[i + h];
                f[i] = a + b;
                f[i + h] = a - b;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
        f[i] *= 0.25f;
}

// Amax of the transformed X^T. A thread holds a 16-row strip of E columns
// in registers (16 loads; a wave reads 1 KiB of each row), transforms each
// column's 16 values and keeps the max; workgroups stride over strips; one
// partial per workgroup. Ordinary loads, so the block pass that follows
// finds the tensor in the memory-side cache.
template <typename T>
__global__ __launch_bounds__(kWG) void k_rht_amax_partial(const T* __restrict__ x, int64_t R, int64_t C,
                                                          uint32_t signs, float* __restrict__ partials)
{
    __shared__ float lds[4];
    constexpr int E = In<T>::kE, WC = kWG * E;  // columns per workgroup strip
    const int64_t nwc = cdiv(C, WC), nstrips = (R / 16) * nwc;
    float m = 0.0f;
    for (int64_t st = blockIdx.x; st < nstrips; st += gridDim.x) {
        const int64_t r0 = (st / nwc) * 16;
        const int64_t c = (st % nwc) * WC + (int64_t)threadIdx.x * E;
        if (c >= C)
            continue;
        u32x4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = ld16(x + (r0 + i) * C + c);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            float f[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (E == 8)
                    f[i] = (j & 1) ? bf16_hi(v[i][j >> 1]) : bf16_lo(v[i][j >> 1]);
                else
                    f[i] = __uint_as_float(v[i][j]);
            }
            rht16(f, signs);
            m = fmaxf(m, absmax<16>(f));
        }
    }
    const float a = max_workgroup(m, lds);
    if (threadIdx.x == 0)
        partials[blockIdx.x] = a;
}

// Rowwise 1x16 with stochastic rounding: thread = block of 16 elements
// (two 16-byte loads of bf16, four of fp32), grid-stride over blocks, the
// next block's loads issued before the current block's arithmetic.
template <typename T>
__global__ __launch_bounds__(kWG) void k_nvfp4_1x16_sr(const T* __restrict__ x, int64_t nblk, ScaleSrc src,
                                                       uint64_t seed, uint64_t offset, uint8_t* __restrict__ p,
                                                       uint8_t* __restrict__ codes, float* S_out, float* amax_out)
{
    __shared__ float lds[4];
    __shared__ float rtab[128];
    constexpr int E = In<T>::kE, NL = 16 / E;
    const int64_t first = (int64_t)blockIdx.x * kWG + threadIdx.x, stride = (int64_t)gridDim.x * kWG;
    u32x4 v[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k)
        v[k] = first < nblk ? ld16_stream(x + first * 16 + k * E) : u32x4{0u, 0u, 0u, 0u};
    float alpha_s, S, A;
    nvfp4_tensor(src, lds, rtab, alpha_s, S, A);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (S_out)
            *S_out = S;
        if (amax_out)
            *amax_out = A;
    }
    for (int64_t b = first; b < nblk; b += stride) {
        float f[16];
#pragma unroll
        for (int k = 0; k < NL; ++k)
            In<T>::unpack(v[k], f + k * E);
        const int64_t nb = b + stride;
#pragma unroll
        for (int k = 0; k < NL; ++k)
            v[k] = nb < nblk ? ld16_stream(x + nb * 16 + k * E) : u32x4{0u, 0u, 0u, 0u};
        uint32_t code;
        float r;
        nvfp4_block(absmax<16>(f), alpha_s, rtab, code, r);
        const uint64_t s = 2 * offset;  // plane 0
        u32x2 out;
        out[0] = enc8_e2m1_sr(f, r, sr_group(2 * (uint64_t)b, s, seed));
        out[1] = enc8_e2m1_sr(f + 8, r, sr_group(2 * (uint64_t)b + 1, s, seed));
        st8_stream(p + b * 8, out);
        codes[b] = (uint8_t)code;
    }
}

template <typename T>
__global__ __launch_bounds__(kWG) void k_nvfp4_1x16(const T* __restrict__ x, int64_t n, ScaleSrc src,
                                                    uint8_t* __restrict__ p, uint8_t* __restrict__ codes,
                                                    float* S_out, float* amax_out)
{
    __shared__ float lds[4];
    __shared__ float rtab[128];
    constexpr int E = In<T>::kE, U = 64 * E, LPB = 16 / E;
    const int lane = threadIdx.x & 63;
    const int64_t nunits = cdiv(n, U);
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    // the first step's loads go out before the tensor scale is resolved
    u32x4 v[kLoads];
    int64_t u0 = wave * kLoads;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int64_t e = (u0 + j) * U + lane * E;
        v[j] = (u0 + j < nunits && e < n) ? ld16_stream(x + e) : u32x4{0u, 0u, 0u, 0u};
    }
    float alpha_s, S, A;
    nvfp4_tensor(src, lds, rtab, alpha_s, S, A);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (S_out)
            *S_out = S;
        if (amax_out)
            *amax_out = A;
    }
    for (; u0 < nunits; u0 += nwaves * kLoads) {
        if (u0 != wave * kLoads) {
#pragma unroll
            for (int j = 0; j < kLoads; ++j) {
                const int64_t e = (u0 + j) * U + lane * E;
                v[j] = (u0 + j < nunits && e < n) ? ld16_stream(x + e) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            if (u0 + j >= nunits)
                break;
            const int64_t e = (u0 + j) * U + lane * E;
            float f[E];
            In<T>::unpack(v[j], f);
            const float a = max_lanes<LPB>(absmax<E>(f));
            uint32_t code;
            float r;
            nvfp4_block(a, alpha_s, rtab, code, r);
            if (e < n) {
                Fp4Store<E>::store(p + e / 2, f, r);
                if ((lane & (LPB - 1)) == 0)
                    codes[e / 16] = (uint8_t)code;
            }
        }
    }
}

// One 16-row strip of a 16x16 pass: lane E-column group at column c, loads
// v[16] already issued. Block amax over the lane pair, then codes and nibbles.
template <typename T>
__device__ __forceinline__ void strip_16x16(const u32x4* v, int64_t r0, int64_t c, int64_t C, float alpha_s,
                                            const float* rtab, uint8_t* __restrict__ p, uint8_t* __restrict__ codes)
{
    constexpr int E = In<T>::kE, LPB = 16 / E;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float f[E];
        In<T>::unpack(v[i], f);
        m = fmaxf(m, absmax<E>(f));
    }
    const float a = max_lanes<LPB>(m);
    uint32_t code;
    float r;
    nvfp4_block(a, alpha_s, rtab, code, r);
    if (c >= C)
        return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float f[E];
        In<T>::unpack(v[i], f);
        Fp4Store<E>::store(p + (r0 + i) * (C / 2) + c / 2, f, r);
    }
    if ((threadIdx.x & (LPB - 1)) == 0)
        codes[(r0 / 16) * (C / 16) + c / 16] = (uint8_t)code;
}

template <typename T>
__global__ __launch_bounds__(kWG) void k_nvfp4_16x16(const T* __restrict__ x, int64_t R, int64_t C, ScaleSrc src,
                                                     uint8_t* __restrict__ p, uint8_t* __restrict__ codes,
                                                     float* S_out, float* amax_out)
{
    __shared__ float lds[4];
    __shared__ float rtab[128];
    constexpr int E = In<T>::kE, WC = kWG * E;  // columns per workgroup
    const int64_t nwc = cdiv(C, WC), nstrips = (R / 16) * nwc;
    // one 16-row strip per workgroup (the grid is capped, so beyond 2^16
    // strips workgroups go on to further strips); the first strip's loads go
    // out before the tensor scale is resolved, so the partials' round trip
    // overlaps them
    int64_t t = blockIdx.x;
    int64_t r0 = (t / nwc) * 16, c = (t % nwc) * WC + (int64_t)threadIdx.x * E;
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = c < C ? ld16_stream(x + (r0 + i) * C + c) : u32x4{0u, 0u, 0u, 0u};
    float alpha_s, S, A;
    nvfp4_tensor(src, lds, rtab, alpha_s, S, A);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (S_out)
            *S_out = S;
        if (amax_out)
            *amax_out = A;
    }
    strip_16x16<T>(v, r0, c, C, alpha_s, rtab, p, codes);
    for (t += gridDim.x; t < nstrips; t += gridDim.x) {
        r0 = (t / nwc) * 16;
        c = (t % nwc) * WC + (int64_t)threadIdx.x * E;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = c < C ? ld16_stream(x + (r0 + i) * C + c) : u32x4{0u, 0u, 0u, 0u};
        strip_16x16<T>(v, r0, c, C, alpha_s, rtab, p, codes);
    }
}

// Colwise 1x16 copy (1x16 blocks of X^T = 16 rows of one column of X) in
// 128-row x 64-column tiles (workgroups stride over them), so each row of
// X^T gets 64 contiguous bytes per tile. Thread t: column c = t >> 2 of the tile and
// q = t & 3, which owns the blocks at rows 16q and 64 + 16q. The tile sits in
// LDS with its 16-byte chunks XOR-swizzled by the row's 16-row group, so the
// four rows 16 apart that a wave reads at each step hit distinct banks.
// Lane pairs (q even, q odd) swap one 8-byte half with DPP so each lane
// stores 16 contiguous bytes (blocks 2h, 2h+1 or 2h+4, 2h+5): a wave writes
// 16 whole 64-byte row segments per store instruction. Tiles that are not
// full, or rows of X^T that are only 8-byte aligned (R % 32 == 16), take
// 8-byte stores instead.
template <typename T, bool SR, bool RHT>
__global__ __launch_bounds__(kWG) void k_nvfp4_colt(const T* __restrict__ x, int64_t R, int64_t C, ScaleSrc src,
                                                    uint8_t* __restrict__ pt, uint8_t* __restrict__ ct,
                                                    float* S_out, float* amax_out, uint64_t seed, uint64_t offset,
                                                    uint32_t signs)
{
    constexpr int TC = 64, E = In<T>::kE, CPR = TC / E, SW = 16 / E;  // 16-byte chunks per row; swizzle step
    __shared__ float lds[4];
    __shared__ float rtab[128];
    __shared__ __align__(16) T tile[128][TC];
    const int64_t ntc = C / TC + (C % TC != 0), ntiles = ntc * cdiv(R, 128);
    float alpha_s, S, A;
    nvfp4_tensor(src, lds, rtab, alpha_s, S, A);  // includes a workgroup barrier
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (S_out)
            *S_out = S;
        if (amax_out)
            *amax_out = A;
    }
    const int c = threadIdx.x >> 2, q = threadIdx.x & 3;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * 128, c0 = tc * TC;
        const int64_t rows_in = min((int64_t)128, R - r0);
        __syncthreads();  // the previous tile's LDS reads are done
        // stage the tile: chunk j of row r goes to chunk j ^ (SW * ((r >> 4) & 3))
        for (int i = threadIdx.x; i < 128 * CPR; i += kWG) {
            const int r = i / CPR, j = i % CPR;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (r < rows_in && c0 + j * E < C)
                v = ld16_stream(x + (r0 + r) * C + c0 + j * E);
            *reinterpret_cast<u32x4*>(&tile[r][(j ^ (SW * ((r >> 4) & 3))) * E]) = v;
        }
        __syncthreads();
        const bool in = c0 + c < C;
        uint32_t wb[2][2];
        uint32_t codes[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int rb = 64 * half + 16 * q;  // first row of this block in the tile
            float f[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int r = rb + k;
                f[k] = In<T>::load1(&tile[r][0], ((c / E) ^ (SW * q)) * E + (c % E));
            }
            if constexpr (RHT)
                rht16(f, signs);
            uint32_t code;
            float rr;
            nvfp4_block(absmax<16>(f), alpha_s, rtab, code, rr);
            codes[half] = code;
            if constexpr (SR) {
                const uint64_t e0 = (uint64_t)((c0 + c) * R + r0 + rb), s = 2 * offset + 1;
                wb[half][0] = enc8_e2m1_sr(f, rr, sr_group(e0 / 8, s, seed));
                wb[half][1] = enc8_e2m1_sr(f + 8, rr, sr_group(e0 / 8 + 1, s, seed));
            } else {
                wb[half][0] = enc8_e2m1(f, rr);
                wb[half][1] = enc8_e2m1(f + 8, rr);
            }
        }
        uint8_t* rowp = pt + (c0 + c) * (R / 2) + r0 / 2;  // this column's row of X^T, from row r0
        const bool wide = rows_in == 128 && (R % 32) == 0;  // uniform over the workgroup
        if (wide) {
            // even q sends its second block, odd q its first; both then hold two adjacent blocks
            const bool odd = q & 1;
            const uint32_t s0 = odd ? wb[0][0] : wb[1][0], s1 = odd ? wb[0][1] : wb[1][1];
            const uint32_t r0w = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s0, kDppXor1, 0xF, 0xF, false);
            const uint32_t r1w = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s1, kDppXor1, 0xF, 0xF, false);
            u32x4 o;
            if (odd)
                o = u32x4{r0w, r1w, wb[1][0], wb[1][1]};  // blocks q + 3, q + 4 (= 2h + 4, 2h + 5)
            else
                o = u32x4{wb[0][0], wb[0][1], r0w, r1w};  // blocks q, q + 1
            if (in)
                st16_stream(rowp + (odd ? 32 + 8 * (q - 1) : 8 * q), o);
        } else if (in) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int rb = 64 * half + 16 * q;
                if (rb < rows_in) {
                    u32x2 v2;
                    v2[0] = wb[half][0];
                    v2[1] = wb[half][1];
                    st8_stream(rowp + rb / 2, v2);
                }
            }
        }
        if (in) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int rb = 64 * half + 16 * q;
                if (rb < rows_in)
                    ct[(c0 + c) * (R / 16) + (r0 + rb) / 16] = (uint8_t)codes[half];
            }
        }
    }
}

// The colwise copy of 1x16 blocks, with the rowwise copy from the same read
// (ROW), from bf16: a 128x128 tile per workgroup. Rowwise from registers as
// in k_nvfp4_1x16 (a block is the 16-byte chunks of a lane pair; a tile row
// leaves as 64 contiguous bytes of nibbles). The tile is staged in LDS with
// its 16-byte chunks XOR-swizzled by the row's 64-row half, and after one
// LDS-only barrier thread t takes column t >> 1 over rows 64g .. 64g + 63
// (g = t & 1): four 16x1 blocks, as k_nvfp4_colt encodes them (with its
// random Hadamard transform and stochastic rounding when asked), written as
// 32 contiguous bytes of X^T (the lane pair's pieces of a 64-byte segment
// meet in L2) and one 4-byte word of block codes. R % 128 == 0,
// C % 128 == 0. ROW only with round to nearest and no transform.
template <bool ROW, bool SR, bool RHT>
__global__ __launch_bounds__(kWG) void k_nvfp4_1x16_rowcol(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                           ScaleSrc src, uint8_t* __restrict__ p,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ pt,
                                                           uint8_t* __restrict__ ct, float* S_out, float* amax_out,
                                                           uint64_t seed, uint64_t offset, uint32_t signs)
{
    static_assert(!(ROW && (SR || RHT)), "the fused rowwise copy rounds to nearest, untransformed");
    constexpr int TC = 128, E = 8, CPR = TC / E, RPR = kWG / CPR, ROUNDS = 128 / RPR;
    __shared__ float lds[4];
    __shared__ float rtab[128];
    __shared__ __align__(16) uint16_t tile[128][TC];
    const int64_t ntc = C / TC;
    const int64_t r0 = (int64_t)(blockIdx.x / ntc) * 128, c0 = (int64_t)(blockIdx.x % ntc) * TC;
    const int j = threadIdx.x % CPR, rr0 = threadIdx.x / CPR;  // this lane's chunk of its rows; first row
    // the tile's loads go out before the tensor scale is resolved
    u32x4 v[ROUNDS];
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k)
        v[k] = ld16_stream(x + (r0 + rr0 + k * RPR) * C + c0 + j * E);
    float alpha_s, S, A;
    nvfp4_tensor(src, lds, rtab, alpha_s, S, A);  // includes a workgroup barrier
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (S_out)
            *S_out = S;
        if (amax_out)
            *amax_out = A;
    }
    // stage: chunk j of row r at chunk j ^ (4 * ((r >> 6) & 1))
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
        const int r = rr0 + k * RPR;
        *reinterpret_cast<u32x4*>(&tile[r][(j ^ (4 * ((r >> 6) & 1))) * E]) = v[k];
    }
    // rowwise: a 1x16 block is the chunk pair (j, j ^ 1)
    if constexpr (ROW) {
#pragma unroll
        for (int k = 0; k < ROUNDS; ++k) {
            const int64_t row = r0 + rr0 + k * RPR;
            float f[E];
            In<uint16_t>::unpack(v[k], f);
            const float a = max_lanes2(absmax<E>(f));
            uint32_t code;
            float r;
            nvfp4_block(a, alpha_s, rtab, code, r);
            Fp4Store<E>::store(p + row * (C / 2) + (c0 + j * E) / 2, f, r);
            if ((j & 1) == 0)
                codes[row * (C / 16) + (c0 + j * E) / 16] = (uint8_t)code;
        }
    }
    lds_barrier();
    // colwise: column c, rows 64g .. 64g + 63 (column c's place in them: its
    // chunk XOR 4g)
    const int c = threadIdx.x >> 1, g = threadIdx.x & 1;
    const int col = ((c / E) ^ (4 * g)) * E + (c % E);
    u32x4 w0, w1;
    uint32_t cw = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        float f[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            f[k] = In<uint16_t>::load1(&tile[64 * g + 16 * b + k][0], col);
        if constexpr (RHT)
            rht16(f, signs);
        uint32_t code;
        float r;
        nvfp4_block(absmax<16>(f), alpha_s, rtab, code, r);
        uint32_t lo, hi;
        if constexpr (SR) {
            // the block's first element in X^T (flat) and the colwise plane's stream
            const uint64_t e0 = (uint64_t)((c0 + c) * R + r0 + 64 * g + 16 * b), st = 2 * offset + 1;
            lo = enc8_e2m1_sr(f, r, sr_group(e0 / 8, st, seed));
            hi = enc8_e2m1_sr(f + 8, r, sr_group(e0 / 8 + 1, st, seed));
        } else {
            lo = enc8_e2m1(f, r);
            hi = enc8_e2m1(f + 8, r);
        }
        if (b < 2) {
            w0[2 * b] = lo;
            w0[2 * b + 1] = hi;
        } else {
            w1[2 * b - 4] = lo;
            w1[2 * b - 3] = hi;
        }
        cw |= code << (8 * b);
    }
    uint8_t* out = pt + (c0 + c) * (R / 2) + (r0 + 64 * g) / 2;  // 16-byte aligned: R % 128 == 0
    *reinterpret_cast<u32x4*>(out) = w0;
    *reinterpret_cast<u32x4*>(out + 16) = w1;
    *reinterpret_cast<uint32_t*>(ct + (c0 + c) * (R / 16) + (r0 + 64 * g) / 16) = cw;
}

// The colwise copy of 16x16 blocks and, with ROW, the rowwise copy from the
// same read (bf16): a 128x128 tile per workgroup, loaded as in
// k_nvfp4_1x16_rowcol (16 lanes per tile row, 16 rows per round), so round k
// covers block row k of the tile and the lane pair (j, j ^ 1) block column
// j >> 1. A block's max: the pair's, then the wave's four row groups (two
// lane shuffles), then the four waves (LDS); 64 threads turn the tile's 64
// block maxima into codes and multipliers, shared in LDS. The rowwise codes
// come from registers (the rowwise pass's packing), the colwise ones from
// the tile staged in LDS (two lanes per column, four blocks each, as in
// k_nvfp4_1x16_rowcol). R % 128 == 0, C % 128 == 0.
template <bool ROW>
__global__ __launch_bounds__(kWG) void k_nvfp4_16x16_tile(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                          ScaleSrc src, uint8_t* __restrict__ p,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ pt,
                                                          uint8_t* __restrict__ ct, float* S_out, float* amax_out)
{
    constexpr int TC = 128, E = 8, CPR = TC / E, RPR = kWG / CPR, ROUNDS = 128 / RPR, NBC = TC / 16;
    static_assert(RPR == 16, "a round is one 16-row block row");
    __shared__ float lds[4];
    __shared__ float rtab[128];
    __shared__ __align__(16) uint16_t tile[128][TC];
    __shared__ float wmax[4][ROUNDS][NBC];  // each wave's block maxima over its four rows of a round
    __shared__ float bmul[ROUNDS][NBC];     // the tile's block multipliers
    const int64_t ntc = C / TC;
    const int64_t r0 = (int64_t)(blockIdx.x / ntc) * 128, c0 = (int64_t)(blockIdx.x % ntc) * TC;
    const int j = threadIdx.x % CPR, rr0 = threadIdx.x / CPR;  // this lane's chunk of its rows; first row
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // the tile's loads go out before the tensor scale is resolved
    u32x4 v[ROUNDS];
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k)
        v[k] = ld16_stream(x + (r0 + rr0 + k * RPR) * C + c0 + j * E);
    float alpha_s, S, A;
    nvfp4_tensor(src, lds, rtab, alpha_s, S, A);  // includes a workgroup barrier
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (S_out)
            *S_out = S;
        if (amax_out)
            *amax_out = A;
    }
    // stage for the colwise pass: chunk j of row r at chunk j ^ (4 * ((r >> 6) & 1))
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
        const int r = rr0 + k * RPR;
        *reinterpret_cast<u32x4*>(&tile[r][(j ^ (4 * ((r >> 6) & 1))) * E]) = v[k];
    }
    // block maxima of block row k: the lane pair, the wave's four row groups
    // (lanes 16 and 32 apart), then the waves
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
        float f[E];
        In<uint16_t>::unpack(v[k], f);
        float m = max_lanes2(absmax<E>(f));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (lane < 16 && (j & 1) == 0)
            wmax[wv][k][j >> 1] = m;
    }
    lds_barrier();
    if (threadIdx.x < ROUNDS * NBC) {
        const int k = threadIdx.x / NBC, cb = threadIdx.x % NBC;
        const float a = fmaxf(fmaxf(wmax[0][k][cb], wmax[1][k][cb]), fmaxf(wmax[2][k][cb], wmax[3][k][cb]));
        uint32_t code;
        float r;
        nvfp4_block(a, alpha_s, rtab, code, r);
        bmul[k][cb] = r;
        const int64_t br = r0 / 16 + k, bc = c0 / 16 + cb;  // the block's row and column in the block grid
        if constexpr (ROW)
            codes[br * (C / 16) + bc] = (uint8_t)code;
        ct[bc * (R / 16) + br] = (uint8_t)code;
    }
    lds_barrier();
    if constexpr (ROW) {
#pragma unroll
        for (int k = 0; k < ROUNDS; ++k) {
            float f[E];
            In<uint16_t>::unpack(v[k], f);
            Fp4Store<E>::store(p + (r0 + rr0 + k * RPR) * (C / 2) + (c0 + j * E) / 2, f, bmul[k][j >> 1]);
        }
    }
    // colwise: column c, rows 64g .. 64g + 63 (block rows 4g .. 4g + 3)
    const int c = threadIdx.x >> 1, g = threadIdx.x & 1;
    const int col = ((c / E) ^ (4 * g)) * E + (c % E);
    u32x4 w0, w1;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        float f[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            f[k] = In<uint16_t>::load1(&tile[64 * g + 16 * b + k][0], col);
        const float r = bmul[4 * g + b][c >> 4];
        const uint32_t lo = enc8_e2m1(f, r), hi = enc8_e2m1(f + 8, r);
        if (b < 2) {
            w0[2 * b] = lo;
            w0[2 * b + 1] = hi;
        } else {
            w1[2 * b - 4] = lo;
            w1[2 * b - 3] = hi;
        }
    }
    uint8_t* out = pt + (c0 + c) * (R / 2) + (r0 + 64 * g) / 2;  // 16-byte aligned: R % 128 == 0
    *reinterpret_cast<u32x4*>(out) = w0;
    *reinterpret_cast<u32x4*>(out + 16) = w1;
}

// Colwise copy of 16x16 blocks (BR = 16; the 1x16 copy is k_nvfp4_colt):
// the same blocks as rowwise, so the colwise nibbles are the rowwise ones
// transposed. Slab of 32 rows x 256 columns in LDS.
//
// ROW (BR = 16): the rowwise copy too, from the same read. The staged chunks
// stay in registers; each block's multiplier goes to LDS once its column
// pass has it, and after one more barrier every lane encodes its chunks
// rowwise (the rowwise pass's packing, Fp4Store) and writes the block codes
// of both planes.
template <typename T, int BR, bool ROW = false>
__global__ __launch_bounds__(kWG) void k_nvfp4_col(const T* __restrict__ x, int64_t R, int64_t C, ScaleSrc src,
                                                   uint8_t* __restrict__ pt, uint8_t* __restrict__ ct,
                                                   float* S_out, float* amax_out, uint8_t* __restrict__ p = nullptr,
                                                   uint8_t* __restrict__ codes = nullptr)
{
    static_assert(!ROW || BR == 16, "the rowwise copy from the colwise pass needs 16x16 blocks");
    __shared__ float lds[4];
    __shared__ float rtab[128];
    constexpr int TC = 256, E = In<T>::kE, LPR = TC / E, RPR = kWG / LPR, NR = 32 / RPR;
    __shared__ __align__(16) T tile[32][TC];
    __shared__ float rblk[2][TC / 16];  // ROW: the multiplier of each block of the slab
    float alpha_s, S, A;
    nvfp4_tensor(src, lds, rtab, alpha_s, S, A);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (S_out)
            *S_out = S;
        if (amax_out)
            *amax_out = A;
    }
    const int64_t ntc = cdiv(C, TC), nslabs = cdiv(R, 32) * ntc;
    const int cc = (threadIdx.x % LPR) * E;
    // workgroups stride over the 32 x 256 slabs (the grid is capped); every
    // thread runs every iteration, so the barriers below are uniform
    for (int64_t t = blockIdx.x; t < nslabs; t += gridDim.x) {
        const int64_t r0 = (t / ntc) * 32, c0 = (t % ntc) * TC;
        __syncthreads();  // the previous slab's LDS reads are done
        u32x4 v[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int rr = threadIdx.x / LPR + k * RPR;
            v[k] = u32x4{0u, 0u, 0u, 0u};
            if (c0 + cc < C && r0 + rr < R)
                v[k] = ld16_stream(x + (r0 + rr) * C + c0 + cc);
            *reinterpret_cast<u32x4*>(&tile[rr][cc]) = v[k];
        }
        __syncthreads();
        const int c = threadIdx.x;
        const bool in = c0 + c < C;
        const int nb = (r0 + 32 <= R) ? 2 : 1;  // R % 16 == 0
        uint32_t w[4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float f[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                f[k] = In<T>::load1(&tile[0][0], (int64_t)(16 * b + k) * TC + c);
            float a = absmax<16>(f);
            if constexpr (BR == 16)
                a = max_lanes<16>(a);
            uint32_t code;
            float r;
            nvfp4_block(a, alpha_s, rtab, code, r);
            w[2 * b] = enc8_e2m1(f, r);
            w[2 * b + 1] = enc8_e2m1(f + 8, r);
            if constexpr (ROW) {
                if ((c & 15) == 0)
                    rblk[b][c / 16] = r;
            }
            if (in && b < nb) {
                const int64_t rb = (r0 + 16 * b) / 16;
                if constexpr (BR == 1) {
                    ct[(c0 + c) * (R / 16) + rb] = (uint8_t)code;
                } else if ((c & 15) == 0) {
                    ct[((c0 + c) / 16) * (R / 16) + rb] = (uint8_t)code;
                    if constexpr (ROW)
                        codes[rb * (C / 16) + (c0 + c) / 16] = (uint8_t)code;
                }
            }
        }
        if (in) {
            // row c of the colwise plane is only 8-byte aligned (R/2 is a
            // multiple of 8). A thread writes 8 or 16 bytes of a row: ordinary
            // stores, so the pieces of a line meet in L2 before going to memory
            // (streaming stores of such pieces each become a partial-line write,
            // measured 3x slower).
            uint8_t* out = pt + (c0 + c) * (R / 2) + r0 / 2;
            u32x2 v2;
            v2[0] = w[0];
            v2[1] = w[1];
            *reinterpret_cast<u32x2*>(out) = v2;
            if (nb == 2) {
                v2[0] = w[2];
                v2[1] = w[3];
                *reinterpret_cast<u32x2*>(out + 8) = v2;
            }
        }
        if constexpr (ROW) {
            lds_barrier();  // the slab's block multipliers are in rblk
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                const int rr = threadIdx.x / LPR + k * RPR;
                if (c0 + cc < C && r0 + rr < R) {
                    float f[E];
                    In<T>::unpack(v[k], f);
                    Fp4Store<E>::store(p + (r0 + rr) * (C / 2) + (c0 + cc) / 2, f, rblk[rr / 16][cc / 16]);
                }
            }
        }
    }
}

template <typename T>
void launch_t(const void* xv, int64_t R, int64_t C, int br, ScaleSrc src, uint8_t* p, uint8_t* codes, uint8_t* pt,
              uint8_t* codest, float* S_out, float* amax_out, SrArgs sr, RhtArgs rht, hipStream_t stream)
{
    const T* x = (const T*)xv;
    constexpr int E = In<T>::kE;
    if constexpr (std::is_same<T, uint16_t>::value) {
        if (pt && br == 1 && R > 0 && C > 0 && R % 128 == 0 && C % 128 == 0) {
            // the colwise 1x16 copy in 128x128 tiles, with the rowwise one
            // from the same read when both are asked for (a transform is
            // never asked with a rowwise plane)
            const unsigned grid = (unsigned)((R / 128) * (C / 128));
            const uint64_t sd = sr.seed, of = sr.offset;
            const uint32_t sg = rht.signs;
            if (p && !sr.on) {
                k_nvfp4_1x16_rowcol<true, false, false><<<grid, kWG, 0, stream>>>(x, R, C, src, p, codes, pt, codest,
                                                                                 S_out, amax_out, sd, of, sg);
                return;
            }
            float* s2 = S_out;
            float* a2 = amax_out;
            if (p) {
                // stochastic rounding on both planes: the rowwise pass first
                const int64_t nblk = R * C / 16;
                const int g1 = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(nblk, kWG), kMaxGrid1x16));
                k_nvfp4_1x16_sr<T><<<g1, kWG, 0, stream>>>(x, nblk, src, sd, of, p, codes, S_out, amax_out);
                s2 = nullptr;
                a2 = nullptr;
            }
            if (rht.on && sr.on)
                k_nvfp4_1x16_rowcol<false, true, true><<<grid, kWG, 0, stream>>>(x, R, C, src, p, codes, pt, codest,
                                                                                s2, a2, sd, of, sg);
            else if (rht.on)
                k_nvfp4_1x16_rowcol<false, false, true><<<grid, kWG, 0, stream>>>(x, R, C, src, p, codes, pt, codest,
                                                                                 s2, a2, sd, of, sg);
            else if (sr.on)
                k_nvfp4_1x16_rowcol<false, true, false><<<grid, kWG, 0, stream>>>(x, R, C, src, p, codes, pt, codest,
                                                                                 s2, a2, sd, of, sg);
            else
                k_nvfp4_1x16_rowcol<false, false, false><<<grid, kWG, 0, stream>>>(x, R, C, src, p, codes, pt,
                                                                                  codest, s2, a2, sd, of, sg);
            return;
        }
    }
    if constexpr (std::is_same<T, uint16_t>::value) {
        if (pt && br == 16 && R > 0 && C > 0 && R % 128 == 0 && C % 128 == 0) {
            // the colwise copy of 16x16 blocks in 128x128 tiles, and the
            // rowwise one from the same read when both are asked for
            const unsigned grid = (unsigned)((R / 128) * (C / 128));
            if (p)
                k_nvfp4_16x16_tile<true><<<grid, kWG, 0, stream>>>(x, R, C, src, p, codes, pt, codest, S_out, amax_out);
            else
                k_nvfp4_16x16_tile<false><<<grid, kWG, 0, stream>>>(x, R, C, src, p, codes, pt, codest, S_out,
                                                                     amax_out);
            return;
        }
    }
    if (p && pt && br == 16 && R > 0 && C > 0) {
        // both planes of 16x16 blocks from one read
        const int64_t grid = std::min<int64_t>(cdiv(R, 32) * cdiv(C, 256), kMaxSlabGrid);
        k_nvfp4_col<T, 16, true><<<(unsigned)grid, kWG, 0, stream>>>(x, R, C, src, pt, codest, S_out, amax_out, p,
                                                                      codes);
        return;
    }
    bool wrote_scalars = false;
    if (p) {
        if (sr.on) {
            const int64_t nblk = R * C / 16;
            const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(nblk, kWG), kMaxGrid1x16));
            k_nvfp4_1x16_sr<T><<<grid, kWG, 0, stream>>>(x, nblk, src, sr.seed, sr.offset, p, codes, S_out,
                                                         amax_out);
            wrote_scalars = true;
        } else if (br == 1) {
            const int64_t n = R * C;
            const int64_t per_wg = (int64_t)kWG * E * kLoads;
            const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, per_wg), kMaxGrid1x16));
            k_nvfp4_1x16<T><<<grid, kWG, 0, stream>>>(x, n, src, p, codes, S_out, amax_out);
            wrote_scalars = true;
        } else if (R > 0 && C > 0) {
            const int64_t grid = std::min<int64_t>((R / 16) * cdiv(C, (int64_t)kWG * E), kMaxSlabGrid);
            k_nvfp4_16x16<T><<<(unsigned)grid, kWG, 0, stream>>>(x, R, C, src, p, codes, S_out, amax_out);
            wrote_scalars = true;
        }
    }
    if (pt && R > 0 && C > 0) {
        float* s2 = wrote_scalars ? nullptr : S_out;
        float* a2 = wrote_scalars ? nullptr : amax_out;
        if (br == 1) {
            const unsigned g1 = (unsigned)std::min<int64_t>(cdiv(R, 128) * cdiv(C, 64), kMaxGridColt);
            const uint64_t sd = sr.seed, of = sr.offset;
            const uint32_t sg = rht.signs;
            if (rht.on && sr.on)
                k_nvfp4_colt<T, true, true><<<g1, kWG, 0, stream>>>(x, R, C, src, pt, codest, s2, a2, sd, of, sg);
            else if (rht.on)
                k_nvfp4_colt<T, false, true><<<g1, kWG, 0, stream>>>(x, R, C, src, pt, codest, s2, a2, sd, of, sg);
            else if (sr.on)
                k_nvfp4_colt<T, true, false><<<g1, kWG, 0, stream>>>(x, R, C, src, pt, codest, s2, a2, sd, of, sg);
            else
                k_nvfp4_colt<T, false, false><<<g1, kWG, 0, stream>>>(x, R, C, src, pt, codest, s2, a2, sd, of, sg);
        } else {
            const int64_t grid = std::min<int64_t>(cdiv(R, 32) * cdiv(C, 256), kMaxSlabGrid);
            k_nvfp4_col<T, 16><<<(unsigned)grid, kWG, 0, stream>>>(x, R, C, src, pt, codest, s2, a2);
        }
        wrote_scalars = true;
    }
    if (!wrote_scalars) {
        // empty tensor: only the tensor scale and amax
        k_nvfp4_1x16<T><<<1, kWG, 0, stream>>>(x, 0, src, p, codes, S_out, amax_out);
    }
}

}  // namespace

hipError_t launch_nvfp4(const void* x, int in_bf16, int64_t R, int64_t C, int br, ScaleSrc src, uint8_t* p,
                        uint8_t* codes, uint8_t* pt, uint8_t* codest, float* S_out, float* amax_out, SrArgs sr,
                        RhtArgs rht, hipStream_t stream)
{
    if (in_bf16)
        launch_t<uint16_t>(x, R, C, br, src, p, codes, pt, codest, S_out, amax_out, sr, rht, stream);
    else
        launch_t<float>(x, R, C, br, src, p, codes, pt, codest, S_out, amax_out, sr, rht, stream);
    return hipGetLastError();
}

int rht_amax_grid(int64_t R, int64_t C)
{
    const int64_t nstrips = (R / 16) * cdiv(C, (int64_t)kWG * 4);  // upper bound over input types
    return (int)std::max<int64_t>(1, std::min<int64_t>(nstrips, kMaxPartials));
}

hipError_t launch_rht_amax_partial(const void* x, int in_bf16, int64_t R, int64_t C, uint32_t signs,
                                   float* partials, int grid, hipStream_t stream)
{
    if (in_bf16)
        k_rht_amax_partial<uint16_t><<<grid, kWG, 0, stream>>>((const uint16_t*)x, R, C, signs, partials);
    else
        k_rht_amax_partial<float><<<grid, kWG, 0, stream>>>((const float*)x, R, C, signs, partials);
    return hipGetLastError();
}

}  // namespace fq
