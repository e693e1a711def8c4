// k_tensor.hip -- per-tensor scaling kernels: the grid-wide amax, the
// scale+cast pass, the fused delayed-scaling cast and its finish.
//
// Sources: [MP] "混合精度训练：fp16 到 fp8" (garden.houmin.site), section
// "FP8 recipe" items 2 (delayed) and 3 (current); [CS] "FP8 Current
// Scaling：量化、缩放与精度边界" (notes.kuangjux.top), sections "Current
// Scaling" (a, alpha, q, s) and "成本与多 GPU 使用" (two reads of the tensor).
//
// Layout of the work: a flat tensor of n elements is cut into wave units of
// 64 lanes x 16 bytes (512 bf16 or 256 fp32 elements, 1 KiB). Each wave takes
// kLoads consecutive units per step, so every lane has kLoads 16-byte loads
// in flight and each load instruction of the wave reads 1 KiB contiguously.
// Workgroups stride over the units; fewer than one unit of ragged tail is
// handled one element per thread.
//
// Current scaling is two passes: k_amax_partial writes one exact max per
// workgroup (lane max -> DPP within 16 lanes -> shuffles across the wave ->
// LDS across 4 waves), and every workgroup of the cast pass re-reduces those
// few KiB of partials itself (they stay in L2), so no atomics and no third
// kernel are needed and the result does not depend on scheduling order.
//
// Delayed scaling is one pass per step: the cast uses the scale the window
// gave after the previous step and writes this step's amax partials into a
// record in the caller's state. The window update of step t-1 (record its
// amax, new scale from the window's max) is folded into step t's cast: every
// workgroup re-reduces step t-1's record and the window from L2 to get the
// scale it casts with, and workgroup 0 alone writes the window slot and the
// new scale back. So a step is one kernel, with no separate finish launch.
#include <algorithm>

#include "codec.hpp"
#include "launch.hpp"

namespace fq {
namespace {

constexpr int kLoads = 4;
constexpr int kCastMaxGrid = 16384;

template <typename T, int L>
__global__ __launch_bounds__(kWG) void k_amax_partial(const T* __restrict__ x, int64_t n,
                                                      float* __restrict__ partials)
{
    __shared__ float lds[4];
    constexpr int E = In<T>::kE, U = 64 * E;
    const int lane = threadIdx.x & 63;
    const int64_t nunits = n / U;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    float m = 0.0f;
    for (int64_t u0 = wave * L; u0 < nunits; u0 += nwaves * L) {
        u32x4 v[L];
#pragma unroll
        for (int j = 0; j < L; ++j)
            v[j] = (u0 + j < nunits) ? ld16(x + (u0 + j) * U + lane * E) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < L; ++j)
            m = fmaxf(m, In<T>::absmax16(v[j]));
    }
    for (int64_t i = nunits * U + (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG)
        m = fmaxf(m, fabsf(In<T>::load1(x, i)));
    m = max_workgroup(m, lds);
    if (threadIdx.x == 0)
        partials[blockIdx.x] = m;
}

// alpha and s for this launch, from the scale source. Uniform control flow.
template <int FMT>
__device__ __forceinline__ void resolve_scale(const ScaleSrc& src, float* lds, float& alpha, float& s, float& a)
{
    if (src.amax_in) {
        a = *src.amax_in;
    } else {
        const float m = partials_max(src.partials, src.n_partials);
        a = max_workgroup(m, lds);
    }
    tensor_scales(a, Fmt<FMT>::kMax, alpha, s);
}

// Delayed scaling, start of step t: finish step t-1 from its record (if
// dl.prev and the record carries step t-1's tag), giving the scale this
// step casts with; otherwise cast with the state's scale. Every workgroup
// computes the same values; workgroup 0 writes them back (window slot, new
// alpha and s, the s used). All loads (record, tag, window, state scale)
// are issued together: one memory latency. `lds` holds 8 floats. Uniform
// control flow (contains __syncthreads).
__device__ __forceinline__ void delayed_prologue(const DelayedArgs& dl, float* lds, float& alpha, float& s)
{
    const float a0 = *dl.alpha, s0 = *dl.s;
    float mp = 0.0f, mh = 0.0f;
    bool apply = false;
    if (dl.prev) {
        const uint32_t* tag = reinterpret_cast<const uint32_t*>(dl.prev + kMaxPartials);
        const uint32_t t0 = tag[0], t1 = tag[1];
        float h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = (int)threadIdx.x + k * kWG;
            h[k] = (i < dl.H && i != dl.prev_slot) ? dl.hist[i] : 0.0f;
        }
        mp = partials_max(dl.prev, kMaxPartials);
        mh = fmaxf(fmaxf(h[0], h[1]), fmaxf(h[2], h[3]));
        apply = t0 == dl.prev_tag[0] && t1 == dl.prev_tag[1];
    }
    mp = max_wave(mp);
    mh = max_wave(mh);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        lds[w] = mp;
        lds[4 + w] = mh;
    }
    __syncthreads();
    const float a_prev = fmaxf(fmaxf(lds[0], lds[1]), fmaxf(lds[2], lds[3]));
    const float m = fmaxf(fmaxf(fmaxf(lds[4], lds[5]), fmaxf(lds[6], lds[7])), a_prev);
    if (apply && m > 0.0f) {
        tensor_scales(m, dl.fmax, alpha, s);
    } else {
        alpha = a0;
        s = s0;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (apply) {
            dl.hist[dl.prev_slot] = a_prev;
            if (m > 0.0f) {
                *dl.alpha = alpha;
                *dl.s = s;
            }
        }
        if (dl.s_used)
            *dl.s_used = s;
    }
}

// Delayed scaling, end of step t: this workgroup's amax into the step's
// record; workgroup 0 also zeroes the slots beyond the grid and writes the
// tag. Uniform control flow.
__device__ __forceinline__ void delayed_epilogue(const DelayedArgs& dl, float m, float* lds)
{
    m = max_workgroup(m, lds);
    if (threadIdx.x == 0)
        dl.rec[blockIdx.x] = m;
    if (blockIdx.x == 0) {
        for (int i = (int)gridDim.x + (int)threadIdx.x; i < kMaxPartials; i += kWG)
            dl.rec[i] = 0.0f;
        if (threadIdx.x == 0) {
            uint32_t* tag = reinterpret_cast<uint32_t*>(dl.rec + kMaxPartials);
            tag[0] = dl.tag[0];
            tag[1] = dl.tag[1];
        }
    }
}

// q = Q(fp32(alpha * x)) over a flat tensor, current scaling.
template <typename T, int FMT, int L>
__global__ __launch_bounds__(kWG) void k_cast_tensor(const T* __restrict__ x, int64_t n, ScaleSrc src,
                                                     uint8_t* __restrict__ q, float* s_out, float* amax_out)
{
    __shared__ float lds[4];
    constexpr int E = In<T>::kE, U = 64 * E;
    const int lane = threadIdx.x & 63;
    const int64_t nunits = n / U;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    // the first step's loads go out before the scale is resolved, so the
    // partials' round trip overlaps them
    u32x4 v[L];
    int64_t u0 = wave * L;
#pragma unroll
    for (int j = 0; j < L; ++j)
        v[j] = (u0 + j < nunits) ? ld16_stream(x + (u0 + j) * U + lane * E) : u32x4{0u, 0u, 0u, 0u};
    float alpha, s, a;
    resolve_scale<FMT>(src, lds, alpha, s, a);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (s_out)
            *s_out = s;
        if (amax_out)
            *amax_out = a;
    }
    for (; u0 < nunits; u0 += nwaves * L) {
        if (u0 != wave * L) {
#pragma unroll
            for (int j = 0; j < L; ++j)
                v[j] = (u0 + j < nunits) ? ld16_stream(x + (u0 + j) * U + lane * E) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (u0 + j < nunits) {
                float f[E];
                In<T>::unpack(v[j], f);
                Enc8<FMT, E>::store(q + (u0 + j) * U + lane * E, f, alpha);
            }
        }
    }
    for (int64_t i = nunits * U + (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG)
        q[i] = enc1<FMT>(In<T>::load1(x, i), alpha);
}

// One delayed-scaling step over a flat tensor: finish step t-1 (prologue),
// q = Q(fp32(alpha * x)) and the amax in the same read, this step's record
// (epilogue). The first loads go out before the prologue's loads, so its
// round trip overlaps them, and each step's loads go out before the step
// before it is converted.
template <typename T, int FMT, int L>
__global__ __launch_bounds__(kWG) void k_cast_delayed(const T* __restrict__ x, int64_t n, DelayedArgs dl,
                                                      uint8_t* __restrict__ q)
{
    __shared__ float lds[8];
    constexpr int E = In<T>::kE, U = 64 * E;
    const int lane = threadIdx.x & 63;
    const int64_t nunits = n / U;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    u32x4 v[L];
    int64_t u0 = wave * L;
#pragma unroll
    for (int j = 0; j < L; ++j)
        v[j] = (u0 + j < nunits) ? ld16_stream(x + (u0 + j) * U + lane * E) : u32x4{0u, 0u, 0u, 0u};
    float alpha, s;
    delayed_prologue(dl, lds, alpha, s);
    float m = 0.0f;
    for (; u0 < nunits; u0 += nwaves * L) {
        const int64_t un = u0 + nwaves * L;
        u32x4 nx[L];
        if (un < nunits) {
#pragma unroll
            for (int j = 0; j < L; ++j)
                nx[j] = (un + j < nunits) ? ld16_stream(x + (un + j) * U + lane * E) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (u0 + j < nunits) {
                float f[E];
                In<T>::unpack(v[j], f);
                m = fmaxf(m, absmax<E>(f));
                Enc8<FMT, E>::store(q + (u0 + j) * U + lane * E, f, alpha);
            }
        }
        if (un < nunits) {
#pragma unroll
            for (int j = 0; j < L; ++j)
                v[j] = nx[j];
        }
    }
    for (int64_t i = nunits * U + (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) {
        const float v1 = In<T>::load1(x, i);
        m = fmaxf(m, fabsf(v1));
        q[i] = enc1<FMT>(v1, alpha);
    }
    delayed_epilogue(dl, m, lds);
}

// The scale of a per-tensor tile cast: current scaling from src (writing s
// and the amax), or a delayed step's prologue. Uniform control flow.
template <int FMT, bool DELAYED>
__device__ __forceinline__ void tile_cast_scale(const ScaleSrc& src, const DelayedArgs& dl, float* lds,
                                                float* s_out, float* amax_out, float& alpha)
{
    float s;
    if constexpr (DELAYED) {
        delayed_prologue(dl, lds, alpha, s);
    } else {
        float a;
        resolve_scale<FMT>(src, lds, alpha, s, a);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            if (s_out)
                *s_out = s;
            if (amax_out)
                *amax_out = a;
        }
    }
}

// Per-tensor cast through 64x64 tiles, for the transposed (colwise) copy:
// rowwise bytes q[r*C + c] and transposed bytes qt[c*R + r] from one read.
// Byte-granular and bounds-checked: any shape. Current scaling, or one
// delayed-scaling step (then one amax partial per workgroup into the step's
// record).
template <typename T, int FMT, bool DELAYED>
__global__ __launch_bounds__(kWG) void k_cast_tensor_2d(const T* __restrict__ x, int64_t R, int64_t C,
                                                        ScaleSrc src, DelayedArgs dl, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ qt, float* s_out, float* amax_out)
{
    __shared__ float lds[8];
    __shared__ uint8_t tile[64][68];
    float alpha;
    tile_cast_scale<FMT, DELAYED>(src, dl, lds, s_out, amax_out, alpha);
    const int64_t tcols = (C + 63) / 64, ntiles = ((R + 63) / 64) * tcols;
    float m = 0.0f;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        int64_t tr, tc;
        tile_coords(t, tcols, tr, tc);
        const int64_t r0 = tr * 64, c0 = tc * 64;
        __syncthreads();
        for (int i = threadIdx.x; i < 64 * 64; i += kWG) {
            const int r = i >> 6, c = i & 63;
            const int64_t gr = r0 + r, gc = c0 + c;
            uint8_t code = 0;
            if (gr < R && gc < C) {
                const float v = In<T>::load1(x, gr * C + gc);
                m = fmaxf(m, fabsf(v));
                code = enc1<FMT>(v, alpha);
                if (q)
                    q[gr * C + gc] = code;
            }
            tile[r][c] = code;
        }
        __syncthreads();
        if (qt) {
            for (int i = threadIdx.x; i < 64 * 64; i += kWG) {
                const int c = i >> 6, r = i & 63;
                const int64_t gr = r0 + r, gc = c0 + c;
                if (gr < R && gc < C)
                    qt[gc * R + gr] = tile[r][c];
            }
        }
    }
    if constexpr (DELAYED)
        delayed_epilogue(dl, m, lds);
}

// Per-tensor cast with the colwise copy, for R % 16 == 0 and C % 16 == 0:
// 128x128 tiles, workgroups striding over tiles; 16-byte loads, rowwise
// codes stored from registers, and the transposed codes through an LDS tile
// XOR-swizzled in 8-byte units by 16-row group, written with eight lanes per
// 128-byte row of X^T (edge tiles: rows of X^T of rows_in bytes). Current
// scaling, or one delayed-scaling step (then one amax partial per workgroup
// into the step's record).
__device__ __forceinline__ int tile_swizzle(int r) { return 8 * ((r >> 4) & 7); }

template <typename T, int FMT, bool DELAYED>
__global__ __launch_bounds__(kWG) void k_cast_tensor_tile(const T* __restrict__ x, int64_t R, int64_t C,
                                                          ScaleSrc src, DelayedArgs dl, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ qt, float* s_out, float* amax_out)
{
    constexpr int E = In<T>::kE, LPR = 128 / E, RPR = kWG / LPR, ROUNDS = 128 / RPR;
    __shared__ float lds[8];
    __shared__ __align__(16) uint8_t codes[128][128 + 16];
    float alpha;
    tile_cast_scale<FMT, DELAYED>(src, dl, lds, s_out, amax_out, alpha);
    const int64_t ntc = cdiv(C, 128), ntiles = cdiv(R, 128) * ntc;
    const int cc = (threadIdx.x % LPR) * E, rr0 = threadIdx.x / LPR;
    float m = 0.0f;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        int64_t tr, tc;
        tile_coords(t, ntc, tr, tc);
        const int64_t r0 = tr * 128, c0 = tc * 128;
        const int rows_in = (int)min((int64_t)128, R - r0), cols_in = (int)min((int64_t)128, C - c0);
        __syncthreads();  // the previous tile's LDS reads are done
        u32x4 v[ROUNDS];
#pragma unroll
        for (int k = 0; k < ROUNDS; ++k) {
            const int rr = rr0 + k * RPR;
            v[k] = (rr < rows_in && cc < cols_in) ? ld16_stream(x + (r0 + rr) * C + c0 + cc) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < ROUNDS; ++k) {
            const int rr = rr0 + k * RPR;
            float f[E];
            In<T>::unpack(v[k], f);
            if constexpr (DELAYED)
                m = fmaxf(m, absmax<E>(f));
            const bool in = rr < rows_in && cc < cols_in;
            if constexpr (E == 8) {
                u32x2 w;
                w[0] = enc4<FMT>(f[0], f[1], f[2], f[3], alpha);
                w[1] = enc4<FMT>(f[4], f[5], f[6], f[7], alpha);
                if (q && in)
                    st8_stream(q + (r0 + rr) * C + c0 + cc, w);
                if (qt)
                    *reinterpret_cast<u32x2*>(&codes[rr][cc ^ tile_swizzle(rr)]) = w;
            } else {
                const uint32_t w = enc4<FMT>(f[0], f[1], f[2], f[3], alpha);
                if (q && in)
                    st4_stream(q + (r0 + rr) * C + c0 + cc, w);
                if (qt)
                    *reinterpret_cast<uint32_t*>(&codes[rr][cc ^ tile_swizzle(rr)]) = w;
            }
        }
        if (!qt)
            continue;
        __syncthreads();
        const int kq = threadIdx.x & 7;
        for (int c = threadIdx.x >> 3; c < cols_in; c += kWG / 8) {
            u32x4 w;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t word = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int r = 16 * kq + 4 * d + b;
                    word |= (uint32_t)codes[r][c ^ tile_swizzle(r)] << (8 * b);
                }
                w[d] = word;
            }
            if (16 * kq < rows_in)
                st16_stream(qt + (c0 + c) * R + r0 + 16 * kq, w);
        }
    }
    if constexpr (DELAYED)
        delayed_epilogue(dl, m, lds);
}

__global__ __launch_bounds__(kWG) void k_amax_finish(const float* __restrict__ partials, int n, float* out)
{
    __shared__ float lds[4];
    float m = 0.0f;
    for (int i = threadIdx.x; i < n; i += kWG)
        m = fmaxf(m, partials[i]);
    m = max_workgroup(m, lds);
    if (threadIdx.x == 0)
        *out = m;
}

// Delayed scaling, the window update of one step on its own ([MP] recipe 2:
// record the step's amax in the window; the next scale comes from the
// window's max), for windows longer than the cast's prologue reads and for
// fq_delayed_flush. One workgroup reads the record (partials and tag) and
// the window together; nothing changes unless the record carries `tag`.
constexpr int kFinishThreads = 256;

__global__ __launch_bounds__(kFinishThreads) void k_delayed_finish(const float* __restrict__ rec, uint32_t tag_lo,
                                                                   uint32_t tag_hi, float* hist, int H, int slot,
                                                                   float* alpha, float* s, float fmax_v,
                                                                   float* amax_out)
{
    __shared__ float lds[2][kFinishThreads / 64];
    static_assert(kFinishThreads == kWG, "partials_max assumes kWG threads");
    const uint32_t* tag = reinterpret_cast<const uint32_t*>(rec + kMaxPartials);
    const bool apply = tag[0] == tag_lo && tag[1] == tag_hi;
    float mp = partials_max(rec, kMaxPartials), mh = 0.0f;
#pragma unroll 4
    for (int i = threadIdx.x; i < H; i += kFinishThreads)
        if (i != slot)
            mh = fmaxf(mh, hist[i]);
    mp = max_wave(mp);
    mh = max_wave(mh);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        lds[0][w] = mp;
        lds[1][w] = mh;
    }
    __syncthreads();
    if (threadIdx.x == 0 && apply) {
        float at = 0.0f, wm = 0.0f;
        for (int k = 0; k < kFinishThreads / 64; ++k) {
            at = fmaxf(at, lds[0][k]);
            wm = fmaxf(wm, lds[1][k]);
        }
        wm = fmaxf(wm, at);
        hist[slot] = at;
        if (amax_out)
            *amax_out = at;
        if (wm > 0.0f) {
            float al, ss;
            tensor_scales(wm, fmax_v, al, ss);
            *alpha = al;
            *s = ss;
        }
    }
}

template <typename T>
int64_t elems_per_wg_step()
{
    return (int64_t)kWG * (16 / (int)sizeof(T)) * kLoads;
}

}  // namespace

int amax_grid(int64_t n, int elem_bytes, int max_grid)
{
    const int64_t per = (int64_t)kWG * (16 / elem_bytes) * kLoads;
    return (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, per), max_grid));
}

hipError_t launch_amax_partial(const void* x, int in_bf16, int64_t n, float* partials, int grid, hipStream_t stream,
                               int depth)
{
    if (in_bf16 && depth == 8)
        k_amax_partial<uint16_t, 8><<<grid, kWG, 0, stream>>>((const uint16_t*)x, n, partials);
    else if (in_bf16)
        k_amax_partial<uint16_t, kLoads><<<grid, kWG, 0, stream>>>((const uint16_t*)x, n, partials);
    else if (depth == 8)
        k_amax_partial<float, 8><<<grid, kWG, 0, stream>>>((const float*)x, n, partials);
    else
        k_amax_partial<float, kLoads><<<grid, kWG, 0, stream>>>((const float*)x, n, partials);
    return hipGetLastError();
}

hipError_t launch_amax_finish(const float* partials, int n, float* out, hipStream_t stream)
{
    k_amax_finish<<<1, kWG, 0, stream>>>(partials, n, out);
    return hipGetLastError();
}

template <typename T, int FMT>
static void cast_tensor_t(const void* x, int64_t n, ScaleSrc src, uint8_t* q, float* s_out, float* amax_out,
                          int grid, hipStream_t stream)
{
    // eight loads per lane in flight (measured faster inside a full step)
    k_cast_tensor<T, FMT, 8><<<grid, kWG, 0, stream>>>((const T*)x, n, src, q, s_out, amax_out);
}

hipError_t launch_cast_tensor(const void* x, int in_bf16, int fmt, int64_t n, ScaleSrc src, uint8_t* q,
                              float* s_out, float* amax_out, hipStream_t stream)
{
    // a workgroup step covers 8 loads per lane
    const int64_t per = (in_bf16 ? elems_per_wg_step<uint16_t>() : elems_per_wg_step<float>()) * (8 / kLoads);
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, per), kCastMaxGrid));
    if (in_bf16) {
        if (fmt == kE4M3)
            cast_tensor_t<uint16_t, kE4M3>(x, n, src, q, s_out, amax_out, grid, stream);
        else
            cast_tensor_t<uint16_t, kE5M2>(x, n, src, q, s_out, amax_out, grid, stream);
    } else {
        if (fmt == kE4M3)
            cast_tensor_t<float, kE4M3>(x, n, src, q, s_out, amax_out, grid, stream);
        else
            cast_tensor_t<float, kE5M2>(x, n, src, q, s_out, amax_out, grid, stream);
    }
    return hipGetLastError();
}

// Tile casts (colwise copy): vector 128x128 tiles when R and C are multiples
// of 16, else byte-granular 64x64 tiles. A delayed step's grid is at most
// kMaxPartials (one partial per workgroup).
template <typename T, int FMT, bool DELAYED>
static void cast_2d_t(const void* x, int64_t R, int64_t C, ScaleSrc src, const DelayedArgs& dl, uint8_t* q,
                      uint8_t* qt, float* s_out, float* amax_out, hipStream_t stream)
{
    const int max_grid = DELAYED ? kMaxPartials : kCastMaxGrid;
    if (R % 16 == 0 && C % 16 == 0) {
        const int64_t ntiles = cdiv(R, 128) * cdiv(C, 128);
        const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(ntiles, max_grid));
        k_cast_tensor_tile<T, FMT, DELAYED><<<grid, kWG, 0, stream>>>((const T*)x, R, C, src, dl, q, qt, s_out,
                                                                      amax_out);
    } else {
        const int64_t ntiles = cdiv(R, 64) * cdiv(C, 64);
        const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(ntiles, max_grid));
        k_cast_tensor_2d<T, FMT, DELAYED><<<grid, kWG, 0, stream>>>((const T*)x, R, C, src, dl, q, qt, s_out,
                                                                    amax_out);
    }
}

template <bool DELAYED>
static void cast_2d_any(const void* x, int in_bf16, int fmt, int64_t R, int64_t C, ScaleSrc src,
                        const DelayedArgs& dl, uint8_t* q, uint8_t* qt, float* s_out, float* amax_out,
                        hipStream_t stream)
{
    if (in_bf16) {
        if (fmt == kE4M3)
            cast_2d_t<uint16_t, kE4M3, DELAYED>(x, R, C, src, dl, q, qt, s_out, amax_out, stream);
        else
            cast_2d_t<uint16_t, kE5M2, DELAYED>(x, R, C, src, dl, q, qt, s_out, amax_out, stream);
    } else {
        if (fmt == kE4M3)
            cast_2d_t<float, kE4M3, DELAYED>(x, R, C, src, dl, q, qt, s_out, amax_out, stream);
        else
            cast_2d_t<float, kE5M2, DELAYED>(x, R, C, src, dl, q, qt, s_out, amax_out, stream);
    }
}

hipError_t launch_cast_tensor_2d(const void* x, int in_bf16, int fmt, int64_t R, int64_t C, ScaleSrc src,
                                 uint8_t* q, uint8_t* qt, float* s_out, float* amax_out, hipStream_t stream)
{
    cast_2d_any<false>(x, in_bf16, fmt, R, C, src, DelayedArgs{}, q, qt, s_out, amax_out, stream);
    return hipGetLastError();
}

// The flat delayed cast: loads per lane in flight, and the grid (one
// partial per workgroup, at most kMaxPartials).
constexpr int kDelayedLoads = 8;

template <typename T, int FMT>
static void cast_delayed_t(const void* x, int64_t n, const DelayedArgs& dl, uint8_t* q, hipStream_t stream)
{
    const int64_t per = (int64_t)kWG * In<T>::kE * kDelayedLoads;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, per), kMaxPartials));
    k_cast_delayed<T, FMT, kDelayedLoads><<<grid, kWG, 0, stream>>>((const T*)x, n, dl, q);
}

hipError_t launch_cast_delayed(const void* x, int in_bf16, int fmt, int64_t R, int64_t C, const DelayedArgs& dl,
                               uint8_t* q, uint8_t* qt, hipStream_t stream)
{
    if (qt) {
        cast_2d_any<true>(x, in_bf16, fmt, R, C, ScaleSrc{}, dl, q, qt, nullptr, nullptr, stream);
        return hipGetLastError();
    }
    const int64_t n = R * C;
    if (in_bf16) {
        if (fmt == kE4M3)
            cast_delayed_t<uint16_t, kE4M3>(x, n, dl, q, stream);
        else
            cast_delayed_t<uint16_t, kE5M2>(x, n, dl, q, stream);
    } else {
        if (fmt == kE4M3)
            cast_delayed_t<float, kE4M3>(x, n, dl, q, stream);
        else
            cast_delayed_t<float, kE5M2>(x, n, dl, q, stream);
    }
    return hipGetLastError();
}

hipError_t launch_delayed_finish(const float* rec, uint32_t tag_lo, uint32_t tag_hi, float* hist, int H, int slot,
                                 float* alpha, float* s, float fmax_v, float* amax_out, hipStream_t stream)
{
    k_delayed_finish<<<1, kFinishThreads, 0, stream>>>(rec, tag_lo, tag_hi, hist, H, slot, alpha, s, fmax_v,
                                                        amax_out);
    return hipGetLastError();
}

}  // namespace fq
