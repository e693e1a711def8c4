// api.cpp -- the C ABI of libfq.so (include/fq.h): argument validation,
// buffer sizes and dispatch of the HIP kernels onto the caller's stream.
//
// Every check runs on the host before the first launch, so an invalid call
// enqueues nothing and writes nothing.
#include "fq.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.hpp"

namespace {

using namespace fq;

// At most 2^36 elements (128 GiB of bf16). Kernels whose work units can be
// small at narrow shapes (16x16 strips, 32-row slabs, 128-row tiles or
// regions cut by a narrow last column) stride over them with a capped grid;
// every other tiled kernel takes whole 128x128 tiles (both sides multiples
// of 128), at most 2^22 workgroups at this size.
constexpr int64_t kMaxElems = int64_t(1) << 36;
static_assert(kPendingBytes == FQ_DELAYED_PENDING_BYTES, "the pending records' size is part of the ABI");
constexpr int32_t kMaxHistory = 1 << 24;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool per_tensor(int32_t r) { return r == FQ_PER_TENSOR_CURRENT || r == FQ_PER_TENSOR_DELAYED; }

fq_status check_desc(const fq_desc* d)
{
    if (!d)
        return FQ_E_INVALID;
    if (d->recipe < FQ_PER_TENSOR_CURRENT || d->recipe > FQ_NVFP4)
        return FQ_E_INVALID;
    if (d->in_dtype != FQ_IN_F32 && d->in_dtype != FQ_IN_BF16)
        return FQ_E_INVALID;
    if (d->format < FQ_E4M3 || d->format > FQ_E2M1)
        return FQ_E_INVALID;
    if (d->rows < 0 || d->cols < 0)
        return FQ_E_INVALID;
    if ((d->outputs & ~3u) != 0 || (d->outputs & 3u) == 0)
        return FQ_E_INVALID;
    if (d->cols > 0 && d->rows > kMaxElems / d->cols)
        return FQ_E_SHAPE;
    if (d->rounding != FQ_ROUND_NEAREST_EVEN && d->rounding != FQ_ROUND_STOCHASTIC)
        return FQ_E_INVALID;
    if (d->scale_mode != FQ_SCALE_DEFAULT && d->scale_mode != FQ_SCALE_POW2)
        return FQ_E_INVALID;
    if (d->scale_mode == FQ_SCALE_POW2 && d->recipe != FQ_BLOCK_FP32)
        return FQ_E_UNSUPPORTED;
    // stochastic rounding: NVFP4 1x16, and the 8-bit elements of per-tensor
    // current scaling, blockwise 1x128 and MX (E4M3 / E5M2)
    if (d->rounding == FQ_ROUND_STOCHASTIC &&
        !(d->recipe == FQ_NVFP4 && d->block_rows == 1 && d->block_cols == 16) &&
        !(d->recipe == FQ_PER_TENSOR_CURRENT) &&
        !(d->recipe == FQ_BLOCK_FP32 && d->block_rows == 1 && d->block_cols == 128) &&
        !(d->recipe == FQ_MX && d->format != FQ_E2M1))
        return FQ_E_UNSUPPORTED;
    if (d->transform != FQ_TRANSFORM_NONE && d->transform != FQ_TRANSFORM_RHT16)
        return FQ_E_INVALID;
    if (d->transform == FQ_TRANSFORM_RHT16 &&
        !(d->recipe == FQ_NVFP4 && d->block_rows == 1 && d->block_cols == 16 && d->outputs == FQ_COLWISE))
        return FQ_E_UNSUPPORTED;
    const bool col = (d->outputs & FQ_COLWISE) != 0;
    const int64_t R = d->rows, C = d->cols;
    const int br = d->block_rows, bc = d->block_cols;
    switch (d->recipe) {
    case FQ_PER_TENSOR_CURRENT:
    case FQ_PER_TENSOR_DELAYED:
        if (d->format != FQ_E4M3 && d->format != FQ_E5M2)
            return FQ_E_UNSUPPORTED;
        return FQ_OK;
    case FQ_BLOCK_FP32:
        if (d->format != FQ_E4M3)
            return FQ_E_UNSUPPORTED;
        if (!((br == 1 && bc == 128) || (br == 128 && bc == 128)))
            return FQ_E_UNSUPPORTED;
        if (R % br || C % bc)
            return FQ_E_SHAPE;
        if (col && R % 128)
            return FQ_E_SHAPE;
        return FQ_OK;
    case FQ_MX:
        if (d->format != FQ_E4M3 && d->format != FQ_E5M2 && d->format != FQ_E2M1)
            return FQ_E_UNSUPPORTED;
        if (!(br == 1 && bc == 32))
            return FQ_E_UNSUPPORTED;
        if (C % 32 || (col && R % 32))
            return FQ_E_SHAPE;
        return FQ_OK;
    case FQ_NVFP4:
        if (d->format != FQ_E2M1)
            return FQ_E_UNSUPPORTED;
        if (!((br == 1 && bc == 16) || (br == 16 && bc == 16)))
            return FQ_E_UNSUPPORTED;
        if (R % br || C % 16 || (col && R % 16))
            return FQ_E_SHAPE;
        return FQ_OK;
    }
    return FQ_E_INVALID;
}

RhtArgs rht_of(const fq_desc* d)
{
    RhtArgs r;
    r.on = d->transform == FQ_TRANSFORM_RHT16;
    r.signs = d->rht_signs & 0xFFFFu;
    return r;
}

SrArgs sr_of(const fq_desc* d)
{
    SrArgs sr;
    sr.on = d->rounding == FQ_ROUND_STOCHASTIC;
    sr.seed = d->seed;
    sr.offset = d->offset;
    return sr;
}

struct Sizes {
    size_t row_data = 0, row_scale = 0, col_data = 0, col_scale = 0;
    size_t ws = 0;  // what fq_quantize / fq_quantize_with_amax / fq_quantize_delayed need
};

// fq_amax needs the partials for any desc, so fq_sizes reports at least that.
constexpr size_t kAmaxWorkspace = kPartialsBytes;

Sizes sizes_of(const fq_desc* d)
{
    Sizes z;
    const size_t R = (size_t)d->rows, C = (size_t)d->cols;
    const bool row = d->outputs & FQ_ROWWISE, col = d->outputs & FQ_COLWISE;
    switch (d->recipe) {
    case FQ_PER_TENSOR_CURRENT:
        z.row_data = row ? R * C : 0;
        z.col_data = col ? R * C : 0;
        z.ws = kPartialsBytes;
        break;
    case FQ_PER_TENSOR_DELAYED:
        // the amax partials live in the state's pending records
        z.row_data = row ? R * C : 0;
        z.col_data = col ? R * C : 0;
        break;
    case FQ_BLOCK_FP32:
        z.row_data = row ? R * C : 0;
        z.col_data = col ? R * C : 0;
        if (d->block_rows == 1) {
            z.row_scale = row ? R * (C / 128) * 4 : 0;
            z.col_scale = col ? C * (R / 128) * 4 : 0;
        } else {
            z.row_scale = row ? (R / 128) * (C / 128) * 4 : 0;
            z.col_scale = col ? (C / 128) * (R / 128) * 4 : 0;
        }
        break;
    case FQ_MX:
        z.row_data = row ? R * C / (d->format == FQ_E2M1 ? 2 : 1) : 0;
        z.col_data = col ? R * C / (d->format == FQ_E2M1 ? 2 : 1) : 0;
        z.row_scale = row ? R * (C / 32) : 0;
        z.col_scale = col ? C * (R / 32) : 0;
        break;
    case FQ_NVFP4:
        z.row_data = row ? R * C / 2 : 0;
        z.col_data = col ? R * C / 2 : 0;
        if (d->block_rows == 1) {
            z.row_scale = row ? R * (C / 16) : 0;
            z.col_scale = col ? C * (R / 16) : 0;
        } else {
            z.row_scale = row ? (R / 16) * (C / 16) : 0;
            z.col_scale = col ? (C / 16) * (R / 16) : 0;
        }
        z.ws = kPartialsBytes;
        break;
    }
    return z;
}

// Output planes a recipe needs, present and aligned.
fq_status check_out(const fq_desc* d, const fq_quantized* o, bool need_tensor_scale)
{
    if (!o)
        return FQ_E_INVALID;
    const bool any = d->rows > 0 && d->cols > 0;
    const bool scaled_planes = d->recipe == FQ_BLOCK_FP32 || d->recipe == FQ_MX || d->recipe == FQ_NVFP4;
    const fq_plane* planes[2] = {&o->rowwise, &o->colwise};
    const uint32_t bits[2] = {FQ_ROWWISE, FQ_COLWISE};
    for (int i = 0; i < 2; ++i) {
        if (!(d->outputs & bits[i]))
            continue;
        if (any && !planes[i]->data)
            return FQ_E_INVALID;
        if (any && scaled_planes && !planes[i]->scale)
            return FQ_E_INVALID;
        if (!aligned(planes[i]->data, 16) || !aligned(planes[i]->scale, 16))
            return FQ_E_ALIGN;
    }
    if (need_tensor_scale && !o->tensor_scale)
        return FQ_E_INVALID;
    if (!aligned(o->tensor_scale, 4) || !aligned(o->amax, 4))
        return FQ_E_ALIGN;
    return FQ_OK;
}

fq_status check_x(const fq_desc* d, const void* x)
{
    if (d->rows > 0 && d->cols > 0 && !x)
        return FQ_E_INVALID;
    if (!aligned(x, 16))
        return FQ_E_ALIGN;
    return FQ_OK;
}

fq_status check_ws(const Sizes& z, const void* ws, size_t ws_bytes)
{
    if (z.ws == 0)
        return FQ_OK;
    if (!ws || ws_bytes < z.ws)
        return FQ_E_WORKSPACE;
    if (!aligned(ws, 16))
        return FQ_E_ALIGN;
    return FQ_OK;
}

fq_status hip_status(hipError_t e) { return e == hipSuccess ? FQ_OK : FQ_E_HIP; }

int elem_bytes(const fq_desc* d) { return d->in_dtype == FQ_IN_BF16 ? 2 : 4; }

// Stochastically rounded 8-bit elements of a validated desc (per-tensor with
// src, blockwise 1x128, MX E4M3 / E5M2).
fq_status run_sr8(const fq_desc* d, const void* x, ScaleSrc src, const fq_quantized* o, hipStream_t st)
{
    const bool row = d->outputs & FQ_ROWWISE, col = d->outputs & FQ_COLWISE;
    const int kind = d->recipe == FQ_PER_TENSOR_CURRENT ? 0 : d->recipe == FQ_BLOCK_FP32 ? 1 : 2;
    return hip_status(launch_sr8(x, d->in_dtype == FQ_IN_BF16, d->format, kind, d->scale_mode == FQ_SCALE_POW2,
                                 d->rows, d->cols, src, sr_of(d), row ? (uint8_t*)o->rowwise.data : nullptr,
                                 row ? o->rowwise.scale : nullptr, col ? (uint8_t*)o->colwise.data : nullptr,
                                 col ? o->colwise.scale : nullptr, kind == 0 ? o->tensor_scale : nullptr,
                                 kind == 0 ? o->amax : nullptr, st));
}

// Per-tensor current-scaling cast (amax from partials or given) of a validated desc.
fq_status run_per_tensor_cast(const fq_desc* d, const void* x, ScaleSrc src, const fq_quantized* o, hipStream_t st)
{
    if (d->rounding == FQ_ROUND_STOCHASTIC)
        return run_sr8(d, x, src, o, st);
    const int bf = d->in_dtype == FQ_IN_BF16;
    const int64_t n = d->rows * d->cols;
    uint8_t* q = (d->outputs & FQ_ROWWISE) ? (uint8_t*)o->rowwise.data : nullptr;
    uint8_t* qt = (d->outputs & FQ_COLWISE) ? (uint8_t*)o->colwise.data : nullptr;
    if (qt)
        return hip_status(launch_cast_tensor_2d(x, bf, d->format, d->rows, d->cols, src, q, qt, o->tensor_scale,
                                                o->amax, st));
    return hip_status(launch_cast_tensor(x, bf, d->format, n, src, q, o->tensor_scale, o->amax, st));
}

// A delayed state's fields, present, aligned and in range.
fq_status check_state(const fq_delayed_state* state)
{
    if (!state || !state->amax_history || !state->scale || !state->scale_inv || !state->pending)
        return FQ_E_INVALID;
    if (state->history_len < 1 || state->history_len > kMaxHistory || state->step < 0)
        return FQ_E_INVALID;
    if (!aligned(state->amax_history, 4) || !aligned(state->scale, 4) || !aligned(state->scale_inv, 4) ||
        !aligned(state->pending, 16))
        return FQ_E_ALIGN;
    return FQ_OK;
}

float* record_of(const fq_delayed_state* state, int64_t step)
{
    return state->pending + (step & 1) * kRecordFloats;
}

// The tag of step t's record: (t mod L) + 1 with L = lcm(2, H), the period
// of the window slot and of the record's parity, so every argument of a
// step's kernels repeats with period L (a step captured in a graph replays
// correctly L steps later), and never 0 (a zero-filled record is never
// taken for a step's); then a constant word.
constexpr uint32_t kRecordMagic = 0x46510D1Au;

void record_tag(int64_t t, int64_t H, uint32_t tag[2])
{
    const int64_t L = (H % 2 == 0) ? H : 2 * H;
    tag[0] = (uint32_t)(t % L) + 1u;
    tag[1] = kRecordMagic;
}

float fmax_of(const fq_desc* d) { return d->format == FQ_E4M3 ? 448.0f : 57344.0f; }

}  // namespace

extern "C" {

const char* fq_status_str(fq_status s)
{
    switch (s) {
    case FQ_OK: return "FQ_OK";
    case FQ_E_INVALID: return "FQ_E_INVALID: null pointer, bad enum value or negative size";
    case FQ_E_UNSUPPORTED: return "FQ_E_UNSUPPORTED: recipe, format or block combination not offered";
    case FQ_E_SHAPE: return "FQ_E_SHAPE: shape not divisible by the block, or too large";
    case FQ_E_ALIGN: return "FQ_E_ALIGN: pointer not 16-byte (tensor) or 4-byte (scalar) aligned";
    case FQ_E_WORKSPACE: return "FQ_E_WORKSPACE: workspace missing or too small";
    case FQ_E_HIP: return "FQ_E_HIP: a kernel launch failed";
    }
    return "unknown fq_status";
}

fq_status fq_sizes(const fq_desc* d, size_t* row_data, size_t* row_scale, size_t* col_data, size_t* col_scale,
                   size_t* workspace)
{
    const fq_status st = check_desc(d);
    if (st != FQ_OK)
        return st;
    const Sizes z = sizes_of(d);
    if (row_data)
        *row_data = z.row_data;
    if (row_scale)
        *row_scale = z.row_scale;
    if (col_data)
        *col_data = z.col_data;
    if (col_scale)
        *col_scale = z.col_scale;
    if (workspace)
        *workspace = z.ws > kAmaxWorkspace ? z.ws : kAmaxWorkspace;
    return FQ_OK;
}

fq_status fq_amax(const fq_desc* d, const void* x, float* amax_out, void* ws, size_t ws_bytes, hipStream_t st)
{
    if (!d)
        return FQ_E_INVALID;
    if (d->in_dtype != FQ_IN_F32 && d->in_dtype != FQ_IN_BF16)
        return FQ_E_INVALID;
    if (d->rows < 0 || d->cols < 0)
        return FQ_E_INVALID;
    if (d->cols > 0 && d->rows > kMaxElems / d->cols)
        return FQ_E_SHAPE;
    if (!amax_out)
        return FQ_E_INVALID;
    fq_status s = check_x(d, x);
    if (s != FQ_OK)
        return s;
    if (!aligned(amax_out, 4))
        return FQ_E_ALIGN;
    Sizes z;
    z.ws = kAmaxWorkspace;
    if ((s = check_ws(z, ws, ws_bytes)) != FQ_OK)
        return s;
    const int64_t n = d->rows * d->cols;
    float* partials = (float*)ws;
    int g;
    if (d->transform == FQ_TRANSFORM_RHT16) {
        // the amax of the transformed tensor (NVFP4 1x16 colwise with the RHT)
        if ((s = check_desc(d)) != FQ_OK)
            return s;
        g = rht_amax_grid(d->rows, d->cols);
        s = n > 0 ? hip_status(launch_rht_amax_partial(x, d->in_dtype == FQ_IN_BF16, d->rows, d->cols,
                                                       d->rht_signs & 0xFFFFu, partials, g, st))
                  : hip_status(launch_amax_partial(x, d->in_dtype == FQ_IN_BF16, n, partials, g, st));
    } else {
        if (d->transform != FQ_TRANSFORM_NONE)
            return FQ_E_INVALID;
        g = amax_grid(n, elem_bytes(d), kMaxPartials);
        s = hip_status(launch_amax_partial(x, d->in_dtype == FQ_IN_BF16, n, partials, g, st, 8));
    }
    if (s != FQ_OK)
        return s;
    return hip_status(launch_amax_finish(partials, g, amax_out, st));
}

fq_status fq_quantize(const fq_desc* d, const void* x, const fq_quantized* o, void* ws, size_t ws_bytes,
                      hipStream_t st)
{
    fq_status s = check_desc(d);
    if (s != FQ_OK)
        return s;
    if (d->recipe == FQ_PER_TENSOR_DELAYED)
        return FQ_E_UNSUPPORTED;
    if ((s = check_x(d, x)) != FQ_OK)
        return s;
    const bool tensor_scale = d->recipe == FQ_PER_TENSOR_CURRENT || d->recipe == FQ_NVFP4;
    if ((s = check_out(d, o, tensor_scale)) != FQ_OK)
        return s;
    const Sizes z = sizes_of(d);
    if ((s = check_ws(z, ws, ws_bytes)) != FQ_OK)
        return s;

    const int bf = d->in_dtype == FQ_IN_BF16;
    const int64_t R = d->rows, C = d->cols, n = R * C;
    const bool row = d->outputs & FQ_ROWWISE, col = d->outputs & FQ_COLWISE;
    switch (d->recipe) {
    case FQ_PER_TENSOR_CURRENT: {
        float* partials = (float*)ws;
        const int g = amax_grid(n, elem_bytes(d), kMaxPartials);
        if ((s = hip_status(launch_amax_partial(x, bf, n, partials, g, st, 8))) != FQ_OK)
            return s;
        ScaleSrc src;
        src.partials = partials;
        src.n_partials = g;
        return run_per_tensor_cast(d, x, src, o, st);
    }
    case FQ_BLOCK_FP32: {
        if (n == 0)
            return FQ_OK;
        if (d->rounding == FQ_ROUND_STOCHASTIC)
            return run_sr8(d, x, ScaleSrc(), o, st);
        const int pow2 = d->scale_mode == FQ_SCALE_POW2;
        if (d->block_rows == 1) {
            // a colwise plane: 128x128 tiles (R % 128 == 0), the rowwise plane from the same read
            if (col)
                return hip_status(launch_block_1x128_rowcol(
                    x, bf, pow2, R, C, row ? (uint8_t*)o->rowwise.data : nullptr,
                    row ? (float*)o->rowwise.scale : nullptr, (uint8_t*)o->colwise.data, (float*)o->colwise.scale, st));
            return hip_status(launch_block_1x128(x, bf, pow2, R, C, (uint8_t*)o->rowwise.data,
                                                 (float*)o->rowwise.scale, st));
        }
        return hip_status(launch_block_128x128(x, bf, pow2, R, C, row ? (uint8_t*)o->rowwise.data : nullptr,
                                               row ? (float*)o->rowwise.scale : nullptr,
                                               col ? (uint8_t*)o->colwise.data : nullptr,
                                               col ? (float*)o->colwise.scale : nullptr, st));
    }
    case FQ_MX:
        if (n == 0)
            return FQ_OK;
        if (d->rounding == FQ_ROUND_STOCHASTIC)
            return run_sr8(d, x, ScaleSrc(), o, st);
        if (d->format == FQ_E2M1)
            return hip_status(launch_mxfp4(x, bf, R, C, row ? (uint8_t*)o->rowwise.data : nullptr,
                                           row ? (uint8_t*)o->rowwise.scale : nullptr,
                                           col ? (uint8_t*)o->colwise.data : nullptr,
                                           col ? (uint8_t*)o->colwise.scale : nullptr, st));
        return hip_status(launch_mx(x, bf, d->format, R, C, row ? (uint8_t*)o->rowwise.data : nullptr,
                                    row ? (uint8_t*)o->rowwise.scale : nullptr,
                                    col ? (uint8_t*)o->colwise.data : nullptr,
                                    col ? (uint8_t*)o->colwise.scale : nullptr, st));
    case FQ_NVFP4: {
        const bool rht = d->transform == FQ_TRANSFORM_RHT16;
        const int g = rht ? rht_amax_grid(R, C) : amax_grid(n, elem_bytes(d), kMaxPartials);
        float* partials = (float*)ws;
        if (rht && n > 0)
            s = hip_status(launch_rht_amax_partial(x, bf, R, C, d->rht_signs & 0xFFFFu, partials, g, st));
        else
            s = hip_status(launch_amax_partial(x, bf, n, partials, g, st));
        if (s != FQ_OK)
            return s;
        ScaleSrc src;
        src.partials = partials;
        src.n_partials = g;
        return hip_status(launch_nvfp4(x, bf, R, C, d->block_rows, src, row ? (uint8_t*)o->rowwise.data : nullptr,
                                       row ? (uint8_t*)o->rowwise.scale : nullptr,
                                       col ? (uint8_t*)o->colwise.data : nullptr,
                                       col ? (uint8_t*)o->colwise.scale : nullptr, o->tensor_scale, o->amax,
                                       sr_of(d), rht_of(d), st));
    }
    }
    return FQ_E_INVALID;
}

fq_status fq_quantize_with_amax(const fq_desc* d, const void* x, const float* amax_in, const fq_quantized* o,
                                void* ws, size_t ws_bytes, hipStream_t st)
{
    (void)ws;
    (void)ws_bytes;
    fq_status s = check_desc(d);
    if (s != FQ_OK)
        return s;
    if (d->recipe != FQ_PER_TENSOR_CURRENT && d->recipe != FQ_NVFP4)
        return FQ_E_UNSUPPORTED;
    if (!amax_in)
        return FQ_E_INVALID;
    if (!aligned(amax_in, 4))
        return FQ_E_ALIGN;
    if ((s = check_x(d, x)) != FQ_OK)
        return s;
    if ((s = check_out(d, o, true)) != FQ_OK)
        return s;
    ScaleSrc src;
    src.amax_in = amax_in;
    if (d->recipe == FQ_PER_TENSOR_CURRENT)
        return run_per_tensor_cast(d, x, src, o, st);
    const bool row = d->outputs & FQ_ROWWISE, col = d->outputs & FQ_COLWISE;
    return hip_status(launch_nvfp4(x, d->in_dtype == FQ_IN_BF16, d->rows, d->cols, d->block_rows, src,
                                   row ? (uint8_t*)o->rowwise.data : nullptr,
                                   row ? (uint8_t*)o->rowwise.scale : nullptr,
                                   col ? (uint8_t*)o->colwise.data : nullptr,
                                   col ? (uint8_t*)o->colwise.scale : nullptr, o->tensor_scale, o->amax,
                                   sr_of(d), rht_of(d), st));
}

fq_status fq_quantize_delayed(const fq_desc* d, const void* x, const fq_delayed_state* state,
                              const fq_quantized* o, void* ws, size_t ws_bytes, hipStream_t st)
{
    (void)ws;
    (void)ws_bytes;
    fq_status s = check_desc(d);
    if (s != FQ_OK)
        return s;
    if (d->recipe != FQ_PER_TENSOR_DELAYED)
        return FQ_E_UNSUPPORTED;
    if ((s = check_state(state)) != FQ_OK)
        return s;
    if ((s = check_x(d, x)) != FQ_OK)
        return s;
    if ((s = check_out(d, o, false)) != FQ_OK)
        return s;
    const int64_t t = state->step, H = state->history_len;
    DelayedArgs dl;
    dl.hist = state->amax_history;
    dl.H = (int)H;
    dl.alpha = state->scale;
    dl.s = state->scale_inv;
    dl.fmax = fmax_of(d);
    dl.rec = record_of(state, t);
    record_tag(t, H, dl.tag);
    dl.s_used = o->tensor_scale;
    const bool fold = H <= kFoldMaxHistory;
    if (fold && t >= 1) {
        // this step first finishes step t-1 from its record
        dl.prev = record_of(state, t - 1);
        dl.prev_slot = (int)((t - 1) % H);
        record_tag(t - 1, H, dl.prev_tag);
    }
    uint8_t* q = (d->outputs & FQ_ROWWISE) ? (uint8_t*)o->rowwise.data : nullptr;
    uint8_t* qt = (d->outputs & FQ_COLWISE) ? (uint8_t*)o->colwise.data : nullptr;
    if ((s = hip_status(launch_cast_delayed(x, d->in_dtype == FQ_IN_BF16, d->format, d->rows, d->cols, dl, q, qt,
                                            st))) != FQ_OK)
        return s;
    if (!fold)
        // a long window: this step's update runs now, as its own kernel
        return hip_status(launch_delayed_finish(dl.rec, dl.tag[0], dl.tag[1], dl.hist, dl.H, (int)(t % H), dl.alpha,
                                                dl.s, dl.fmax, o->amax, st));
    if (o->amax)
        return hip_status(launch_amax_finish(dl.rec, kMaxPartials, o->amax, st));
    return FQ_OK;
}

fq_status fq_delayed_flush(const fq_desc* d, const fq_delayed_state* state, hipStream_t st)
{
    fq_status s = check_desc(d);
    if (s != FQ_OK)
        return s;
    if (d->recipe != FQ_PER_TENSOR_DELAYED)
        return FQ_E_UNSUPPORTED;
    if ((s = check_state(state)) != FQ_OK)
        return s;
    const int64_t t = state->step, H = state->history_len;
    if (t == 0)
        return FQ_OK;  // no step has run
    uint32_t tag[2];
    record_tag(t - 1, H, tag);
    return hip_status(launch_delayed_finish(record_of(state, t - 1), tag[0], tag[1], state->amax_history, (int)H,
                                            (int)((t - 1) % H), state->scale, state->scale_inv, fmax_of(d), nullptr,
                                            st));
}

fq_status fq_dequantize(const fq_desc* d, const fq_quantized* in, int32_t which, void* y, int32_t y_dtype,
                        hipStream_t st)
{
    fq_status s = check_desc(d);
    if (s != FQ_OK)
        return s;
    if (which != FQ_ROWWISE && which != FQ_COLWISE)
        return FQ_E_INVALID;
    if (!(d->outputs & (uint32_t)which))
        return FQ_E_INVALID;
    if (y_dtype != FQ_IN_F32 && y_dtype != FQ_IN_BF16)
        return FQ_E_INVALID;
    const bool ts = per_tensor(d->recipe) || d->recipe == FQ_NVFP4;
    if ((s = check_out(d, in, ts)) != FQ_OK)
        return s;
    const int64_t R0 = d->rows, C0 = d->cols;
    if (R0 * C0 == 0)
        return FQ_OK;
    if (!y)
        return FQ_E_INVALID;
    if (!aligned(y, 16))
        return FQ_E_ALIGN;
    const bool colw = which == FQ_COLWISE;
    const int bf = y_dtype == FQ_IN_BF16;
    const fq_plane& p = colw ? in->colwise : in->rowwise;
    // a colwise plane is the rowwise layout of the transposed shape
    const int64_t R = colw ? C0 : R0, C = colw ? R0 : C0;
    switch (d->recipe) {
    case FQ_PER_TENSOR_CURRENT:
    case FQ_PER_TENSOR_DELAYED:
        return hip_status(launch_dequant_tensor((const uint8_t*)p.data, d->format, R * C, in->tensor_scale, y, bf, st));
    case FQ_BLOCK_FP32:
        return hip_status(launch_dequant_block((const uint8_t*)p.data, (const float*)p.scale, R, C,
                                               d->block_rows, 128, y, bf, st));
    case FQ_MX:
        return hip_status(launch_dequant_mx((const uint8_t*)p.data, (const uint8_t*)p.scale, d->format, R, C, y, bf,
                                            st));
    case FQ_NVFP4:
        return hip_status(launch_dequant_nvfp4((const uint8_t*)p.data, (const uint8_t*)p.scale, in->tensor_scale, R,
                                               C, d->block_rows, 16, y, bf, st));
    }
    return FQ_E_INVALID;
}

fq_status fq_requantize_transpose(const fq_desc* d, const fq_quantized* in, const fq_quantized* out, hipStream_t st)
{
    if (!d)
        return FQ_E_INVALID;
    if (d->recipe < FQ_PER_TENSOR_CURRENT || d->recipe > FQ_NVFP4 || d->rows < 0 || d->cols < 0)
        return FQ_E_INVALID;
    if (d->rounding != FQ_ROUND_NEAREST_EVEN && d->rounding != FQ_ROUND_STOCHASTIC)
        return FQ_E_INVALID;
    if (d->scale_mode != FQ_SCALE_DEFAULT && d->scale_mode != FQ_SCALE_POW2)
        return FQ_E_INVALID;
    if (d->transform != FQ_TRANSFORM_NONE && d->transform != FQ_TRANSFORM_RHT16)
        return FQ_E_INVALID;
    // MXFP8, or blockwise 1x128 with power-of-two scales ([MP] "FP8 通信":
    // only power-of-two scales make the restored values exact)
    const bool common = d->format == FQ_E4M3 && d->block_rows == 1 && d->transform == FQ_TRANSFORM_NONE &&
                        d->rounding == FQ_ROUND_NEAREST_EVEN;
    const bool mx = common && d->recipe == FQ_MX && d->block_cols == 32 && d->scale_mode == FQ_SCALE_DEFAULT;
    const bool blk = common && d->recipe == FQ_BLOCK_FP32 && d->block_cols == 128 && d->scale_mode == FQ_SCALE_POW2;
    if (!mx && !blk)
        return FQ_E_UNSUPPORTED;
    if (d->cols > 0 && d->rows > kMaxElems / d->cols)
        return FQ_E_SHAPE;
    const int64_t unit = mx ? 32 : 128;
    if (d->rows % unit || d->cols % unit)
        return FQ_E_SHAPE;
    if (!in || !out)
        return FQ_E_INVALID;
    const int64_t R = d->rows, C = d->cols;
    if (R * C == 0)
        return FQ_OK;
    if (!in->rowwise.data || !in->rowwise.scale || !out->colwise.data || !out->colwise.scale)
        return FQ_E_INVALID;
    if (!aligned(in->rowwise.data, 16) || !aligned(in->rowwise.scale, 16) || !aligned(out->colwise.data, 16) ||
        !aligned(out->colwise.scale, 16))
        return FQ_E_ALIGN;
    if (blk)
        return hip_status(launch_block_requant((const uint8_t*)in->rowwise.data, (const float*)in->rowwise.scale, R,
                                               C, (uint8_t*)out->colwise.data, (float*)out->colwise.scale, st));
    return hip_status(launch_mx_requant((const uint8_t*)in->rowwise.data, (const uint8_t*)in->rowwise.scale, R, C,
                                        (uint8_t*)out->colwise.data, (uint8_t*)out->colwise.scale, st));
}

}  // extern "C"
