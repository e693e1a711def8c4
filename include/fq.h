/*
 * fq.h -- C ABI of libfq.so, FP8/FP4 tensor quantization on AMD MI355X
 * (CDNA4, gfx950).
 *
 * Sources (three web pages on FP8/FP4 training; cited by short label):
 *   [MP]  "混合精度训练：fp16 到 fp8" (garden.houmin.site, infra/mixed-precision-fp8)
 *   [CS]  "FP8 Current Scaling：量化、缩放与精度边界" (notes.kuangjux.top)
 *   [LP]  "从 BF16 到 FP8/FP4：大语言模型低精度训练与混合精度预训练" (r00kie-liu.github.io)
 *
 * Conventions for every entry point:
 *   - Tensors are row-major, contiguous, [rows, cols]. "Rowwise" blocks run
 *     along cols (the contiguous axis); "colwise" planes are stored
 *     transposed, [cols, rows] ([MP] section "Per-tensor Current Scaling",
 *     the Hopper flow with cast + cast_transpose).
 *   - All tensor pointers are DEVICE pointers, owned by the caller, and must
 *     be 16-byte aligned; scalar outputs (float*) must be 4-byte aligned.
 *     The library never allocates, frees or synchronizes. All quantization
 *     state (delayed scaling's window and scales) is in caller memory; the
 *     only thing the library keeps between calls is a per-device cache of
 *     occupancy queries (how many workgroups of a kernel fit at once), which
 *     sets launch shapes, never results.
 *   - Work is enqueued on the given HIP stream, in order; the call returns
 *     when it is enqueued. Calls on one stream with one workspace are
 *     ordered; concurrent calls need distinct workspaces and outputs.
 *   - Every argument is validated on the host before anything is enqueued.
 *     On any error nothing is enqueued and nothing is written. FQ_E_HIP
 *     means a launch failed; faults inside kernels surface at the caller's
 *     next synchronization.
 *   - Inputs must be finite ([CS] "Current Scaling" defines the method for
 *     finite tensors). NaN or Inf inputs give unspecified bytes, never a
 *     fault.
 *   - Every produced byte and scale is deterministic: amax reductions take
 *     an exact max, so results do not depend on the launch order.
 */
#ifndef FQ_H
#define FQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP stream handle (the same opaque type HIP's runtime header declares). */
typedef struct ihipStream_t *hipStream_t;

typedef enum {
    FQ_OK = 0,
    FQ_E_INVALID = 1,     /* null pointer, bad enum value, negative size */
    FQ_E_UNSUPPORTED = 2, /* recipe / format / block combination not offered */
    FQ_E_SHAPE = 3,       /* shape not divisible by the block, or too large */
    FQ_E_ALIGN = 4,       /* a pointer is not 16-byte (tensors) or 4-byte (scalars) aligned */
    FQ_E_WORKSPACE = 5,   /* workspace missing or smaller than fq_sizes reports */
    FQ_E_HIP = 6          /* a kernel launch failed */
} fq_status;

/* Element type of the high-precision input. */
typedef enum { FQ_IN_F32 = 0, FQ_IN_BF16 = 1 } fq_in_dtype;

/*
 * Element formats of the quantized data.
 *   FQ_E4M3: 1 sign, 4 exponent, 3 mantissa bits, bias 7, largest 448, no
 *            infinity ([MP] "FP8 数据格式"; [CS] table in "FP8 的两种格式").
 *   FQ_E5M2: 1/5/2, bias 15, largest 57344, with infinities ([MP], [CS] ibid.).
 *   FQ_E2M1: 1/2/1, bias 1, values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives,
 *            two per byte ([MP] section "NVFP4").
 * Rounding is to nearest, ties to even, and saturating: a scaled value beyond
 * the largest finite one takes that value. Zero results keep their sign.
 */
typedef enum { FQ_E4M3 = 0, FQ_E5M2 = 1, FQ_E2M1 = 2 } fq_format;

/*
 * Recipes ([MP] section "FP8 recipe", items 2 to 6):
 *   FQ_PER_TENSOR_CURRENT  a = max|x| of this tensor, alpha = Fmax/a,
 *                          q = Q(fp32(alpha*x)), s = a/Fmax stored
 *                          ([MP] recipe 3; [CS] "Current Scaling").
 *   FQ_PER_TENSOR_DELAYED  cast with the scale derived from an amax window
 *                          of earlier steps, then record this amax in the
 *                          window ([MP] recipe 2; window length and max rule
 *                          from [LP] section 4.3). See fq_quantize_delayed.
 *   FQ_BLOCK_FP32          per-tile current scaling to E4M3 with an fp32
 *                          scale per tile; tiles 1x128 or 128x128
 *                          ([MP] recipe 4 and "Blockwise scaling").
 *   FQ_MX                  MX: 1x32 blocks sharing one E8M0 power-of-two
 *                          scale 2^(floor(log2 amax) - emax), emax =
 *                          floor(log2 Fmax) of the element format: E4M3
 *                          (MXFP8, emax 8) or E5M2 (emax 15) ([MP] "MXFP8"
 *                          and recipe 5), or E2M1 (MXFP4, emax 2, packed two
 *                          per byte; [LP] section 2.4).
 *   FQ_NVFP4               E2M1 elements, 1x16 or 16x16 blocks with E4M3
 *                          block scales, plus one fp32 tensor scale
 *                          ([MP] recipe 6; [LP] section 2.4).
 */
typedef enum {
    FQ_PER_TENSOR_CURRENT = 0,
    FQ_PER_TENSOR_DELAYED = 1,
    FQ_BLOCK_FP32 = 2,
    FQ_MX = 3,
    FQ_NVFP4 = 4
} fq_recipe;

/* Output selection bits. */
enum { FQ_ROWWISE = 1, FQ_COLWISE = 2 };

/*
 * Element rounding.
 *   FQ_ROUND_NEAREST_EVEN  every recipe (the default).
 *   FQ_ROUND_STOCHASTIC    the elements of NVFP4 with 1x16 blocks ([MP]
 *                          "NVFP4": an option for FP4 values; [LP] section
 *                          2.4 item 5: applied to gradients), and the E4M3 /
 *                          E5M2 elements of CURRENT, BLOCK_FP32 with 1x128
 *                          tiles and MX ([MP] "FP8 数据格式": stochastic
 *                          rounding beside round-to-nearest-even). A scaled
 *                          value of magnitude v below the format's largest
 *                          value Fmax, between neighbouring representable
 *                          magnitudes lo <= v < hi (subnormals included),
 *                          with g = (v - lo) / (hi - lo) and u a 16-bit
 *                          random number, rounds to hi iff
 *                          u + g * 2^16 >= 2^16: the random bits are added
 *                          below the last kept bit and the sum truncated, so
 *                          it rounds up with probability floor(g * 2^16) /
 *                          2^16. v >= Fmax saturates; the sign is kept, also
 *                          on zero; every scale (tensor, tile, block) is
 *                          that of round-to-nearest-even. Each output plane
 *                          draws its own bits, so the colwise copy of a
 *                          CURRENT call is the recipe applied to X^T, not
 *                          the transposed rowwise bytes.
 *                          u comes from Philox4x32-10 (Salmon et al., SC
 *                          2011) with key = seed (low word first): the
 *                          element at index e of an output plane
 *                          (row-major in that plane) uses counter
 *                          (h mod 2^32, h >> 32, s mod 2^32, s >> 32) with
 *                          h = e/8 and s = 2*offset + plane (mod 2^64), plane
 *                          0 rowwise and 1 colwise, and bits 16*(e%2) .. +15
 *                          of output word (e%8)/2.
 *                          Results are a pure function of (input, seed,
 *                          offset), independent of launch shape.
 */
typedef enum { FQ_ROUND_NEAREST_EVEN = 0, FQ_ROUND_STOCHASTIC = 1 } fq_rounding;

/*
 * Transform applied before quantization.
 *   FQ_TRANSFORM_NONE   (default).
 *   FQ_TRANSFORM_RHT16  random Hadamard transform of the weight-gradient GEMM
 *                       inputs ([LP] section 2.4 item 3): NVFP4 with 1x16
 *                       blocks and outputs == FQ_COLWISE only. Each row of
 *                       X^T (the GEMM's contraction runs along it) is
 *                       transformed in 16-element chunks, y = (1/4) H16
 *                       diag(s) x, H16 the Sylvester Hadamard matrix, s_i =
 *                       -1 where bit i of rht_signs is set; computed in fp32
 *                       by the fast Walsh-Hadamard butterfly (stages 1, 2, 4,
 *                       8). The transformed tensor is then quantized: its
 *                       amax sets the tensor scale (fq_amax returns that
 *                       amax for this desc), and dequantization returns
 *                       transformed values. The same rht_signs must be used
 *                       for both operands of the GEMM.
 */
typedef enum { FQ_TRANSFORM_NONE = 0, FQ_TRANSFORM_RHT16 = 1 } fq_transform;

/*
 * Scale encoding of FQ_BLOCK_FP32 (other recipes: FQ_SCALE_DEFAULT only).
 *   FQ_SCALE_DEFAULT  s_B = a_B/448 in fp32.
 *   FQ_SCALE_POW2     s_B = 2^(floor(log2 a_B) - 8), the MX rule on the tile
 *                     amax, stored as its fp32 value (2^-127 for an all-zero
 *                     tile); elements are Q_E4M3(x / s_B), the division exact
 *                     ([MP] "Blockwise scaling": the recipe run as MXFP8 blocks
 *                     sharing one power-of-two scale per tile).
 */
typedef enum { FQ_SCALE_DEFAULT = 0, FQ_SCALE_POW2 = 1 } fq_scale_mode;

/*
 * What to quantize and how.
 *   recipe, in_dtype, format: the enums above.
 *   rows, cols:               tensor shape, each >= 0, rows*cols <= 2^36.
 *   block_rows, block_cols:   FQ_BLOCK_FP32 (1,128) or (128,128);
 *                             FQ_MX (1,32); FQ_NVFP4 (1,16) or (16,16);
 *                             ignored by the per-tensor recipes.
 *   outputs:                  FQ_ROWWISE | FQ_COLWISE, at least one.
 *   rounding, seed, offset:   element rounding (fq_rounding above); seed and
 *                             offset are read only for FQ_ROUND_STOCHASTIC.
 *   scale_mode:               fq_scale_mode above.
 *   transform, rht_signs:     fq_transform above.
 *
 * Supported combinations (anything else is FQ_E_UNSUPPORTED):
 *   CURRENT, DELAYED  E4M3 or E5M2, f32 or bf16 input, any shape
 *   BLOCK_FP32        E4M3, rows % br == 0, cols % 128 == 0;
 *                     colwise of 1x128 also needs rows % 128 == 0
 *   MX                E4M3, E5M2 or E2M1, cols % 32 == 0; colwise needs
 *                     rows % 32 == 0
 *   scale_mode POW2   BLOCK_FP32 only
 *   rounding STOCHASTIC  NVFP4 with 1x16 blocks; CURRENT; BLOCK_FP32
 *                     with 1x128 tiles; MX with E4M3 or E5M2 elements
 *   transform RHT16   NVFP4 with 1x16 blocks, outputs == FQ_COLWISE
 *   NVFP4             E2M1, rows % br == 0, cols % 16 == 0;
 *                     colwise needs rows % 16 == 0
 */
typedef struct {
    int32_t recipe;
    int32_t in_dtype;
    int32_t format;
    int64_t rows;
    int64_t cols;
    int32_t block_rows;
    int32_t block_cols;
    uint32_t outputs;
    int32_t rounding;   /* fq_rounding */
    int32_t scale_mode; /* fq_scale_mode */
    uint64_t seed;      /* stochastic rounding: the Philox key */
    uint64_t offset;    /* stochastic rounding: stream number (e.g. the step) */
    int32_t transform;  /* fq_transform */
    uint32_t rht_signs; /* FQ_TRANSFORM_RHT16: sign mask, bits 0..15 */
} fq_desc;

/* One quantized copy: data codes and per-block scales (device memory). */
typedef struct {
    void *data;
    void *scale;
} fq_plane;

/*
 * Output planes (all device memory, caller-owned; sizes from fq_sizes).
 *
 *   recipe       rowwise.data        rowwise.scale             colwise (transposed)
 *   per-tensor   [R,C] u8            unused                    data [C,R] u8 = rowwise^T
 *   block 1x128  [R,C] u8            [R, C/128] f32            [C,R] u8, [C, R/128] f32
 *   block 128^2  [R,C] u8            [R/128, C/128] f32        [C,R] u8, [C/128, R/128] f32
 *   MX           [R,C] u8            [R, C/32] u8 (E8M0)       [C,R] u8, [C, R/32] u8
 *   MXFP4        [R, C/2] u8 packed  [R, C/32] u8 (E8M0)       [C, R/2] u8, [C, R/32] u8
 *   NVFP4 1x16   [R, C/2] u8 packed  [R, C/16] u8 (E4M3)       [C, R/2] u8, [C, R/16] u8
 *   NVFP4 16x16  [R, C/2] u8 packed  [R/16, C/16] u8 (E4M3)    [C, R/2] u8, [C/16, R/16] u8
 *
 * Scale planes are row-major and unswizzled. FP4 packing: element 2k of a
 * row is bits 3..0 of byte k, element 2k+1 bits 7..4.
 * The colwise copy of a 1-D block recipe quantizes X^T with the same block
 * shape (blocks run down the columns of X); that of a 2-D block recipe or a
 * per-tensor recipe is the transpose of the rowwise codes and scales
 * ([MP] "Blockwise scaling": 2-D tiles give the same values either way).
 *
 *   tensor_scale  per-tensor recipes: s = a/Fmax, the dequantization
 *                 multiplier of these bytes; NVFP4: the fp32 tensor scale S.
 *                 Required for those recipes, unused otherwise.
 *   amax          optional (may be NULL): the tensor amax that was used.
 */
typedef struct {
    fq_plane rowwise;
    fq_plane colwise;
    float *tensor_scale;
    float *amax;
} fq_quantized;

/*
 * Delayed-scaling state, all fields but `step` in device memory.
 *   amax_history  history_len floats; zero-filled by the caller before step 0.
 *   scale         alpha, the multiplier casts use; 1.0 before step 0.
 *   scale_inv     s, its dequantization multiplier; 1.0 before step 0.
 *   pending       FQ_DELAYED_PENDING_BYTES, 16-byte aligned, zero-filled
 *                 before step 0: carries a step's amax (as per-workgroup
 *                 partial maxima, tagged with the step) to the next call,
 *                 which records it in the window. A tensor split by rows
 *                 across ranks ([CS] "成本与多 GPU 使用": local amaxes
 *                 reduced with max; history_len <= 1024): after each call,
 *                 an all-reduce with max over `pending` viewed as
 *                 FQ_DELAYED_PENDING_BYTES / 4 32-bit integers (each word
 *                 is a non-negative float or the same on every rank at one
 *                 step) gives every rank the whole tensor's record, so the
 *                 next call's window update and scale are the global ones.
 *   step          host counter t; the caller advances it after each call.
 * See fq_quantize_delayed for when the window and scales are up to date, and
 * fq_delayed_flush for checkpointing.
 */
#define FQ_DELAYED_PENDING_BYTES 8256
typedef struct {
    float *amax_history;
    int32_t history_len;
    float *scale;
    float *scale_inv;
    float *pending;
    int64_t step;
} fq_delayed_state;

/*
 * Buffer sizes in bytes for a desc. Any output pointer may be NULL. A plane
 * not selected by desc->outputs, or not used by the recipe, reports 0.
 * `workspace` is device scratch large enough for every entry point that
 * takes one (fq_quantize, fq_amax, fq_quantize_with_amax,
 * fq_quantize_delayed) with this desc: 4096 bytes for every desc today.
 * fq_quantize of BLOCK_FP32 and MX uses none and also accepts a NULL
 * workspace. Its contents need no initialization and are not preserved.
 * Returns FQ_OK or the validation error the desc would raise.
 */
fq_status fq_sizes(const fq_desc *desc, size_t *row_data, size_t *row_scale, size_t *col_data,
                   size_t *col_scale, size_t *workspace);

/*
 * Quantize x ([rows, cols] of in_dtype, device) with desc's recipe into the
 * planes of *out. Recipes CURRENT, BLOCK_FP32, MX and NVFP4 (DELAYED has its
 * own entry point).
 *   CURRENT: two passes over x, first the amax, then scale and cast
 *     ([MP] recipe 3 and [CS] "成本与多 GPU 使用": the tensor is read twice).
 *   NVFP4: the tensor amax first, then the block pass.
 *   BLOCK_FP32, MX: one pass; block scales are local.
 */
fq_status fq_quantize(const fq_desc *desc, const void *x, const fq_quantized *out, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * amax_out[0] = max|x| over the whole tensor (device float). The first step
 * of current scaling, split out so that a sharded tensor can reduce its
 * shards' amaxes (a max across devices) before casting ([CS] "成本与多 GPU
 * 使用": compute amax, synchronize it, then scale and cast; [MP] "FP8 通信").
 * Uses desc's in_dtype, rows and cols only.
 */
fq_status fq_amax(const fq_desc *desc, const void *x, float *amax_out, void *workspace,
                  size_t workspace_bytes, hipStream_t stream);

/*
 * The second step of current scaling with a given amax (device float),
 * typically the all-reduced max of every shard's fq_amax. Produces the same
 * bytes as fq_quantize on the whole tensor when amax_in is its amax.
 * Recipes CURRENT and NVFP4 (for NVFP4 amax_in is the tensor amax A).
 */
fq_status fq_quantize_with_amax(const fq_desc *desc, const void *x, const float *amax_in,
                                const fq_quantized *out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * One step t = state->step of per-tensor delayed scaling (desc->recipe must
 * be FQ_PER_TENSOR_DELAYED) ([MP] recipe 2: one read of the tensor casts it
 * with the old scale while its amax is recorded in the window):
 *   q = Q(fp32(alpha_old * x))               alpha_old = the scale after step t-1
 *   a_t = max|x|;  amax_history[t mod H] = a_t
 *   m = max(amax_history)
 *   if m > 0: scale = Fmax/m, scale_inv = m/Fmax   (else both unchanged)
 * The codes, and out->tensor_scale (optional: s_old, the multiplier that
 * dequantizes them), are this step's when the call's work completes. The
 * window update of step t runs at the start of step t+1's call, in the same
 * kernel as its cast, from a_t carried in state->pending: so after the call
 * for step t, amax_history and scale/scale_inv are those after step t-1,
 * unless history_len > 1024, in which case the update runs as a second kernel
 * of this call. out->amax (optional) receives a_t (one more small kernel).
 * The workspace is unused (may be NULL). The caller increments state->step
 * afterwards; calls for one state must be ordered (one stream, or events).
 * Every kernel argument of the call for step t repeats with period
 * lcm(2, history_len) in t, so a call captured in a HIP graph at step t
 * replays correctly at steps t + k * lcm(2, history_len).
 */
fq_status fq_quantize_delayed(const fq_desc *desc, const void *x, const fq_delayed_state *state,
                              const fq_quantized *out, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Bring a delayed-scaling state up to date after the call for step
 * state->step - 1 (state->step as the caller advanced it): record that
 * step's amax in the window and set scale/scale_inv from the window, as the
 * next call would; a no-op if state->step == 0. Idempotent: the next call,
 * or a second flush, repeats the same update and changes nothing. After a
 * flush, (amax_history, scale, scale_inv, step) is the whole state:
 * checkpoint those; on resume, zero-fill `pending` (a zero-filled record is
 * never taken for a step's) or restore it too.
 * Uses desc->recipe (FQ_PER_TENSOR_DELAYED) and desc->format.
 */
fq_status fq_delayed_flush(const fq_desc *desc, const fq_delayed_state *state, hipStream_t stream);

/*
 * y = the values that `in` represents ([CS] "Current Scaling": the code value
 * times s), for the plane `which` (FQ_ROWWISE or FQ_COLWISE): y has the shape
 * of that plane's data in elements ([rows, cols] or [cols, rows]), element
 * type y_dtype (FQ_IN_F32 or FQ_IN_BF16), 16-byte aligned device memory.
 *   per-tensor: dec(q) * s;  block: dec(q) * s_tile;
 *   MX: dec(q) * 2^(code-127);  NVFP4: dec(q) * fp32(dec(c_block) * S).
 * Every product is one fp32 multiply, rounded to nearest even; bf16 output
 * rounds that fp32 value to nearest even once more.
 */
fq_status fq_dequantize(const fq_desc *desc, const fq_quantized *in, int32_t which, void *y, int32_t y_dtype,
                        hipStream_t stream);

/*
 * The colwise copy from the rowwise copy alone: de-quantize in->rowwise and
 * re-quantize in the other direction into out->colwise ([MP] section "FP8
 * 通信": the expert-parallel backward pass receives only rowwise FP8 data and
 * needs the colwise copy; power-of-two scales are required so that the
 * double quantization matches a single one up to special values). Round to
 * nearest even, no transform, E4M3 elements, and one of:
 *   FQ_MX, blocks (1,32) (MXFP8): the MX recipe applied down the columns of
 *     the restored values (32x1 blocks, stored transposed: codes [cols,
 *     rows], E8M0 codes [cols, rows/32]); rows % 32 == 0, cols % 32 == 0.
 *   FQ_BLOCK_FP32, blocks (1,128), FQ_SCALE_POW2: the blockwise recipe with
 *     power-of-two scales applied to X_hat^T with 1x128 tiles (codes [cols,
 *     rows], fp32 scales [cols, rows/128]); in->rowwise.scale holds the
 *     [rows, cols/128] fp32 tile scales; rows % 128 == 0, cols % 128 == 0.
 * The restored values dec(q) * scale are exact in fp32. The result equals
 * quantizing the original tensor down the columns except where an element
 * is subnormal or saturated in one of the two scalings. desc->outputs is
 * ignored. Reads one code byte and writes one per element.
 */
fq_status fq_requantize_transpose(const fq_desc *desc, const fq_quantized *in, const fq_quantized *out,
                                  hipStream_t stream);

/*
 * fq_quantize without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same recipes, arguments, results and errors as
 * fq_quantize. The scratch that fq_quantize takes from `workspace` (the amax
 * partials of CURRENT and NVFP4) comes from a 4096-byte array that the
 * library holds on each GPU it runs on, for the life of the process; the call
 * itself allocates nothing. Returns FQ_E_WORKSPACE if a desc needs more
 * scratch than that array holds (none does: every desc needs 4096 bytes or
 * less, whatever its size). Calls on one stream are ordered and safe; calls
 * that overlap in time on one GPU (unordered streams, several host threads)
 * share that GPU's array and race: their results are undefined.
 */
fq_status fq_quantize_noalloc(const fq_desc *desc, const void *x, const fq_quantized *out, hipStream_t stream);

/* A static, human-readable name for a status code. */
const char *fq_status_str(fq_status status);

#ifdef __cplusplus
}
#endif

#endif /* FQ_H */
