// launch.hpp -- host-side launchers of the HIP kernels, called by api.cpp
// after it has validated every argument. Each launcher enqueues on `stream`
// and returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fq {

// Number of workgroups of one kernel that fit on the current device at once
// (occupancy x CUs), for persistent kernels whose workgroups loop over
// tiles. Computed once per device; the library keeps no other state.
struct ResidentGrid {
    static constexpr int kMaxDevices = 64;
    std::atomic<int> slots[kMaxDevices][2] = {};  // [device][lds > 0]
    template <typename K>
    int get(K kernel, int threads, size_t lds)
    {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
            return 1024;
        std::atomic<int>& slot = slots[dev][lds > 0];
        int c = slot.load(std::memory_order_relaxed);
        if (c > 0)
            return c;
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel), threads,
                                                         lds) != hipSuccess ||
            cus <= 0 || per_cu <= 0)
            return 1024;
        c = cus * per_cu;
        slot.store(c, std::memory_order_relaxed);
        return c;
    }
};

// Workspace layout of the per-tensor and NVFP4 paths: one fp32 amax partial
// per workgroup of the amax pass, at most kMaxPartials. They are combined
// without atomics: every workgroup of the second pass (or the delayed-scaling
// finish) re-reduces them from L2.
constexpr int kMaxPartials = 1024;
static_assert(kMaxPartials <= 4 * 256, "consumers read the partials with four loads per thread");
constexpr size_t kPartialsBytes = kMaxPartials * sizeof(float);

// Where a per-tensor cast takes its amax from (current scaling).
struct ScaleSrc {
    const float* partials = nullptr;  // reduce partials[0..n_partials)
    int n_partials = 0;
    const float* amax_in = nullptr;   // or a given amax (quantize_with_amax)
};

// Delayed scaling keeps one record per step in the caller's state: the
// step's amax partials (one per workgroup of its cast, zero beyond the grid)
// followed by a two-word tag naming the step (never all zero). Two records
// alternate by step parity, so step t reads step t-1's record while it
// writes its own.
constexpr int kRecordFloats = kMaxPartials + 8;
constexpr size_t kPendingBytes = 2 * kRecordFloats * sizeof(float);
// Windows up to this length are finished inside the next step's cast (each
// thread of a workgroup reads at most four window slots, in one batch of
// loads); longer windows take a separate one-workgroup finish kernel.
constexpr int kFoldMaxHistory = 4 * 256;

// One delayed-scaling cast (step t).
struct DelayedArgs {
    float* hist = nullptr;            // the window, H floats
    int H = 0;
    const float* prev = nullptr;      // step t-1's record to finish first, or null (t = 0, or H > kFoldMaxHistory)
    int prev_slot = 0;                // (t-1) mod H
    uint32_t prev_tag[2] = {0u, 0u};  // the tag that record carries if it is step t-1's
    float* alpha = nullptr;           // the state's scale (alpha) and scale_inv (s): read, and
    float* s = nullptr;               // written by workgroup 0 when it finishes step t-1
    float fmax = 0.0f;
    float* rec = nullptr;             // this step's record
    uint32_t tag[2] = {0u, 0u};       // this step's tag
    float* s_used = nullptr;          // optional: the s that dequantizes this step's codes
};

// Number of workgroups of an amax pass over n elements of the given size,
// at most max_grid.
int amax_grid(int64_t n, int elem_bytes, int max_grid);

// partials[g] = max|x| over workgroup g's share; grid from amax_grid().
hipError_t launch_amax_partial(const void* x, int in_bf16, int64_t n, float* partials, int grid,
                               hipStream_t stream, int depth = 4);  // depth: 16-byte loads per lane, 4 or 8
// out[0] = max(partials[0..n)).
hipError_t launch_amax_finish(const float* partials, int n, float* out, hipStream_t stream);

// Per-tensor cast of a flat tensor (rowwise bytes only), current scaling.
hipError_t launch_cast_tensor(const void* x, int in_bf16, int fmt, int64_t n, ScaleSrc src, uint8_t* q,
                              float* s_out, float* amax_out, hipStream_t stream);

// Per-tensor cast of a [R, C] tensor writing rowwise bytes q (may be null)
// and transposed bytes qt (may be null), current scaling.
hipError_t launch_cast_tensor_2d(const void* x, int in_bf16, int fmt, int64_t R, int64_t C, ScaleSrc src,
                                 uint8_t* q, uint8_t* qt, float* s_out, float* amax_out, hipStream_t stream);

// One delayed-scaling step: finish step t-1 from its record (if dl.prev),
// cast with the resulting scale, write this step's record. Rowwise bytes q
// and/or transposed bytes qt of the [R, C] tensor.
hipError_t launch_cast_delayed(const void* x, int in_bf16, int fmt, int64_t R, int64_t C, const DelayedArgs& dl,
                               uint8_t* q, uint8_t* qt, hipStream_t stream);

// Finish a delayed step from its record (one workgroup): if rec carries the
// tag (tag_lo, tag_hi), a = max(its partials), hist[slot] = a, m =
// max(hist), and alpha = Fmax/m, s = m/Fmax if m > 0; amax_out (optional)
// receives a. A record with another tag (zero-filled, or another step's)
// changes nothing.
hipError_t launch_delayed_finish(const float* rec, uint32_t tag_lo, uint32_t tag_hi, float* hist, int H, int slot,
                                 float* alpha, float* s, float fmax_v, float* amax_out, hipStream_t stream);

// Blockwise fp32 scales, E4M3. 1x128: flat blocks; 128x128: tiles.
// pow2 = 1: tile scales rounded to the MX power of two 2^(floor(log2 a) - 8).
hipError_t launch_block_1x128(const void* x, int in_bf16, int pow2, int64_t R, int64_t C, uint8_t* q, float* s,
                              hipStream_t stream);
// The colwise copy of 1x128 tiles, and the rowwise one from the same read
// if q is not null. R % 128 == 0, C % 128 == 0.
hipError_t launch_block_1x128_rowcol(const void* x, int in_bf16, int pow2, int64_t R, int64_t C, uint8_t* q,
                                     float* s, uint8_t* qt, float* st, hipStream_t stream);
hipError_t launch_block_128x128(const void* x, int in_bf16, int pow2, int64_t R, int64_t C, uint8_t* q, float* s,
                                uint8_t* qt, float* st, hipStream_t stream);

// MX with E4M3 (fmt 0) or E5M2 (fmt 1) elements: rowwise 1x32 and/or colwise 32x1 (transposed).
hipError_t launch_mx(const void* x, int in_bf16, int fmt, int64_t R, int64_t C, uint8_t* q, uint8_t* e,
                     uint8_t* qt, uint8_t* et, hipStream_t stream);

// MXFP4 from bf16, both planes from one read (tile kernel in k_mx.hip).
hipError_t launch_mxfp4_bf16(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, uint8_t* e, uint8_t* qt,
                             uint8_t* et, hipStream_t stream);

// MXFP4 (E2M1 elements packed two per byte): rowwise 1x32 and/or colwise 32x1 (transposed).
hipError_t launch_mxfp4(const void* x, int in_bf16, int64_t R, int64_t C, uint8_t* q, uint8_t* e, uint8_t* qt,
                        uint8_t* et, hipStream_t stream);

// Stochastic rounding of elements: Philox4x32-10 keyed by seed, stream 2*offset + plane.
struct SrArgs {
    int on = 0;
    uint64_t seed = 0, offset = 0;
};

// Stochastic rounding of the elements to E4M3 / E5M2 (fmt 0 / 1): kind 0
// per-tensor (scale from src), 1 blockwise 1x128 (E4M3; pow2: power-of-two
// scales), 2 MX 1x32. Rowwise codes q (+ scales sq) and/or the colwise copy
// qt (+ sqt) of the [R, C] tensor; s_out / amax_out for per-tensor. Each
// plane draws its own random bits (plane 0 rowwise, 1 colwise).
hipError_t launch_sr8(const void* x, int in_bf16, int fmt, int kind, int pow2, int64_t R, int64_t C, ScaleSrc src,
                      SrArgs sr, uint8_t* q, void* sq, uint8_t* qt, void* sqt, float* s_out, float* amax_out,
                      hipStream_t stream);

// Random Hadamard transform of 16-element chunks along the rows of X^T.
struct RhtArgs {
    int on = 0;
    uint32_t signs = 0;
};

// NVFP4 block pass (after the amax pass): 1x16 or 16x16 blocks; sr.on only
// with 1x16; rht.on only with 1x16 and the colwise plane alone.
hipError_t launch_nvfp4(const void* x, int in_bf16, int64_t R, int64_t C, int br, ScaleSrc src, uint8_t* p,
                        uint8_t* codes, uint8_t* pt, uint8_t* codest, float* S_out, float* amax_out, SrArgs sr,
                        RhtArgs rht, hipStream_t stream);

// partials[g] = max|RHT(X^T)| over workgroup g's share of 16-row strips;
// grid = rht_amax_grid(R, C) (<= kMaxPartials). R % 16 == 0, C % 16 == 0.
int rht_amax_grid(int64_t R, int64_t C);
hipError_t launch_rht_amax_partial(const void* x, int in_bf16, int64_t R, int64_t C, uint32_t signs,
                                   float* partials, int grid, hipStream_t stream);

// Blockwise 1x128 with power-of-two scales: colwise copy (transposed codes,
// fp32 scales [C, R/128]) from the rowwise codes and scales. R % 128 == 0,
// C % 128 == 0.
hipError_t launch_block_requant(const uint8_t* q, const float* s, int64_t R, int64_t C, uint8_t* qt, float* st,
                                hipStream_t stream);

// MXFP8 colwise copy (transposed codes and E8M0 codes) from the rowwise copy.
hipError_t launch_mx_requant(const uint8_t* q, const uint8_t* e, int64_t R, int64_t C, uint8_t* qt, uint8_t* et,
                             hipStream_t stream);

// Dequantization to fp32 (bf = 0) or bf16 (bf = 1).
hipError_t launch_dequant_tensor(const uint8_t* q, int fmt, int64_t n, const float* s, void* y, int bf,
                                 hipStream_t stream);
hipError_t launch_dequant_block(const uint8_t* q, const float* s, int64_t R, int64_t C, int br, int bc, void* y,
                                int bf, hipStream_t stream);
hipError_t launch_dequant_mx(const uint8_t* q, const uint8_t* e, int fmt, int64_t R, int64_t C, void* y, int bf,
                             hipStream_t stream);
hipError_t launch_dequant_nvfp4(const uint8_t* p, const uint8_t* codes, const float* S, int64_t R, int64_t C,
                                int br, int bc, void* y, int bf, hipStream_t stream);

}  // namespace fq
