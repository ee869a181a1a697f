// Internal interface between the C-ABI dispatcher and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

constexpr int kTileM = 256;        // output tile rows of every GEMM kernel
constexpr int kTileN = 256;        // output tile columns
constexpr int kSliceBytesABI = 128; // bytes of contraction per operand row and k-slice (split-K granule)

// Element type of x and W (and of the chunk's logits/dlogits buffer).
enum class In { BF16 = 0, FP32 = 1 };

// Per-call normalisation, written on the device by the scale kernel before anything reads it:
// `grad` multiplies each counted token's dlogits row (1 / counted tokens for a mean, 1 for a
// sum); the loss is the sum of the per-token losses divided by `denom` (counted tokens, or 1).
struct Scale {
  float grad;
  float pad;
  double denom;
};

// Which tokens count: a target equal to ignore_index (when ignore_on) contributes no loss and a
// zero dlogits row; every other target counts (one outside [0, V) raises the data flag).
struct Ignore {
  int64_t index;
  int on;
  __host__ __device__ bool skip(int64_t t) const { return on && t == index; }
};

struct ScaleArgs {
  const int64_t* t;     // all N targets
  int64_t n;
  Ignore ign;
  int sum;              // 1: reduction "sum"
  Scale* out;
};

struct LogitsArgs {
  const void* x;        // chunk's first token row, [rows][H]
  const void* W;        // [V][H]
  const int64_t* t;     // chunk's targets [rows]
  void* z;              // logits buffer [rows][ldz] (in-type), may be null (pass-1 only)
  float* pm;            // per-(vocab tile, row) max   [tiles_n][pstride]
  float* ps;            // per-(vocab tile, row) sum of exp(z - max)
  float* zt;            // target logit per row (fp32 accumulator value) [rows]
  int64_t ldz;
  int pstride;
  int rows, H, V;
  int tiles_m, tiles_n;
  unsigned long long* clk; // null, or [2]: summed workgroup lifetimes in shader-clock and 100 MHz ticks
};

struct CombineArgs {
  const float* pm;
  const float* ps;
  const float* zt;
  const int64_t* t;
  float* lse;           // [rows]
  float* loss_rows;     // [rows]
  int* flag;            // bit 0: a target outside [0, V)
  Ignore ign;
  int pstride, tiles_n, rows, V;
};

struct DlogitsArgs {
  void* z;              // [rows][ldz] in-type: z - M per 256-column tile, overwritten with G
  const float* pm;      // [ldz / 256][pstride] the tile maxima M
  int pstride;
  const float* lse;
  const int64_t* t;
  int64_t ldz;
  int rows, V;
  Ignore ign;
  const Scale* scale;
};

struct DxArgs {
  const void* g;        // [rows][ldg]
  const void* W;        // [V][H]
  float* part;          // [splits][rows_max][H] fp32 when splits > 1
  void* dx;             // chunk's first row of dx [rows][H]
  int64_t ldg;
  int64_t part_stride;  // rows_max * H
  int rows, H, V;
  int k_per_split, splits;
  int tiles_m, tiles_n;
  int dx_fp32;
  int accumulate;       // 0: overwrite dx rows, 1: dx += G W (splits == 1 only; else in the reduce)
  unsigned long long* clk; // null, or [2]: summed workgroup lifetimes in shader-clock and 100 MHz ticks
};

struct DxReduceArgs {
  const float* part;
  void* dx;
  int64_t part_stride;
  int64_t count;        // rows * H
  int splits;
  int dx_fp32;
  int accumulate;       // 0: overwrite, 1: add into dx
};

struct DwArgs {
  const void* g;        // [rows][ldg]
  const void* x;        // chunk's first token row [rows][H]
  void* dW;             // [V][H]
  int64_t ldg;
  int rows, H, V;
  int tiles_m, tiles_n;
  int dw_fp32;
  int accumulate;       // 0: overwrite dW, 1: dW += G^T x
  unsigned long long* clk; // null, or [2]: summed workgroup lifetimes in shader-clock and 100 MHz ticks
};

struct FinalizeArgs {
  const float* loss_rows;
  float* loss;
  int64_t n;
  const Scale* scale;   // loss = sum / scale->denom
};

// Fused variant, pass 2: a workgroup owns a block of bm x bn tiles of (tokens x vocabulary); it
// recomputes their logits once, keeps the block's dlogits in its own bf16 buffer in the workspace,
// then, per 256-wide slice of H, forms whole dx and dW tiles over the block and adds each with one
// fp32 atomic per element.  The atomic count, rows V H (1 / (256 bn) + 1 / (256 bm)), sets the
// time (measured at the Llama-3 chunk, fused_bwd per 4096 tokens: 2 x 2 tiles 32.8 ms, 4 x 4 19.2,
// 4 x 8 18.0, 8 x 4 17.1), so the largest block is best as long as there are enough blocks to keep
// every compute unit busy.  The shapes the kernel is built for, largest first:
constexpr int kFusedShapes[4][2] = {{8, 4}, {4, 4}, {4, 2}, {2, 2}};
constexpr int64_t kFusedGBlockBytes = (int64_t)8 * kTileM * 4 * kTileN * 2;   // 4 MiB: the largest shape's buffer
constexpr int kFusedMaxGrid = 256;                          // resident workgroups (one per compute unit)

struct FusedBlockArgs {
  const void* x;        // first token row of the launch [rows][H] (bf16)
  const void* W;        // [V][H] (bf16)
  const int64_t* t;     // targets of those rows [rows]
  const float* lse;     // their log-sum-exp [rows]
  float* dx_acc;        // fp32 [rows][H], cleared (or holding the values to add to) before the launch
  float* dw_acc;        // fp32 [V][H], cleared before the first launch of a call
  char* gbuf;           // [gridDim.x][kFusedGBlockBytes]: each workgroup's dlogits block (bf16)
  int rows, H, V;
  int tiles_h;
  int bm, bn;               // block shape in tiles: one of kFusedShapes
  int blocks_m, blocks_n;   // token blocks of the launch, vocabulary blocks
  int group_m;              // blocks are walked in groups of group_m token blocks that sweep all vocabulary blocks
  Ignore ign;
  const Scale* scale;
};

struct FillArgs {
  float* p;
  int64_t n;            // multiple of 4
};

struct CastArgs {       // fp32 -> bf16, round to nearest even
  const float* src;
  void* dst;
  int64_t n;            // multiple of 4
  int accumulate;       // 1: dst = bf16(dst + src)
};

// RMSNorm in front of the head, per token chunk: x = h * rstd * gamma with
// rstd = 1 / sqrt(mean(h^2) + eps), and its backward from the chunk's fp32 dL/dx.
struct RmsFwdArgs {
  const void* h;        // chunk's first row [rows][H] (in-type)
  const void* gamma;    // [H] (in-type)
  void* x;              // [rows][H] (in-type)
  float* rstd;          // [rows]
  int rows, H;
  float eps;
};

constexpr int kRmsRowsPerBlock = 8;   // rows whose dgamma contributions one backward block sums

struct RmsBwdArgs {
  const float* dx;      // [rows][H] fp32
  const void* h;        // [rows][H] (in-type)
  const void* gamma;    // [H] (in-type)
  const float* rstd;    // [rows]
  void* dh;             // chunk's first row of dh [rows][H]
  float* part;          // [ceil(rows / kRmsRowsPerBlock)][H] fp32 dgamma partials
  int rows, H;
  int dh_fp32;
  int accumulate;       // 1: dh += result
};

struct RmsReduceArgs {  // acc[k] += sum over b of part[b][k], b in order
  const float* part;
  float* acc;
  int nblk, H;
};

hipError_t launch_logits(In in, const LogitsArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_dlogits(In in, const DlogitsArgs& a, hipStream_t s);
hipError_t launch_dx(In in, const DxArgs& a, hipStream_t s);
hipError_t launch_dx_reduce(const DxReduceArgs& a, hipStream_t s);
hipError_t launch_dw(In in, const DwArgs& a, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);
hipError_t launch_fused_block(const FusedBlockArgs& a, int grid, hipStream_t s);
hipError_t launch_fill_zero(const FillArgs& a, hipStream_t s);
hipError_t launch_cast_bf16(const CastArgs& a, hipStream_t s);
hipError_t launch_scale(const ScaleArgs& a, hipStream_t s);
hipError_t launch_rms_fwd(In in, const RmsFwdArgs& a, hipStream_t s);
hipError_t launch_rms_bwd(In in, const RmsBwdArgs& a, hipStream_t s);
hipError_t launch_rms_reduce(const RmsReduceArgs& a, hipStream_t s);

}  // namespace flce
