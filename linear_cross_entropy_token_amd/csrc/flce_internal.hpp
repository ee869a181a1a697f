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

// Fused variant, pass 2.  The (token x vocabulary) plane of a launch is cut into blocks of bt x bv
// tiles (planned per launch, at most 1536 tiles), taken row by row (token blocks outer) in steps of
// up to `slots` blocks.  Per step, two kernels:
//   Z: recompute every logits tile of the step's blocks and store it as bf16 dlogits in the block's
//      slot buffer (bt 256 rows x bv 256 columns);
//   P: form the blocks' dx tiles (slot rows times W, contraction over the block's vocabulary ids)
//      and dW tiles (slot columns times x, contraction over its tokens) for every 256-wide slice of
//      H and add each into the fp32 accumulators with one atomic per element.
// Every dx / dW element thus receives one atomic per vocabulary / token block.  In both kernels the
// workgroups form `groups` groups of `gsize` (one group per XCD: consecutive logical workgroups sit
// on one XCD); group g takes the step's blocks g, g + groups, ... and its workgroups deal each
// block's items round-robin, so that a group works on one block at a time and its L2 shares that
// block's dlogits and operand strips.
struct StepPlan {
  int tm, tv;         // token and vocabulary tiles of the launch
  int bt, bv;         // block shape in tiles
  int blocks_v;       // vocabulary blocks per token block: ceil(tv / bv)
  int first, count;   // the step's blocks: first (global index) .. first + count - 1
  int groups, gsize;  // workgroup groups and their size (groups * gsize = gridDim.x)
  int th;             // 256-wide slices of H
};

// Row-major grid of TM x TN items dealt in groups of gm rows, rows fastest inside a group (the
// tile order that lets consecutive items share operand strips).
__host__ __device__ inline void grid_item(int q, int TM, int TN, int gm, int& m, int& n) {
  const int per_group = gm * TN;
  const int g = q / per_group, first = g * gm;
  const int rows = TM - first < gm ? TM - first : gm;
  const int r = q - g * per_group;
  m = first + r % rows;
  n = r / rows;
}

// Block j (0 .. count - 1) of the step: its first token tile, first vocabulary tile, and extents.
__host__ __device__ inline void step_block(const StepPlan& sp, int j, int& mt0, int& vt0, int& nt, int& nv) {
  const int b = sp.first + j;
  const int r = b / sp.blocks_v, c = b - r * sp.blocks_v;
  mt0 = r * sp.bt;
  vt0 = c * sp.bv;
  nt = sp.tm - mt0 < sp.bt ? sp.tm - mt0 : sp.bt;
  nv = sp.tv - vt0 < sp.bv ? sp.tv - vt0 : sp.bv;
}

// Items of a block in each kernel: Z, its logits tiles; P, its dx and dW tile products.
__host__ __device__ inline int z_items(int nt, int nv) { return nt * nv; }
__host__ __device__ inline int p_items(const StepPlan& sp, int nt, int nv) { return (nt + nv) * sp.th; }

// Walks the items of workgroup (group g, position w): calls f(j, q) for block j's item q.
template <bool PRODUCTS, class F>
__host__ __device__ inline void step_items(const StepPlan& sp, int g, int w, F&& f) {
  int seen = 0;   // items of the group's earlier blocks
  for (int j = g; j < sp.count; j += sp.groups) {
    int mt0, vt0, nt, nv;
    step_block(sp, j, mt0, vt0, nt, nv);
    const int n = PRODUCTS ? p_items(sp, nt, nv) : z_items(nt, nv);
    int q = (w - seen) % sp.gsize;
    if (q < 0) q += sp.gsize;
    for (; q < n; q += sp.gsize) f(j, q);
    seen += n;
  }
}

constexpr int64_t kFusedSlotBudget = (int64_t)3 << 29;   // 1.5 GiB of dlogits slots per step
constexpr int kFusedGrid = 256;        // workgroups of each pass-2 kernel
constexpr int kFusedOwnedMaxTiles = 64;   // bf16 dW: token tiles per pass-2 launch (one token block, 16,384 tokens)

struct FusedStepArgs {
  const void* x;        // first token row of the launch [rows][H] (bf16)
  const void* W;        // [V][H] (bf16)
  const int64_t* t;     // targets of those rows [rows]
  const float* lse;     // their log-sum-exp [rows]
  float* dx_acc;        // fp32 [rows][H], cleared (or holding the values to add to) before the first step
  float* dw_acc;        // fp32 [V][H], cleared before the first launch of a call (dw_owned == 0)
  void* dw_out;         // dw_owned: dW itself [V][H] (bf16), stored (dw_add: added) by its one product
  int dw_owned;         // 1: one token block covers the launch, so each dW tile has one product: no atomics
  int dw_add;           // dw_owned: add into dW instead of overwriting it
  char* slots;          // [count][slot_bytes]: the step's dlogits blocks (bf16, bv 256 per row)
  int64_t slot_bytes;
  int rows, H, V;
  StepPlan sp;
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
hipError_t launch_fused_step(const FusedStepArgs& a, hipStream_t s);   // the step's Z then P kernel
hipError_t launch_fill_zero(const FillArgs& a, hipStream_t s);
hipError_t launch_cast_bf16(const CastArgs& a, hipStream_t s);
hipError_t launch_scale(const ScaleArgs& a, hipStream_t s);
hipError_t launch_rms_fwd(In in, const RmsFwdArgs& a, hipStream_t s);
hipError_t launch_rms_bwd(In in, const RmsBwdArgs& a, hipStream_t s);
hipError_t launch_rms_reduce(const RmsReduceArgs& a, hipStream_t s);

}  // namespace flce
