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

// Fused variant, pass 2.  The work is a grid of cells: one cell is a row of bm token tiles (bm x 256
// tokens) by one vocabulary tile.  A workgroup takes its cells in pieces: a piece is bm token tiles by
// at most bnmax consecutive vocabulary tiles of one row, whose logits it recomputes once, keeps as
// dlogits in its own bf16 buffer in the workspace, and then turns into whole dx and dW tiles (per
// 256-wide slice of H) added with one fp32 atomic per element.  A piece of bm x w tiles costs
// bm x w tile products of each kind and 16 (bm + w) atomic tile adds, so wide, tall pieces are cheap
// per tile.  Two ways of dealing the pieces:
//
// * blocks (BLOCKS): every piece is bm x bn (the last of a row narrower); workgroup L takes blocks
//   L, L + G, ... in groups of gm rows that sweep the vocabulary (a round of workgroups shares the
//   group's rows of x and of dx).  Used when the blocks fill the rounds of G workgroups (nearly)
//   exactly.
// * spans (SPANS): the workgroups' shares are made equal to within one cell, so that no round is
//   left partly filled.  The cells are ordered vocabulary super-range first, then row, then
//   vocabulary tile: super-range s holds tiles [s ws, (s + 1) ws) of every row, ws = ceil(tv / S),
//   and the segment (s, r) is its part of row r.  With at least as many workgroups as segments,
//   consecutive workgroups split each segment into near-equal runs; with fewer, each takes whole
//   consecutive segments.  A run is cut into ceil(n / bnmax) near-equal pieces.  Consecutive
//   logical workgroups sit on one XCD, so an XCD works on one super-range of every row.
struct SpanPlan {
  int blocks;  // 1: blocks of bm x bnmax tiles in groups of gm rows; 0: spans
  int R;       // rows of cells (token blocks)
  int tv;      // vocabulary tiles
  int S;       // vocabulary super-ranges (spans)
  int gm;      // rows per group (blocks)
  int G;       // workgroups
  int bnmax;   // widest piece, in vocabulary tiles (blocks: the block width)
};

__host__ __device__ inline int span_ws(const SpanPlan& sp) { return (sp.tv + sp.S - 1) / sp.S; }
__host__ __device__ inline int span_seg_width(const SpanPlan& sp, int i) {
  const int ws = span_ws(sp), s = i / sp.R;
  const int hi = (s + 1) * ws < sp.tv ? (s + 1) * ws : sp.tv;
  return hi - s * ws;
}

// Super-ranges for tv vocabulary tiles: up to 8 (one per XCD), none of them empty.
__host__ __device__ inline int span_supers(int tv) {
  int S = tv < 8 ? tv : 8;
  while (S > 1 && (S - 1) * ((tv + S - 1) / S) >= tv) --S;
  return S < 1 ? 1 : S;
}

// Piece k (0, 1, ...) of logical workgroup L: its row, first vocabulary tile and width in tiles;
// false once L has no more pieces.  A function of (L, k) alone, so that a kernel carries only k from
// one piece to the next.
__host__ __device__ inline bool span_piece(const SpanPlan& sp, int L, int k, int& row, int& vt0, int& nvt) {
  if (sp.blocks) {
    const int bn_count = (sp.tv + sp.bnmax - 1) / sp.bnmax;
    const int blk = L + k * sp.G;
    if (blk >= sp.R * bn_count) return false;
    // groups of gm rows (the last group shorter); rows fastest inside a group
    const int per_group = sp.gm * bn_count;
    const int g = blk / per_group, first = g * sp.gm;
    const int rows = sp.R - first < sp.gm ? sp.R - first : sp.gm;
    const int r = blk - g * per_group;
    row = first + r % rows;
    vt0 = (r / rows) * sp.bnmax;
    nvt = sp.tv - vt0 < sp.bnmax ? sp.tv - vt0 : sp.bnmax;
    return true;
  }
  const int NS = sp.S * sp.R;
  int i, i_end, k0, k1;
  if (sp.G >= NS) {   // one run: the workgroup's part of one segment
    i = (int)((int64_t)L * NS / sp.G);
    const int first = (int)(((int64_t)i * sp.G + NS - 1) / NS);
    const int next = (int)(((int64_t)(i + 1) * sp.G + NS - 1) / NS);
    const int q = next - first, w = span_seg_width(sp, i);
    i_end = i + 1;
    k0 = (int)((int64_t)(L - first) * w / q);
    k1 = (int)((int64_t)(L - first + 1) * w / q);
  } else {            // whole segments
    i = (int)((int64_t)L * NS / sp.G);
    i_end = (int)((int64_t)(L + 1) * NS / sp.G);
    k0 = 0;
    k1 = i < i_end ? span_seg_width(sp, i) : 0;
  }
  while (i < i_end) {
    const int n = k1 - k0;
    const int p = (n + sp.bnmax - 1) / sp.bnmax;
    if (k < p) {
      const int a = (int)((int64_t)n * k / p), b = (int)((int64_t)n * (k + 1) / p);
      row = i % sp.R;
      vt0 = (i / sp.R) * span_ws(sp) + k0 + a;
      nvt = b - a;
      return true;
    }
    k -= p;
    if (++i < i_end) {
      k0 = 0;
      k1 = span_seg_width(sp, i);
    }
  }
  return false;
}

constexpr int kFusedPieceTiles = 48;   // bm x bnmax tiles of bf16 dlogits per workgroup: 6 MiB
constexpr int kFusedMaxGrid = 256;     // resident workgroups (one per compute unit)

struct FusedBlockArgs {
  const void* x;        // first token row of the launch [rows][H] (bf16)
  const void* W;        // [V][H] (bf16)
  const int64_t* t;     // targets of those rows [rows]
  const float* lse;     // their log-sum-exp [rows]
  float* dx_acc;        // fp32 [rows][H], cleared (or holding the values to add to) before the launch
  float* dw_acc;        // fp32 [V][H], cleared before the first launch of a call
  char* gbuf;           // [gridDim.x][gstride]: each workgroup's dlogits piece (bf16, gld per row)
  int64_t gstride;      // bytes per workgroup: bm 256 rows of gld elements
  int gld;              // elements per row of a dlogits piece: bnmax 256
  int rows, H, V;
  int tiles_h;
  int bm;               // token tiles per row of cells
  SpanPlan span;        // span.G == gridDim.x
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
