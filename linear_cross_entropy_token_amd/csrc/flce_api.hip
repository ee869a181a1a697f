// C-ABI dispatcher of the FLCE library: validation, chunk plan, workspace,
// and the launch sequence on the caller's stream.
//
// The loop is the token-chunk loop of the core-idea section of the "Fused
// Linear Cross-Entropy" page (42jerrykim.github.io): for each chunk of C
// tokens, project, turn the logits buffer into dlogits in place, produce dx
// rows, accumulate dW; the loss and both gradients carry 1/N for the global
// token count (with options: 1 / the count of tokens not ignored, or 1 for a
// sum, counted on the device).  Unlike that page's listing, nothing
// synchronises the host inside the loop: the per-token losses stay on the
// device and one final kernel reduces them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <new>
#include <vector>

#include "flce.h"
#include "flce_internal.hpp"

namespace {

using flce::In;

constexpr int64_t kTile = flce::kTileM;
constexpr size_t kAlign = 256;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int64_t N = 0, H = 0, V = 0, C = 0, Vp = 0;
  int tiles_v = 0, tiles_h = 0;
  int splits = 1;
  int64_t k_per_split = 0;
  size_t off_z = 0, off_pm = 0, off_ps = 0, off_zt = 0, off_lse = 0, off_loss = 0, off_part = 0;
  size_t off_dxacc = 0;                  // fused variant: fp32 dx accumulator of a chunk for bf16 dx
  size_t off_gbuf = 0;                   // fused variant: the workgroups' dlogits block buffers
  int fused_bt = 0, fused_bv = 0;        // fused variant: pass-2 block shape in tiles (tokens, vocabulary)
  int fused_slots = 0;                   // fused variant: dlogits block slots (blocks per pass-2 step)
  int64_t fused_slot_bytes = 0;          // fused variant: bytes per slot
  bool fused_all = false;                // fused variant: one pass 2 over all N (fp32 dx) instead of per chunk
  bool fused_dw_owned = false;           // fused variant: bf16 dW stored by its one product per chunk (no accumulator)
  size_t off_scale = 0;                  // flce::Scale of the call
  size_t off_xc = 0, off_dxc = 0, off_rstd = 0, off_rpart = 0, off_dgacc = 0;   // RMSNorm path
  bool fused = false;
  bool grads = true;                     // false: forward only (no logits buffer, no accumulators)
  size_t total = 0;
};

// Per-call options in the form the launch sequence uses.
struct Opts {
  flce::Ignore ign{0, 0};
  int sum = 0;
  bool accumulate = false;
  bool grads = true;
};

}  // namespace

namespace {

enum Kernel {
  K_LOGITS = 0, K_COMBINE, K_DLOGITS, K_DX, K_DX_REDUCE, K_DW, K_FINALIZE, K_FUSED_BWD, K_FILL, K_CAST,
  K_SCALE, K_RMS_FWD, K_RMS_BWD, K_RMS_REDUCE, K_COUNT
};
const char* const kKernelNames[K_COUNT] = {"logits_lse", "lse_combine", "dlogits", "dx", "dx_reduce",
                                           "dw", "finalize", "fused_bwd", "fill_zero", "cast_bf16",
                                           "scale", "rms_fwd", "rms_bwd", "rms_reduce"};

struct Mark {
  int kind;                 // Kernel, or -1 for the event that closes a call
  hipEvent_t ev;
  double flops, bytes;
};

struct Stat {
  int64_t launches = 0;
  double ms = 0, flops = 0, bytes = 0;
};

}  // namespace

struct flce_handle_s {
  flce_config_t cfg;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  int* flag = nullptr;      // device int (16 bytes allocated), bit 0 = out-of-range target seen
  bool flag_ready = false;  // the flag has been cleared by a kernel on a caller's stream
  bool ws_pinned = false;   // a call was captured into a graph: the workspace may no longer move
  bool clk_reset = false;   // the clock counters are cleared before the next profiled launch
  bool profiling = false;
  unsigned long long* clk = nullptr;   // device [K_COUNT][2]: GEMM workgroup lifetimes (shader, 100 MHz ticks)
  std::vector<Mark> marks;  // pending events, in stream order
  std::vector<hipEvent_t> pool;
  Stat stats[K_COUNT];
};

namespace {

struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) {
      err = hipSetDevice(dev);
      changed = err == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

// What one call runs with: its handle, the device memory it works in (the handle's workspace, or
// the no-allocation scratch), the data flag it raises, and whether it is traced.
struct Exec {
  flce_handle_s* h;
  char* ws;
  int* flag;
  bool prof;
};

// The device clock counters of a GEMM kernel kind while profiling, else null.
unsigned long long* clock_of(const Exec& e, int kind) {
  return e.prof && e.h->clk != nullptr ? e.h->clk + 2 * kind : nullptr;
}

// Records a profiling event before a launch of `kind` (or kind -1 after the last launch).
hipError_t mark(const Exec& e, int kind, double flops, double bytes, hipStream_t st) {
  if (!e.prof) return hipSuccess;
  flce_handle_s* h = e.h;
  hipEvent_t ev;
  if (!h->pool.empty()) {
    ev = h->pool.back();
    h->pool.pop_back();
  } else {
    const hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) return e;
  }
  h->marks.push_back(Mark{kind, ev, flops, bytes});
  return hipEventRecord(ev, st);
}

hipError_t fold_marks(flce_handle_s* h) {
  hipError_t err = hipSuccess;
  for (size_t i = 0; i + 1 < h->marks.size(); ++i) {
    const Mark& m = h->marks[i];
    if (m.kind < 0) continue;
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(h->marks[i + 1].ev);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, m.ev, h->marks[i + 1].ev);
    if (e != hipSuccess) {
      err = e;
      continue;
    }
    Stat& s = h->stats[m.kind];
    s.launches += 1;
    s.ms += ms;
    s.flops += m.flops;
    s.bytes += m.bytes;
  }
  for (const Mark& m : h->marks) h->pool.push_back(m.ev);
  h->marks.clear();
  return err;
}

inline size_t in_size(const flce_config_t& c) { return c.in_dtype == FLCE_BF16 ? 2 : 4; }

bool sizes_ok(int64_t N, int64_t H, int64_t V) {
  return N >= 1 && H >= 1 && V >= 1;
}

flce_status_t sizes_supported(int64_t N, int64_t H, int64_t V) {
  if (H % 8 != 0) return FLCE_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 30;
  if (N > lim || H > lim || V > lim) return FLCE_ERR_UNSUPPORTED;
  return FLCE_OK;
}

int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Automatic chunk: the size rule of the FLCE page's trade-offs section (next power of two of
// N / ceil(V / H)), raised to 4096 tokens: on MI355X the per-chunk GEMMs run faster with the
// longer token contraction (dW) and the larger output (dx needs no split at 4096 x 4096), and
// below ~2048 tokens the per-chunk re-read of W dominates.  Capped at 8192 and so that the
// chunk's bf16/fp32 logits buffer stays within 1.5 GB.
int64_t effective_chunk(int64_t N, int64_t H, int64_t V, int64_t chunk, int64_t es) {
  if (!sizes_ok(N, H, V)) return 0;
  if (chunk > 0) return std::min(chunk, N);
  const int64_t inc = cdiv(V, H);
  int64_t c = next_pow2(cdiv(N, inc));
  c = std::max<int64_t>(c, 4096);
  c = std::min<int64_t>(c, 8192);
  const int64_t Vp = cdiv(V, kTile) * kTile;
  while (c > 256 && c * Vp * es > (int64_t)1500000000) c /= 2;
  return std::min(c, N);
}

// Pass 2 of the fused variant over tm token tiles and tv vocabulary tiles with blocks of bt x bv
// tiles: the slots of a step (as many blocks as 1.5 GiB holds, a multiple of the 8 workgroup groups
// when there are that many, so that every group (XCD) gets the same number of a step's blocks).
int64_t fused_slots_for(int64_t tm, int64_t tv, int bt, int bv) {
  const int64_t blocks = cdiv(tm, bt) * cdiv(tv, bv);
  int64_t slots = std::min<int64_t>(blocks, flce::kFusedSlotBudget / ((int64_t)bt * bv * kTile * kTile * 2));
  if (slots > 8) slots -= slots % 8;
  return std::max<int64_t>(1, slots);
}

// Relative time of pass 2 with blocks of bt x bv tiles: over the steps, the busiest group's blocks,
// each costing its tile pairs (one logits tile and its share of the dx and dW products) plus
// kAtomicWeight per tile of its two atomic streams.  The weight is fitted to the block shapes
// measured on the Llama-3, Qwen3, long-context and Llama-2 workloads (16 x 16, 32 x 16, 16 x 32,
// 32 x 32 and 24 x 24 tiles), whose pass-2 times it orders correctly.
constexpr double kAtomicWeight = 0.93;
double fused_cost(int64_t tm, int64_t tv, int bt, int bv, bool dw_owned) {
  const int64_t bvn = cdiv(tv, bv), nb = cdiv(tm, bt) * bvn, slots = fused_slots_for(tm, tv, bt, bv);
  double total = 0.0;
  for (int64_t first = 0; first < nb; first += slots) {
    const int64_t count = std::min(slots, nb - first);
    double worst = 0.0;
    for (int64_t g = 0; g < 8; ++g) {
      double w = 0.0;
      for (int64_t j = g; j < count; j += 8) {
        const int64_t b = first + j, r = b / bvn, c = b - r * bvn;
        const double nt = (double)std::min<int64_t>(bt, tm - r * bt), nv = (double)std::min<int64_t>(bv, tv - c * bv);
        w += nt * nv + kAtomicWeight * (dw_owned ? nt : nt + nv);
      }
      worst = std::max(worst, w);
    }
    total += worst;
  }
  return total;
}

// Block shape of pass 2: heights of 32, 16 or 8 token tiles (dw_owned: all tm of the launch, one
// token block), widths of 8 .. 48 vocabulary tiles (dw_owned: 1 .. 96), at most 1536 tiles (192 MiB
// of slot, so that a step holds at least 8 blocks); the cheapest under fused_cost, the larger block
// (fewer atomics) on a tie.
void fused_block_shape(int64_t tm, int64_t tv, bool dw_owned, int& bt, int& bv) {
  double best = 0.0;
  bt = bv = 0;
  for (const int h0 : {32, 16, 8}) {
    const int h = dw_owned ? (int)tm : (int)std::min<int64_t>(h0, tm);
    for (int w0 = dw_owned ? 96 : 48; w0 >= (dw_owned ? 1 : 8); --w0) {
      const int w = (int)std::min<int64_t>(w0, tv);
      if (h * w > 1536) continue;
      const double c = fused_cost(tm, tv, h, w, dw_owned);
      if (bt == 0 || c < best * (1.0 - 1e-9)) {
        best = c;
        bt = h;
        bv = w;
      }
    }
  }
}

// Whether the fused variant may run pass 2 once over all N tokens: dx in fp32 (dx is its own
// accumulator) and N rows of x and of dx within the kernels' 32-bit buffer offsets (make_plan also
// requires fp32 dW: bf16 dW takes pass 2 per chunk, one token block per launch).
bool fused_pass2_over_all(const flce_config_t& cfg, int64_t N, int64_t H) {
  const int64_t lim = (int64_t)0xFFFFFF00 - 4096;
  return cfg.dx_dtype == FLCE_FP32 && N * H * 2 < lim && (N + kTile) * H * 4 < lim;
}

Plan make_plan(const flce_config_t& cfg, int64_t N, int64_t H, int64_t V, int64_t chunk, bool grads = true,
               bool rms = false) {
  Plan p;
  p.N = N;
  p.H = H;
  p.V = V;
  p.C = effective_chunk(N, H, V, chunk, (int64_t)in_size(cfg));
  p.Vp = cdiv(V, kTile) * kTile;
  p.tiles_v = (int)(p.Vp / kTile);
  p.tiles_h = (int)cdiv(H, kTile);
  // dx = G W has only ceil(C/256) x ceil(H/256) output tiles: split the vocabulary contraction
  // into the fewest parts (at most 8, each at least 8 k-slices) whose tiles fill the rounds of
  // 256 compute units to at least 90% (e.g. 384 tiles, 1.5 rounds, become 768 in 3 rounds).
  const int64_t tiles_dx = cdiv(p.C, kTile) * p.tiles_h;
  const int64_t bk = flce::kSliceBytesABI / (int64_t)in_size(cfg);   // contraction elements per k-slice
  const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(8, p.Vp / (8 * bk)));
  int64_t s = 1;
  for (; s < smax; ++s) {
    const int64_t n = tiles_dx * s;
    if ((double)n >= 0.9 * (double)(cdiv(n, 256) * 256)) break;
  }
  p.splits = (int)s;
  p.k_per_split = cdiv(cdiv(p.Vp, s), bk) * bk;

  p.fused = cfg.variant == FLCE_FUSED;
  p.grads = grads;
  size_t off = 0;
  p.off_scale = off;
  off = align_up(off + sizeof(flce::Scale));
  p.off_z = off;
  if (!p.fused && grads) off = align_up(off + (size_t)p.C * p.Vp * in_size(cfg));
  p.off_pm = off;   off = align_up(off + (size_t)p.tiles_v * p.C * sizeof(float));
  p.off_ps = off;   off = align_up(off + (size_t)p.tiles_v * p.C * sizeof(float));
  p.off_zt = off;   off = align_up(off + (size_t)N * sizeof(float));
  p.off_lse = off;  off = align_up(off + (size_t)N * sizeof(float));
  p.off_loss = off; off = align_up(off + (size_t)N * sizeof(float));
  p.off_part = off;
  if (!p.fused && grads && p.splits > 1) off = align_up(off + (size_t)p.splits * p.C * H * sizeof(float));
  p.off_dxacc = off;
  if (p.fused && grads && cfg.dx_dtype == FLCE_BF16) off = align_up(off + (size_t)p.C * H * sizeof(float));
  // bf16 dW: pass 2 per chunk with one token block per launch, so that every dW tile has one product
  // per chunk and is stored (added, after the first chunk) into dW directly: no V x H fp32 accumulator
  p.fused_dw_owned = p.fused && grads && cfg.dw_dtype == FLCE_BF16;
  p.off_gbuf = off;
  if (p.fused && grads) {   // pass 2: dlogits block slots for one step (at most 1.5 GiB)
    p.fused_all = fused_pass2_over_all(cfg, N, H) && !p.fused_dw_owned;
    int64_t tm = cdiv(p.fused_all ? N : p.C, kTile);
    if (p.fused_dw_owned) tm = std::min<int64_t>(tm, flce::kFusedOwnedMaxTiles);   // launches of <= this many
    fused_block_shape(tm, p.tiles_v, p.fused_dw_owned, p.fused_bt, p.fused_bv);
    p.fused_slot_bytes = (int64_t)p.fused_bt * p.fused_bv * kTile * kTile * 2;
    p.fused_slots = (int)fused_slots_for(tm, p.tiles_v, p.fused_bt, p.fused_bv);
    off = align_up(off + (size_t)p.fused_slots * (size_t)p.fused_slot_bytes);
  }
  if (rms) {   // the chunk's normalised rows, their fp32 dL/dx, rstd, dgamma partials and sum
    p.off_xc = off;    off = align_up(off + (size_t)p.C * H * in_size(cfg));
    p.off_dxc = off;   if (grads) off = align_up(off + (size_t)p.C * H * sizeof(float));
    p.off_rstd = off;  off = align_up(off + (size_t)p.C * sizeof(float));
    p.off_rpart = off;
    if (grads) off = align_up(off + (size_t)cdiv(p.C, flce::kRmsRowsPerBlock) * H * sizeof(float));
    p.off_dgacc = off;
    if (grads && cfg.dw_dtype == FLCE_BF16) off = align_up(off + (size_t)H * sizeof(float));
  }
  p.total = off;
  return p;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte range [lo, hi) of one caller tensor; empty for a null pointer.
struct Span {
  uintptr_t lo = 0, hi = 0;
  Span(const void* p, int64_t bytes) {
    if (p != nullptr && bytes > 0) {
      lo = reinterpret_cast<uintptr_t>(p);
      hi = lo + (uintptr_t)bytes;
    }
  }
};
inline bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

// True when no output overlaps an input or another output: the kernels read inputs after
// outputs have been written (later chunks read x and W after earlier chunks wrote dx and dW).
bool outputs_disjoint(std::initializer_list<Span> in, std::initializer_list<Span> out) {
  for (auto o = out.begin(); o != out.end(); ++o) {
    for (const Span& i : in)
      if (overlap(*o, i)) return false;
    for (auto o2 = o + 1; o2 != out.end(); ++o2)
      if (overlap(*o, *o2)) return false;
  }
  return true;
}

// Allocates (or grows) the workspace and the data flag.  Nothing is enqueued on any stream: the
// flag is cleared by the next call's first kernel on the caller's stream (prepare_call).  Once a
// call has been captured into a graph the workspace is pinned, since the graph holds its address.
flce_status_t ensure_workspace(flce_handle_s* h, size_t need) {
  if (h->cfg.workspace_limit > 0 && need > (size_t)h->cfg.workspace_limit) return FLCE_ERR_OOM;
  DeviceGuard g(h->cfg.device);
  if (g.err != hipSuccess) return FLCE_ERR_HIP;
  if (h->flag == nullptr) {
    if (hipMalloc(reinterpret_cast<void**>(&h->flag), 16) != hipSuccess) {
      h->flag = nullptr;
      (void)hipGetLastError();
      return FLCE_ERR_OOM;
    }
    h->flag_ready = false;
  }
  if (need <= h->ws_bytes) return FLCE_OK;
  if (h->ws_pinned) return FLCE_ERR_UNSUPPORTED;
  void* p = nullptr;
  if (hipMalloc(&p, need) != hipSuccess) {
    (void)hipGetLastError();
    return FLCE_ERR_OOM;
  }
  if (h->ws != nullptr) (void)hipFree(h->ws);
  h->ws = p;
  h->ws_bytes = need;
  return FLCE_OK;
}

// The kernels address each operand through a 32-bit buffer range: W, one chunk of x and the
// chunk's logits buffer must each stay below 4 GiB (minus a guard band used for masked lanes).
flce_status_t validate_sizes(const flce_config_t& cfg, int64_t N, int64_t H, int64_t V, int64_t chunk) {
  if (!sizes_ok(N, H, V)) return FLCE_ERR_INVALID_ARG;
  const flce_status_t st = sizes_supported(N, H, V);
  if (st != FLCE_OK) return st;
  const int64_t lim = (int64_t)0xFFFFFF00 - 4096;
  const int64_t es = (int64_t)in_size(cfg);
  const int64_t C = effective_chunk(N, H, V, chunk, es);
  const int64_t Vp = cdiv(V, kTile) * kTile;
  if (V * H * es >= lim || C * H * es >= lim || C * Vp * es >= lim) return FLCE_ERR_UNSUPPORTED;
  // the fused variant adds into fp32 accumulators ([C, H] per chunk and [V, H]) through 32-bit
  // buffer offsets, with up to one tile of rows past the end
  if (cfg.variant == FLCE_FUSED && ((V + kTile) * H * 4 >= lim || (C + kTile) * H * 4 >= lim))
    return FLCE_ERR_UNSUPPORTED;
  return FLCE_OK;
}

#define FLCE_LAUNCH(call)                         \
  do {                                            \
    if ((call) != hipSuccess) return FLCE_ERR_HIP; \
  } while (0)

// Checks a call against graph capture before anything is enqueued: under capture nothing may be
// allocated, so the workspace (and flag) must already hold the plan; the workspace is then pinned
// for the handle's lifetime.  Call before ensure_workspace.
flce_status_t capture_check(flce_handle_s* h, size_t need, hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return FLCE_ERR_HIP;
  }
  if (cs == hipStreamCaptureStatusNone) return FLCE_OK;
  if (h->flag == nullptr || h->ws == nullptr || need > h->ws_bytes) return FLCE_ERR_UNSUPPORTED;
  h->ws_pinned = true;
  return FLCE_OK;
}

// First kernels of a call, on its stream: clear the data flag after its allocation and the clock
// counters after profiling was (re-)enabled.
flce_status_t prepare_call(flce_handle_s* h, hipStream_t st) {
  if (!h->flag_ready) {
    flce::FillArgs z{reinterpret_cast<float*>(h->flag), 4};
    FLCE_LAUNCH(flce::launch_fill_zero(z, st));
    h->flag_ready = true;
  }
  if (h->profiling && h->clk_reset && h->clk != nullptr) {
    flce::FillArgs z{reinterpret_cast<float*>(h->clk), (int64_t)(2 * K_COUNT * sizeof(unsigned long long) / 4)};
    FLCE_LAUNCH(flce::launch_fill_zero(z, st));
    h->clk_reset = false;
  }
  return FLCE_OK;
}

// Token count and normalisation of the call, on the device (no host synchronisation).
flce_status_t launch_scale(const Exec& e, const Plan& p, const Opts& o, const int64_t* t, hipStream_t st) {
  flce::ScaleArgs sa{};
  sa.t = t;
  sa.n = p.N;
  sa.ign = o.ign;
  sa.sum = o.sum;
  sa.out = reinterpret_cast<flce::Scale*>(e.ws + p.off_scale);
  FLCE_LAUNCH(mark(e, K_SCALE, 0.0, 8.0 * p.N, st));
  FLCE_LAUNCH(flce::launch_scale(sa, st));
  return FLCE_OK;
}

// Where one chunk's dx rows go.
struct DxOut {
  void* p;          // chunk's first row
  bool fp32;
  bool accumulate;
};

// One chunk of the token-chunked path: logits + statistics, combine, and (with gradients)
// dlogits, dx rows of the chunk, dW update.  x_c: the chunk's first row of x.
flce_status_t chunk_flce(const Exec& e, const Plan& p, const Opts& o, int64_t s, int rows, const void* x_c,
                         const void* W, const int64_t* t, float* lse, const DxOut& dxo, void* dW, hipStream_t st) {
  const flce_config_t& cfg = e.h->cfg;
  const In in = cfg.in_dtype == FLCE_BF16 ? In::BF16 : In::FP32;
  const size_t es = in_size(cfg);
  char* ws = e.ws;
  void* z = ws + p.off_z;
  float* pm = reinterpret_cast<float*>(ws + p.off_pm);
  float* ps = reinterpret_cast<float*>(ws + p.off_ps);
  float* zt = reinterpret_cast<float*>(ws + p.off_zt);
  float* loss_rows = reinterpret_cast<float*>(ws + p.off_loss);
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  const flce::Scale* scale = reinterpret_cast<const flce::Scale*>(ws + p.off_scale);
  const double b_in = (double)es, b_dx = dxo.fp32 ? 4.0 : 2.0;
  const double b_dw = cfg.dw_dtype == FLCE_BF16 ? 2.0 : 4.0;
  const double VH = (double)p.V * (double)p.H;
  const int tiles_m = (int)cdiv(rows, kTile);
  const double gemm_flops = 2.0 * rows * VH;
  const double zbytes = o.grads ? (double)rows * (double)p.V * b_in : 0.0;

  flce::LogitsArgs la{};
  la.x = x_c;
  la.W = W;
  la.t = t + s;
  la.z = o.grads ? z : nullptr;   // forward only: statistics, no logits buffer
  la.pm = pm;
  la.ps = ps;
  la.zt = zt + s;
  la.ldz = p.Vp;
  la.pstride = (int)p.C;
  la.rows = rows;
  la.H = (int)p.H;
  la.V = (int)p.V;
  la.tiles_m = tiles_m;
  la.tiles_n = p.tiles_v;
  la.clk = clock_of(e, K_LOGITS);
  FLCE_LAUNCH(mark(e, K_LOGITS, gemm_flops, (double)rows * p.H * b_in + VH * b_in + zbytes, st));
  FLCE_LAUNCH(flce::launch_logits(in, la, st));

  flce::CombineArgs ca{};
  ca.pm = pm;
  ca.ps = ps;
  ca.zt = zt + s;
  ca.t = t + s;
  ca.lse = lse + s;
  ca.loss_rows = loss_rows + s;
  ca.flag = e.flag;
  ca.ign = o.ign;
  ca.pstride = (int)p.C;
  ca.tiles_n = p.tiles_v;
  ca.rows = rows;
  ca.V = (int)p.V;
  FLCE_LAUNCH(mark(e, K_COMBINE, 0.0, 8.0 * rows * p.tiles_v + 16.0 * rows, st));
  FLCE_LAUNCH(flce::launch_combine(ca, st));
  if (!o.grads) return FLCE_OK;

  flce::DlogitsArgs ga{};
  ga.z = z;
  ga.pm = pm;
  ga.pstride = (int)p.C;
  ga.lse = lse + s;
  ga.t = t + s;
  ga.ldz = p.Vp;
  ga.rows = rows;
  ga.V = (int)p.V;
  ga.ign = o.ign;
  ga.scale = scale;
  FLCE_LAUNCH(mark(e, K_DLOGITS, 0.0, 2.0 * zbytes + 4.0 * rows * p.tiles_v, st));
  FLCE_LAUNCH(flce::launch_dlogits(in, ga, st));

  flce::DxArgs xa{};
  xa.g = z;
  xa.W = W;
  xa.part = part;
  xa.dx = dxo.p;
  xa.ldg = p.Vp;
  xa.part_stride = p.C * p.H;
  xa.rows = rows;
  xa.H = (int)p.H;
  xa.V = (int)p.V;
  xa.k_per_split = (int)p.k_per_split;
  xa.splits = p.splits;
  xa.tiles_m = tiles_m;
  xa.tiles_n = p.tiles_h;
  xa.dx_fp32 = dxo.fp32;
  xa.accumulate = dxo.accumulate;
  xa.clk = clock_of(e, K_DX);
  FLCE_LAUNCH(mark(e, K_DX, gemm_flops, zbytes + VH * b_in + (double)rows * p.H * b_dx, st));
  FLCE_LAUNCH(flce::launch_dx(in, xa, st));
  if (p.splits > 1) {
    flce::DxReduceArgs ra{};
    ra.part = part;
    ra.dx = xa.dx;
    ra.part_stride = xa.part_stride;
    ra.count = (int64_t)rows * p.H;
    ra.splits = p.splits;
    ra.dx_fp32 = xa.dx_fp32;
    ra.accumulate = xa.accumulate;
    FLCE_LAUNCH(mark(e, K_DX_REDUCE, 0.0, (double)rows * p.H * (4.0 * p.splits + b_dx), st));
    FLCE_LAUNCH(flce::launch_dx_reduce(ra, st));
  }

  flce::DwArgs wa{};
  wa.g = z;
  wa.x = x_c;
  wa.dW = dW;
  wa.ldg = p.Vp;
  wa.rows = rows;
  wa.H = (int)p.H;
  wa.V = (int)p.V;
  wa.tiles_m = p.tiles_v;
  wa.tiles_n = p.tiles_h;
  wa.dw_fp32 = cfg.dw_dtype == FLCE_FP32;
  wa.accumulate = s > 0 || o.accumulate;
  wa.clk = clock_of(e, K_DW);
  FLCE_LAUNCH(mark(e, K_DW, gemm_flops,
                   zbytes + (double)rows * p.H * b_in + VH * b_dw * (wa.accumulate ? 2.0 : 1.0), st));
  FLCE_LAUNCH(flce::launch_dw(in, wa, st));
  return FLCE_OK;
}

flce_status_t finalize_loss(const Exec& e, const Plan& p, float* loss, hipStream_t st) {
  char* ws = e.ws;
  flce::FinalizeArgs fa{};
  fa.loss_rows = reinterpret_cast<float*>(ws + p.off_loss);
  fa.loss = loss;
  fa.n = p.N;
  fa.scale = reinterpret_cast<const flce::Scale*>(ws + p.off_scale);
  FLCE_LAUNCH(mark(e, K_FINALIZE, 0.0, 4.0 * p.N + 4.0, st));
  FLCE_LAUNCH(flce::launch_finalize(fa, st));
  return FLCE_OK;
}

flce_status_t run_chunked(const Exec& e, const Plan& p, const Opts& o, const void* x, const void* W,
                          const int64_t* t, float* loss, void* dx, void* dW, float* lse_out,
                          hipStream_t st) {
  const flce_config_t& cfg = e.h->cfg;
  const size_t es = in_size(cfg);
  const size_t dx_es = cfg.dx_dtype == FLCE_BF16 ? 2 : 4;
  float* lse = lse_out != nullptr ? lse_out : reinterpret_cast<float*>(e.ws + p.off_lse);
  flce_status_t r = launch_scale(e, p, o, t, st);
  if (r != FLCE_OK) return r;
  for (int64_t s = 0; s < p.N; s += p.C) {
    const int rows = (int)std::min(p.C, p.N - s);
    const DxOut dxo{o.grads ? static_cast<char*>(dx) + (size_t)s * p.H * dx_es : nullptr,
                    cfg.dx_dtype == FLCE_FP32, o.accumulate};
    r = chunk_flce(e, p, o, s, rows, static_cast<const char*>(x) + (size_t)s * p.H * es, W, t, lse, dxo, dW, st);
    if (r != FLCE_OK) return r;
  }
  r = finalize_loss(e, p, loss, st);
  if (r != FLCE_OK) return r;
  FLCE_LAUNCH(mark(e, -1, 0.0, 0.0, st));
  return FLCE_OK;
}

// RMSNorm in front of the head, per chunk: x_c = rmsnorm(h_c) into the workspace, the FLCE
// chunk with its dx rows in an fp32 workspace buffer, then dh rows and dgamma partials from
// them; dgamma is summed in fp32 across chunks and written (or added) in its dtype at the end.
flce_status_t run_rmsnorm(const Exec& e, const Plan& p, const Opts& o, const void* hid, const void* gamma,
                          float eps, const void* W, const int64_t* t, float* loss, void* dh, void* dgamma,
                          void* dW, float* lse_out, hipStream_t st) {
  const flce_config_t& cfg = e.h->cfg;
  const In in = cfg.in_dtype == FLCE_BF16 ? In::BF16 : In::FP32;
  const size_t es = in_size(cfg);
  const size_t dh_es = cfg.dx_dtype == FLCE_BF16 ? 2 : 4;
  char* ws = e.ws;
  float* lse = lse_out != nullptr ? lse_out : reinterpret_cast<float*>(ws + p.off_lse);
  void* xc = ws + p.off_xc;
  float* dxc = reinterpret_cast<float*>(ws + p.off_dxc);
  float* rstd = reinterpret_cast<float*>(ws + p.off_rstd);
  float* rpart = reinterpret_cast<float*>(ws + p.off_rpart);
  const bool dg32 = cfg.dw_dtype == FLCE_FP32;
  float* dg_acc = dg32 ? static_cast<float*>(dgamma) : reinterpret_cast<float*>(ws + p.off_dgacc);
  const double H = (double)p.H;
  flce_status_t r = launch_scale(e, p, o, t, st);
  if (r != FLCE_OK) return r;
  if (o.grads && !(dg32 && o.accumulate)) {   // fp32 dgamma is its own accumulator
    flce::FillArgs zg{dg_acc, p.H};
    FLCE_LAUNCH(mark(e, K_FILL, 0.0, 4.0 * H, st));
    FLCE_LAUNCH(flce::launch_fill_zero(zg, st));
  }
  for (int64_t s = 0; s < p.N; s += p.C) {
    const int rows = (int)std::min(p.C, p.N - s);
    const void* hc = static_cast<const char*>(hid) + (size_t)s * p.H * es;
    flce::RmsFwdArgs fa{hc, gamma, xc, rstd, rows, (int)p.H, eps};
    FLCE_LAUNCH(mark(e, K_RMS_FWD, 0.0, (2.0 * rows + 1.0) * H * (double)es + 4.0 * rows, st));
    FLCE_LAUNCH(flce::launch_rms_fwd(in, fa, st));
    r = chunk_flce(e, p, o, s, rows, xc, W, t, lse, DxOut{dxc, true, false}, dW, st);
    if (r != FLCE_OK) return r;
    if (!o.grads) continue;
    const int nblk = (int)cdiv(rows, flce::kRmsRowsPerBlock);
    flce::RmsBwdArgs ba{dxc, hc, gamma, rstd, static_cast<char*>(dh) + (size_t)s * p.H * dh_es, rpart,
                        rows, (int)p.H, cfg.dx_dtype == FLCE_FP32, o.accumulate};
    FLCE_LAUNCH(mark(e, K_RMS_BWD, 0.0, rows * H * (4.0 + (double)es + (double)dh_es) + nblk * H * 4.0, st));
    FLCE_LAUNCH(flce::launch_rms_bwd(in, ba, st));
    flce::RmsReduceArgs ra{rpart, dg_acc, nblk, (int)p.H};
    FLCE_LAUNCH(mark(e, K_RMS_REDUCE, 0.0, (nblk + 2.0) * H * 4.0, st));
    FLCE_LAUNCH(flce::launch_rms_reduce(ra, st));
  }
  if (o.grads && !dg32) {
    flce::CastArgs cg{dg_acc, dgamma, p.H, o.accumulate};
    FLCE_LAUNCH(mark(e, K_CAST, 0.0, 6.0 * H, st));
    FLCE_LAUNCH(flce::launch_cast_bf16(cg, st));
  }
  r = finalize_loss(e, p, loss, st);
  if (r != FLCE_OK) return r;
  FLCE_LAUNCH(mark(e, -1, 0.0, 0.0, st));
  return FLCE_OK;
}

// Pass 2 of the fused variant over `rows` tokens starting at token s: the (token x vocabulary)
// plane in blocks of the plan's shape, in steps of up to fused_slots blocks, each step a Z kernel
// (dlogits of its blocks into the slots) and a P kernel (dx and dW tile products from the slots,
// added into dx_acc (rows x H, fp32) with atomics, and into dw_acc (V x H, fp32) with atomics or,
// with one token block per launch (fused_dw_owned), stored into dW).  A launch over fewer tokens than
// the plan's (the last chunk) has fewer blocks of the same shape.
flce_status_t launch_pass2(const Exec& e, const Plan& p, const Opts& o, int64_t s, int64_t rows, const void* x,
                           const void* W, const int64_t* t, const float* lse, float* dx_acc, float* dw_acc,
                           void* dW, hipStream_t st) {
  const double VH = (double)p.V * (double)p.H;
  flce::FusedStepArgs fa{};
  fa.x = static_cast<const char*>(x) + (size_t)s * p.H * 2;
  fa.W = W;
  fa.t = t + s;
  fa.lse = lse + s;
  fa.dx_acc = dx_acc;
  fa.dw_acc = dw_acc;
  fa.dw_out = dW;
  fa.dw_owned = p.fused_dw_owned ? 1 : 0;
  fa.dw_add = (s > 0 || o.accumulate) ? 1 : 0;   // dw_owned: the first chunk overwrites dW
  fa.slots = e.ws + p.off_gbuf;
  fa.slot_bytes = p.fused_slot_bytes;
  fa.rows = (int)rows;
  fa.H = (int)p.H;
  fa.V = (int)p.V;
  fa.ign = o.ign;
  fa.scale = reinterpret_cast<const flce::Scale*>(e.ws + p.off_scale);
  flce::StepPlan& sp = fa.sp;
  sp.tm = (int)cdiv(rows, kTile);
  sp.tv = p.tiles_v;
  sp.bt = p.fused_bt;
  sp.bv = p.fused_bv;
  sp.blocks_v = (int)cdiv(sp.tv, sp.bv);
  sp.groups = 8;   // one group per XCD
  sp.gsize = flce::kFusedGrid / sp.groups;
  sp.th = p.tiles_h;
  const int blocks = (int)cdiv(sp.tm, sp.bt) * sp.blocks_v;
  // recompute (2 rows V H) + dx partials (2 rows V H) + dW partials (2 rows V H), all steps
  FLCE_LAUNCH(mark(e, K_FUSED_BWD, 6.0 * (double)rows * VH, 2.0 * ((double)rows * p.H * 2 + VH * 2), st));
  for (int first = 0; first < blocks; first += p.fused_slots) {
    sp.first = first;
    sp.count = std::min(p.fused_slots, blocks - first);
    FLCE_LAUNCH(flce::launch_fused_step(fa, st));
  }
  return FLCE_OK;
}

// Fused variant: per chunk, pass 1 (logits statistics only, no logits store) and the combine into
// each token's lse; pass 2 (recompute, dlogits per block, dx and dW by fp32 atomics) once over all
// tokens when dx is fp32 (dx is then its own accumulator, and one launch has the most blocks),
// else per chunk into an fp32 chunk accumulator cast to bf16 after it; outputs converted last.
flce_status_t run_fused(const Exec& e, const Plan& p, const Opts& o, const void* x, const void* W,
                        const int64_t* t, float* loss, void* dx, void* dW, float* lse_out, hipStream_t st) {
  const flce_config_t& cfg = e.h->cfg;
  char* ws = e.ws;
  float* pm = reinterpret_cast<float*>(ws + p.off_pm);
  float* ps = reinterpret_cast<float*>(ws + p.off_ps);
  float* zt = reinterpret_cast<float*>(ws + p.off_zt);
  float* lse = lse_out != nullptr ? lse_out : reinterpret_cast<float*>(ws + p.off_lse);
  float* loss_rows = reinterpret_cast<float*>(ws + p.off_loss);
  const bool dx32 = cfg.dx_dtype == FLCE_FP32, dw32 = cfg.dw_dtype == FLCE_FP32;
  // fp32 dW is its own atomic accumulator; bf16 dW is stored by its one product per chunk
  float* dw_acc = dw32 ? static_cast<float*>(dW) : nullptr;
  const flce::Scale* scale = reinterpret_cast<const flce::Scale*>(ws + p.off_scale);
  const double VH = (double)p.V * (double)p.H;
  const flce_status_t sc = launch_scale(e, p, o, t, st);
  if (sc != FLCE_OK) return sc;

  // fp32 outputs are the accumulators themselves: cleared unless the call accumulates into them
  if (o.grads && !p.fused_dw_owned && !o.accumulate) {
    flce::FillArgs zw{dw_acc, p.V * p.H};
    FLCE_LAUNCH(mark(e, K_FILL, 0.0, 4.0 * VH, st));
    FLCE_LAUNCH(flce::launch_fill_zero(zw, st));
  }
  if (o.grads && p.fused_all && !o.accumulate) {
    flce::FillArgs zx{static_cast<float*>(dx), p.N * p.H};
    FLCE_LAUNCH(mark(e, K_FILL, 0.0, 4.0 * (double)p.N * p.H, st));
    FLCE_LAUNCH(flce::launch_fill_zero(zx, st));
  }
  for (int64_t s = 0; s < p.N; s += p.C) {
    const int rows = (int)std::min(p.C, p.N - s);
    const int tiles_m = (int)cdiv(rows, kTile);
    const double gemm_flops = 2.0 * rows * VH;

    flce::LogitsArgs la{};
    la.x = static_cast<const char*>(x) + (size_t)s * p.H * 2;
    la.W = W;
    la.t = t + s;
    la.z = nullptr;
    la.pm = pm;
    la.ps = ps;
    la.zt = zt + s;
    la.ldz = p.Vp;
    la.pstride = (int)p.C;
    la.rows = rows;
    la.H = (int)p.H;
    la.V = (int)p.V;
    la.tiles_m = tiles_m;
    la.tiles_n = p.tiles_v;
    la.clk = clock_of(e, K_LOGITS);
    FLCE_LAUNCH(mark(e, K_LOGITS, gemm_flops, (double)rows * p.H * 2 + VH * 2, st));
    FLCE_LAUNCH(flce::launch_logits(In::BF16, la, st));

    flce::CombineArgs ca{};
    ca.pm = pm;
    ca.ps = ps;
    ca.zt = zt + s;
    ca.t = t + s;
    ca.lse = lse + s;
    ca.loss_rows = loss_rows + s;
    ca.flag = e.flag;
    ca.ign = o.ign;
    ca.pstride = (int)p.C;
    ca.tiles_n = p.tiles_v;
    ca.rows = rows;
    ca.V = (int)p.V;
    FLCE_LAUNCH(mark(e, K_COMBINE, 0.0, 8.0 * rows * p.tiles_v + 16.0 * rows, st));
    FLCE_LAUNCH(flce::launch_combine(ca, st));
    if (!o.grads || p.fused_all) continue;

    float* dx_acc = dx32 ? static_cast<float*>(dx) + (size_t)s * p.H : reinterpret_cast<float*>(ws + p.off_dxacc);
    if (!(dx32 && o.accumulate)) {
      flce::FillArgs zx{dx_acc, (int64_t)rows * p.H};
      FLCE_LAUNCH(mark(e, K_FILL, 0.0, 4.0 * rows * p.H, st));
      FLCE_LAUNCH(flce::launch_fill_zero(zx, st));
    }
    // with owned dW tiles a launch covers at most fused_bt token tiles (one token block): longer
    // chunks take several launches, each storing (adding, after the call's first) its dW tiles
    const int64_t span = p.fused_dw_owned ? (int64_t)p.fused_bt * kTile : (int64_t)rows;
    for (int64_t u = 0; u < rows; u += span) {
      const int64_t n = std::min<int64_t>(span, rows - u);
      const flce_status_t r = launch_pass2(e, p, o, s + u, n, x, W, t, lse, dx_acc + (size_t)u * p.H, dw_acc, dW, st);
      if (r != FLCE_OK) return r;
    }
    if (!dx32) {
      flce::CastArgs cx{dx_acc, static_cast<char*>(dx) + (size_t)s * p.H * 2, (int64_t)rows * p.H, o.accumulate};
      FLCE_LAUNCH(mark(e, K_CAST, 0.0, 6.0 * rows * p.H, st));
      FLCE_LAUNCH(flce::launch_cast_bf16(cx, st));
    }
  }
  if (o.grads && p.fused_all) {
    const flce_status_t r = launch_pass2(e, p, o, 0, p.N, x, W, t, lse, static_cast<float*>(dx), dw_acc, dW, st);
    if (r != FLCE_OK) return r;
  }
  flce::FinalizeArgs fa{};
  fa.loss_rows = loss_rows;
  fa.loss = loss;
  fa.n = p.N;
  fa.scale = scale;
  FLCE_LAUNCH(mark(e, K_FINALIZE, 0.0, 4.0 * p.N + 4.0, st));
  FLCE_LAUNCH(flce::launch_finalize(fa, st));
  FLCE_LAUNCH(mark(e, -1, 0.0, 0.0, st));
  return FLCE_OK;
}


// Options in launch form; false for malformed ones.
bool parse_options(const flce_options_t* opt, Opts& o) {
  if (opt == nullptr) return true;
  if ((opt->reduction != FLCE_MEAN && opt->reduction != FLCE_SUM) ||
      (opt->flags & ~(FLCE_ACCUMULATE | FLCE_FORWARD_ONLY)) != 0 ||
      ((opt->flags & FLCE_ACCUMULATE) && (opt->flags & FLCE_FORWARD_ONLY)) || opt->ignore_on < 0 ||
      opt->ignore_on > 1 || opt->reserved != 0)
    return false;
  o.sum = opt->reduction == FLCE_SUM;
  o.accumulate = (opt->flags & FLCE_ACCUMULATE) != 0;
  o.grads = (opt->flags & FLCE_FORWARD_ONLY) == 0;
  o.ign = flce::Ignore{opt->ignore_index, opt->ignore_on};
  return true;
}

// Largest H of the RMSNorm path: its backward keeps one fp32 dgamma row of H in LDS.
constexpr int64_t kRmsMaxH = 32768;

flce_status_t validate_rmsnorm(const flce_config_t& cfg, int64_t H, float eps) {
  if (!(eps >= 0.f) || eps > 1e30f) return FLCE_ERR_INVALID_ARG;   // rejects NaN too
  if (cfg.variant != FLCE_CHUNKED || H > kRmsMaxH) return FLCE_ERR_UNSUPPORTED;
  return FLCE_OK;
}

}  // namespace

// ---- device memory of the no-allocation entry point ------------------------------------------
// One array per device (the code object's copy on each GPU it is loaded on, held until the process
// ends).  Bytes [0, 256) hold the data flag (zero at load, cleared again by flce_check), the rest
// the call's workspace.  In host code `scratch` is a host-side stand-in, not a device address:
// only the address hipGetSymbolAddress returns for a device is ever passed to a kernel.
namespace {
constexpr size_t kScratchBytes = (size_t)256 << 20;   // 256 MiB
constexpr size_t kScratchFlagBytes = 256;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on device `dev`, looked up once per device (with that device
// current) and kept; null if it has not been looked up (lookup = false) or the lookup failed.
char* scratch_on(int dev, bool lookup) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev] == nullptr && lookup) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = static_cast<char*>(p);
  }
  return g_scratch[dev];
}

// Chunk of a no-allocation call: a positive chunk as given (clamped to N); otherwise the
// automatic chunk, halved until the call's workspace fits the scratch.  0 if nothing fits.
int64_t noalloc_chunk(const flce_config_t& cfg, int64_t N, int64_t H, int64_t V, int64_t chunk) {
  const size_t cap = kScratchBytes - kScratchFlagBytes;
  int64_t c = effective_chunk(N, H, V, chunk, (int64_t)in_size(cfg));
  if (chunk > 0) return make_plan(cfg, N, H, V, c).total <= cap ? c : 0;
  while (c > 1 && make_plan(cfg, N, H, V, c).total > cap) c = (c + 1) / 2;
  return make_plan(cfg, N, H, V, c).total <= cap ? c : 0;
}

}  // namespace

extern "C" {

const char* flce_status_string(flce_status_t s) {
  switch (s) {
    case FLCE_OK: return "FLCE_OK";
    case FLCE_ERR_INVALID_ARG: return "FLCE_ERR_INVALID_ARG: invalid argument";
    case FLCE_ERR_UNSUPPORTED: return "FLCE_ERR_UNSUPPORTED: unsupported size, alignment or dtype combination";
    case FLCE_ERR_OOM: return "FLCE_ERR_OOM: workspace allocation failed or exceeds the configured limit";
    case FLCE_ERR_HIP: return "FLCE_ERR_HIP: HIP runtime error";
    case FLCE_ERR_DATA: return "FLCE_ERR_DATA: a target id was outside [0, V)";
  }
  return "unknown flce status";
}

flce_status_t flce_create(const flce_config_t* cfg, flce_handle_t* out) {
  if (cfg == nullptr || out == nullptr) return FLCE_ERR_INVALID_ARG;
  auto dt_ok = [](int32_t d) { return d == FLCE_BF16 || d == FLCE_FP32; };
  if (!dt_ok(cfg->in_dtype) || !dt_ok(cfg->dx_dtype) || !dt_ok(cfg->dw_dtype)) return FLCE_ERR_INVALID_ARG;
  if (cfg->variant != FLCE_CHUNKED && cfg->variant != FLCE_FUSED) return FLCE_ERR_INVALID_ARG;
  if (cfg->reserved != 0 || cfg->workspace_limit < 0 || cfg->device < 0) return FLCE_ERR_INVALID_ARG;
  if (cfg->in_dtype == FLCE_FP32 && (cfg->dx_dtype != FLCE_FP32 || cfg->dw_dtype != FLCE_FP32))
    return FLCE_ERR_UNSUPPORTED;
  if (cfg->variant == FLCE_FUSED && cfg->in_dtype != FLCE_BF16) return FLCE_ERR_UNSUPPORTED;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device >= ndev) {
    (void)hipGetLastError();
    return FLCE_ERR_HIP;
  }
  flce_handle_s* h = new (std::nothrow) flce_handle_s;
  if (h == nullptr) return FLCE_ERR_OOM;
  h->cfg = *cfg;
  *out = h;
  return FLCE_OK;
}

flce_status_t flce_destroy(flce_handle_t h) {
  if (h == nullptr) return FLCE_OK;
  {
    DeviceGuard g(h->cfg.device);
    (void)fold_marks(h);
    for (hipEvent_t e : h->pool) (void)hipEventDestroy(e);
    if (h->ws != nullptr) (void)hipFree(h->ws);
    if (h->flag != nullptr) (void)hipFree(h->flag);
    if (h->clk != nullptr) (void)hipFree(h->clk);
  }
  delete h;
  return FLCE_OK;
}

int64_t flce_effective_chunk(int64_t N, int64_t H, int64_t V, int64_t chunk) {
  return effective_chunk(N, H, V, chunk, 2);
}

size_t flce_workspace_bytes(flce_handle_t h, int64_t N, int64_t H, int64_t V, int64_t chunk) {
  if (h == nullptr || validate_sizes(h->cfg, N, H, V, chunk) != FLCE_OK) return 0;
  return make_plan(h->cfg, N, H, V, chunk).total;
}

size_t flce_workspace_bytes_opt(flce_handle_t h, int64_t N, int64_t H, int64_t V, int64_t chunk,
                                const flce_options_t* opt) {
  if (h == nullptr || validate_sizes(h->cfg, N, H, V, chunk) != FLCE_OK) return 0;
  Opts o;
  if (!parse_options(opt, o)) return 0;
  return make_plan(h->cfg, N, H, V, chunk, o.grads).total;
}

flce_status_t flce_reserve(flce_handle_t h, int64_t N, int64_t H, int64_t V, int64_t chunk) {
  if (h == nullptr) return FLCE_ERR_INVALID_ARG;
  const flce_status_t v = validate_sizes(h->cfg, N, H, V, chunk);
  if (v != FLCE_OK) return v;
  return ensure_workspace(h, make_plan(h->cfg, N, H, V, chunk).total);
}

flce_status_t flce_forward_backward_opt(flce_handle_t h, const void* x, const void* W,
                                        const int64_t* targets, int64_t N, int64_t H, int64_t V,
                                        int64_t chunk, const flce_options_t* opt, float* loss, void* dx,
                                        void* dW, float* lse, void* stream) {
  Opts o;
  if (!parse_options(opt, o)) return FLCE_ERR_INVALID_ARG;
  if (h == nullptr || x == nullptr || W == nullptr || targets == nullptr || loss == nullptr ||
      (o.grads && (dx == nullptr || dW == nullptr)))
    return FLCE_ERR_INVALID_ARG;
  const flce_status_t v = validate_sizes(h->cfg, N, H, V, chunk);
  if (v != FLCE_OK) return v;
  if (!aligned16(x) || !aligned16(W) || (o.grads && (!aligned16(dx) || !aligned16(dW))) ||
      (reinterpret_cast<uintptr_t>(targets) & 7u) || (reinterpret_cast<uintptr_t>(loss) & 3u) ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return FLCE_ERR_UNSUPPORTED;
  {
    const int64_t es = (int64_t)in_size(h->cfg);
    const int64_t dx_es = h->cfg.dx_dtype == FLCE_BF16 ? 2 : 4, dw_es = h->cfg.dw_dtype == FLCE_BF16 ? 2 : 4;
    if (!outputs_disjoint({Span(x, N * H * es), Span(W, V * H * es), Span(targets, N * 8)},
                          {Span(loss, 4), Span(o.grads ? dx : nullptr, N * H * dx_es),
                           Span(o.grads ? dW : nullptr, V * H * dw_es), Span(lse, N * 4)}))
      return FLCE_ERR_INVALID_ARG;
  }
  const Plan p = make_plan(h->cfg, N, H, V, chunk, o.grads);
  hipStream_t st = static_cast<hipStream_t>(stream);
  flce_status_t ws = capture_check(h, p.total, st);
  if (ws != FLCE_OK) return ws;
  ws = ensure_workspace(h, p.total);
  if (ws != FLCE_OK) return ws;
  DeviceGuard g(h->cfg.device);
  if (g.err != hipSuccess) return FLCE_ERR_HIP;
  ws = prepare_call(h, st);
  if (ws != FLCE_OK) return ws;
  const Exec e{h, static_cast<char*>(h->ws), h->flag, h->profiling};
  if (p.fused) return run_fused(e, p, o, x, W, targets, loss, dx, dW, lse, st);
  return run_chunked(e, p, o, x, W, targets, loss, dx, dW, lse, st);
}


size_t flce_rmsnorm_workspace_bytes(flce_handle_t h, int64_t N, int64_t H, int64_t V, int64_t chunk,
                                    const flce_options_t* opt) {
  Opts o;
  if (h == nullptr || !parse_options(opt, o) || validate_sizes(h->cfg, N, H, V, chunk) != FLCE_OK ||
      validate_rmsnorm(h->cfg, H, 0.f) != FLCE_OK)
    return 0;
  return make_plan(h->cfg, N, H, V, chunk, o.grads, true).total;
}

flce_status_t flce_rmsnorm_forward_backward(flce_handle_t h, const void* hidden, const void* gamma, float eps,
                                            const void* W, const int64_t* targets, int64_t N, int64_t H,
                                            int64_t V, int64_t chunk, const flce_options_t* opt, float* loss,
                                            void* dhidden, void* dgamma, void* dW, float* lse, void* stream) {
  Opts o;
  if (!parse_options(opt, o)) return FLCE_ERR_INVALID_ARG;
  if (h == nullptr || hidden == nullptr || gamma == nullptr || W == nullptr || targets == nullptr ||
      loss == nullptr || (o.grads && (dhidden == nullptr || dgamma == nullptr || dW == nullptr)))
    return FLCE_ERR_INVALID_ARG;
  flce_status_t v = validate_sizes(h->cfg, N, H, V, chunk);
  if (v != FLCE_OK) return v;
  v = validate_rmsnorm(h->cfg, H, eps);
  if (v != FLCE_OK) return v;
  if (!aligned16(hidden) || !aligned16(gamma) || !aligned16(W) ||
      (o.grads && (!aligned16(dhidden) || !aligned16(dgamma) || !aligned16(dW))) ||
      (reinterpret_cast<uintptr_t>(targets) & 7u) || (reinterpret_cast<uintptr_t>(loss) & 3u) ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return FLCE_ERR_UNSUPPORTED;
  {
    const int64_t es = (int64_t)in_size(h->cfg);
    const int64_t dx_es = h->cfg.dx_dtype == FLCE_BF16 ? 2 : 4, dw_es = h->cfg.dw_dtype == FLCE_BF16 ? 2 : 4;
    if (!outputs_disjoint({Span(hidden, N * H * es), Span(gamma, H * es), Span(W, V * H * es), Span(targets, N * 8)},
                          {Span(loss, 4), Span(o.grads ? dhidden : nullptr, N * H * dx_es),
                           Span(o.grads ? dgamma : nullptr, H * dw_es), Span(o.grads ? dW : nullptr, V * H * dw_es),
                           Span(lse, N * 4)}))
      return FLCE_ERR_INVALID_ARG;
  }
  const Plan p = make_plan(h->cfg, N, H, V, chunk, o.grads, true);
  hipStream_t st = static_cast<hipStream_t>(stream);
  flce_status_t ws = capture_check(h, p.total, st);
  if (ws != FLCE_OK) return ws;
  ws = ensure_workspace(h, p.total);
  if (ws != FLCE_OK) return ws;
  DeviceGuard g(h->cfg.device);
  if (g.err != hipSuccess) return FLCE_ERR_HIP;
  ws = prepare_call(h, st);
  if (ws != FLCE_OK) return ws;
  const Exec e{h, static_cast<char*>(h->ws), h->flag, h->profiling};
  return run_rmsnorm(e, p, o, hidden, gamma, eps, W, targets, loss, dhidden, dgamma, dW, lse, st);
}

flce_status_t flce_forward_backward_ex(flce_handle_t h, const void* x, const void* W,
                                       const int64_t* targets, int64_t N, int64_t H, int64_t V,
                                       int64_t chunk, float* loss, void* dx, void* dW, float* lse,
                                       void* stream) {
  return flce_forward_backward_opt(h, x, W, targets, N, H, V, chunk, nullptr, loss, dx, dW, lse, stream);
}

flce_status_t flce_forward_backward(flce_handle_t h, const void* x, const void* W,
                                    const int64_t* targets, int64_t N, int64_t H, int64_t V,
                                    int64_t chunk, float* loss, void* dx, void* dW, void* stream) {
  return flce_forward_backward_opt(h, x, W, targets, N, H, V, chunk, nullptr, loss, dx, dW, nullptr, stream);
}

flce_status_t flce_forward_backward_noalloc(flce_handle_t h, const void* x, const void* W,
                                            const int64_t* targets, int64_t N, int64_t H, int64_t V,
                                            int64_t chunk, float* loss, void* dx, void* dW, void* stream) {
  if (h == nullptr || x == nullptr || W == nullptr || targets == nullptr || loss == nullptr || dx == nullptr ||
      dW == nullptr)
    return FLCE_ERR_INVALID_ARG;
  if (h->cfg.variant != FLCE_CHUNKED) return FLCE_ERR_UNSUPPORTED;
  const flce_status_t v = validate_sizes(h->cfg, N, H, V, chunk);
  if (v != FLCE_OK) return v;
  if (!aligned16(x) || !aligned16(W) || !aligned16(dx) || !aligned16(dW) ||
      (reinterpret_cast<uintptr_t>(targets) & 7u) || (reinterpret_cast<uintptr_t>(loss) & 3u))
    return FLCE_ERR_UNSUPPORTED;
  {
    const int64_t es = (int64_t)in_size(h->cfg);
    const int64_t dx_es = h->cfg.dx_dtype == FLCE_BF16 ? 2 : 4, dw_es = h->cfg.dw_dtype == FLCE_BF16 ? 2 : 4;
    if (!outputs_disjoint({Span(x, N * H * es), Span(W, V * H * es), Span(targets, N * 8)},
                          {Span(loss, 4), Span(dx, N * H * dx_es), Span(dW, V * H * dw_es)}))
      return FLCE_ERR_INVALID_ARG;
  }
  const int64_t C = noalloc_chunk(h->cfg, N, H, V, chunk);
  if (C == 0) return FLCE_ERR_UNSUPPORTED;   // the call's workspace exceeds the scratch
  const Plan p = make_plan(h->cfg, N, H, V, C);
  DeviceGuard g(h->cfg.device);
  if (g.err != hipSuccess) return FLCE_ERR_HIP;
  char* base = scratch_on(h->cfg.device, true);
  if (base == nullptr) return FLCE_ERR_HIP;
  const Exec e{h, base + kScratchFlagBytes, reinterpret_cast<int*>(base), false};
  return run_chunked(e, p, Opts{}, x, W, targets, loss, dx, dW, nullptr, static_cast<hipStream_t>(stream));
}

flce_status_t flce_profile_enable(flce_handle_t h, int enable) {
  if (h == nullptr) return FLCE_ERR_INVALID_ARG;
  DeviceGuard g(h->cfg.device);
  if (g.err != hipSuccess) return FLCE_ERR_HIP;
  (void)fold_marks(h);
  for (Stat& s : h->stats) s = Stat{};
  if (enable != 0) {
    const size_t bytes = 2 * K_COUNT * sizeof(unsigned long long);
    if (h->clk == nullptr && hipMalloc(reinterpret_cast<void**>(&h->clk), bytes) != hipSuccess) {
      h->clk = nullptr;
      (void)hipGetLastError();
      return FLCE_ERR_OOM;
    }
    h->clk_reset = true;   // cleared by the next call's first kernel, on its stream
  }
  h->profiling = enable != 0;
  return FLCE_OK;
}

flce_status_t flce_profile_read(flce_handle_t h, flce_kernel_stat_t* out, int capacity, int* count) {
  if (h == nullptr || count == nullptr || capacity < 0 || (capacity > 0 && out == nullptr))
    return FLCE_ERR_INVALID_ARG;
  DeviceGuard g(h->cfg.device);
  if (g.err != hipSuccess) return FLCE_ERR_HIP;
  hipError_t e = fold_marks(h);
  unsigned long long clk[2 * K_COUNT] = {};
  if (h->clk != nullptr && !h->clk_reset) {   // blocking copy (null stream) of the clock counters
    const hipError_t e2 = hipMemcpy(clk, h->clk, sizeof(clk), hipMemcpyDeviceToHost);
    if (e2 != hipSuccess) e = e2;
  }
  int n = 0;
  for (int k = 0; k < K_COUNT; ++k) {
    const Stat& s = h->stats[k];
    if (s.launches == 0) continue;
    if (n < capacity) {
      flce_kernel_stat_t& o = out[n];
      std::memset(&o, 0, sizeof(o));
      std::strncpy(o.name, kKernelNames[k], sizeof(o.name) - 1);
      o.launches = s.launches;
      o.total_ms = s.ms;
      o.flops = s.flops;
      o.bytes = s.bytes;
      o.sclk_mhz = clk[2 * k + 1] > 0 ? 100.0 * (double)clk[2 * k] / (double)clk[2 * k + 1] : 0.0;
    }
    ++n;
  }
  *count = n;
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

flce_status_t flce_check(flce_handle_t h, void* stream) {
  if (h == nullptr) return FLCE_ERR_INVALID_ARG;
  // the handle's flag (once a call has cleared it) and the device's no-allocation flag (once a
  // no-allocation call has run on the device)
  int* flags[2] = {h->flag != nullptr && h->flag_ready ? h->flag : nullptr,
                   reinterpret_cast<int*>(scratch_on(h->cfg.device, false))};
  if (flags[0] == nullptr && flags[1] == nullptr) return FLCE_OK;
  DeviceGuard g(h->cfg.device);
  if (g.err != hipSuccess) return FLCE_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  bool bad = false;
  for (int* fl : flags) {
    if (fl == nullptr) continue;
    int f = 0;
    if (hipMemcpyAsync(&f, fl, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return FLCE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return FLCE_ERR_HIP;
    if (f != 0) {
      const int zero = 0;
      if (hipMemcpyAsync(fl, &zero, sizeof(int), hipMemcpyHostToDevice, st) != hipSuccess) return FLCE_ERR_HIP;
      if (hipStreamSynchronize(st) != hipSuccess) return FLCE_ERR_HIP;
      bad = true;
    }
  }
  return bad ? FLCE_ERR_DATA : FLCE_OK;
}

}  // extern "C"
