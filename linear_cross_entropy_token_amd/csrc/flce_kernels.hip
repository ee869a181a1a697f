// HIP kernels of the token-chunked FLCE path for gfx950.
//
// Per token chunk (the four steps of the core idea of the "Fused Linear
// Cross-Entropy" page, 42jerrykim.github.io):
//   logits_lse   z = x_c W^T on MFMA; the epilogue reduces each row of the
//                256-wide vocabulary tile to (max, sum exp(z - max)) in
//                registers, picks up the target logit, and stores z - max into
//                the chunk buffer (online-softmax statistics as on the "Unsloth
//                deep architecture" page, streaming CE kernel; the shift keeps
//                the bf16 rounding of the softmax relative at any logit scale).
//   lse_combine  lse_n = M + ln sum_j s_j e^(m_j - M) over the vocab tiles,
//                per-row loss lse_n - z[n, t_n] (0 for an ignored token).
//   dlogits      G = (exp(z - lse) - onehot(t)) * scale written over z - max
//                (softmax - one_hot in the same buffer, step 2; scale = 1/N
//                for the mean over N tokens, the page's reduction).
//   dx           dx_c (+)= G W (contraction over the vocabulary, split-K).
//   dw           dW (+)= G^T x_c (contraction over the chunk's tokens).
// and once per call: scale (count of the tokens that count, on the device)
// before the chunks, finalize (loss = sum_n loss_n / count, deterministic)
// after them.
#include "flce_device.hpp"
#include "flce_internal.hpp"

namespace flce {

static_assert(kTile == kTileM && kTile == kTileN, "tile sizes of the dispatcher and the engine differ");

// ---------------------------------------------------------------------------
// logits + LSE partials + target gather + z store
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void logits_lse_kernel(LogitsArgs a) {
  const ClockSpan span(a.clk);
  constexpr int kEpiBytes = 2 * kWaveCols * kTile * (int)sizeof(float) + kTile * (int)sizeof(int);
  static_assert(kSmemBytes + kEpiBytes <= kDeepRingBytes, "epilogue scratch fits behind the z tile");
  __shared__ __attribute__((aligned(16))) char smem[kDeepRingBytes];
  const int tid = threadIdx.x;
  const int L = xcd_remap(blockIdx.x, a.tiles_m * a.tiles_n);
  int tm, tn;
  grouped_tile(L, a.tiles_m, a.tiles_n, kGroupM, tm, tn);
  const int m0 = tm * kTile;   // tokens
  const int n0 = tn * kTile;   // vocabulary ids
  constexpr int ES = (int)sizeof(T);

  Operand<T, true> C, R;      // columns: W rows (vocab), rows: x rows (tokens)
  C.init(static_cast<const T*>(a.W), a.H, n0, a.V, (uint32_t)((int64_t)a.V * a.H * ES));
  R.init(static_cast<const T*>(a.x), a.H, m0, a.rows, (uint32_t)((int64_t)a.rows * a.H * ES));
  // target column of each tile row (-1: not in this tile); loaded before the GEMM so its
  // latency hides behind it
  int rel = -1;
  if (tid < kTile && m0 + tid < a.rows) {
    const int64_t d = a.t[m0 + tid] - (int64_t)n0;
    rel = (d >= 0 && d < kTile) ? (int)d : -1;
  }
  f32x16 acc[kColBlocks][4];
  gemm_tile_balanced<T>(acc, smem, C, R, 0, a.H, threadIdx.x);

  const Frag f = frag_coords();
  // [2][kWaveCols][kTile]: per column-wave max, then sum; then the target column per row.  The
  // ring below them holds the bf16 z tile (layout of the dW epilogue) on its way to HBM.
  float* red = reinterpret_cast<float*>(smem + kSmemBytes);
  int* trel = reinterpret_cast<int*>(smem + kSmemBytes + 2 * kWaveCols * kTile * sizeof(float));
  if (tid < kTile) trel[tid] = rel;
  phase_barrier<false, true>();

  const float ninf = -__builtin_inff();
  const int wc = (tid >> 6) % kWaveCols;
  const int vlim = a.V - n0;                // columns >= vlim are padding
  const bool full = vlim >= kTile;          // wave-uniform: no padding column in this tile
  T* Z = static_cast<T*>(a.z);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = f.row(j);
    const int grow = m0 + row;
    float mx = ninf;
    if (full) {
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) mx = fmaxf(mx, acc[i][j][rg]);
    } else {
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
        for (int rg = 0; rg < 16; ++rg)
          if (f.col0(i, rg >> 2) + (rg & 3) < vlim) mx = fmaxf(mx, acc[i][j][rg]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // sum of exp(z - mx) as exp2(z log2 e - mx log2 e): one fma per element before the exp
    const float mxl = mx * kLog2e;
    float s = 0.f;
    if (full) {
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][rg], kLog2e, -mxl));
    } else {
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
        for (int rg = 0; rg < 16; ++rg)
          if (f.col0(i, rg >> 2) + (rg & 3) < vlim)
            s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][rg], kLog2e, -mxl));
    }
    s += __shfl_xor(s, 32, 64);
    if (f.lane < 32) {
      red[wc * kTile + row] = mx;
      red[(kWaveCols + wc) * kTile + row] = s;
    }
    if (grow < a.rows) {
      // the lane holding this row's target column (at most one per row) stores its logit;
      // selected without branches
      const int tr = trel[row];
      float zsel = 0.f;
      bool hit = false;
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool h = f.col0(i, q) + e == tr;
            zsel = h ? acc[i][j][4 * q + e] : zsel;
            hit = hit || h;
          }
      if (hit) a.zt[grow] = zsel;
    }
  }
  phase_barrier<false, true>();   // per-wave row statistics visible in LDS
  if (Z != nullptr) {   // null: statistics-only pass
    // The buffer holds z - M, M the row's maximum over this 256-column tile (the tile's LSE
    // partial), so that the values that carry the softmax mass sit near zero, where bf16 is
    // finest: rounding then perturbs exp(z - lse) by ~2^-9 relatively at any logit scale,
    // where rounding z itself would perturb it by |z| 2^-9 (3% at |z| = 40).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = f.row(j);
      float M = red[row];
#pragma unroll
      for (int w = 1; w < kWaveCols; ++w) M = fmaxf(M, red[w * kTile + row]);
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c0 = f.col0(i, q);
          const f32x4 v{acc[i][j][4 * q] - M, acc[i][j][4 * q + 1] - M, acc[i][j][4 * q + 2] - M,
                        acc[i][j][4 * q + 3] - M};
          if constexpr (ES == 2) {
            const int c = c0 >> 3;
            *reinterpret_cast<u32x2*>(smem + row * 512 + ((c ^ (row & 31)) << 4) + 8 * (f.lane >> 5)) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          } else if (m0 + row < a.rows) {
            *reinterpret_cast<f32x4*>(Z + (int64_t)(m0 + row) * a.ldz + n0 + c0) = v;
          }
        }
    }
  }
  phase_barrier<false, true>();   // the z tile visible in LDS
  if constexpr (ES == 2) {
    if (Z != nullptr) {   // full 512-byte rows of z: 2 rows per 1 KiB block, 16 blocks per wave
      const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
      const int lane = tid & 63;
      constexpr int kPerWave = kTile * kTile * 2 / 1024 / kWaves;
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int b = wave * kPerWave + i;
        const int r = 2 * b + (lane >> 5);
        const int c = (lane & 31) ^ (r & 31);
        if (m0 + r < a.rows)
          *reinterpret_cast<u32x4*>(Z + (int64_t)(m0 + r) * a.ldz + n0 + 8 * c) =
              *reinterpret_cast<const u32x4*>(smem + b * 1024 + 16 * lane);
      }
    }
  }
  if (tid < kTile && m0 + tid < a.rows) {
    float M = ninf;
#pragma unroll
    for (int w = 0; w < kWaveCols; ++w) M = fmaxf(M, red[w * kTile + tid]);
    float S = 0.f;
#pragma unroll
    for (int w = 0; w < kWaveCols; ++w) {
      const float m = red[w * kTile + tid];
      if (m != ninf) S += red[(kWaveCols + w) * kTile + tid] * fast_exp(m - M);
    }
    a.pm[(int64_t)tn * a.pstride + m0 + tid] = M;
    a.ps[(int64_t)tn * a.pstride + m0 + tid] = S;
  }
}

// ---------------------------------------------------------------------------
// per-row combine of the vocabulary-tile partials: 32 rows per block, 8 lanes
// per row each folding every 8th tile, then a fold of the 8 partial results
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lse_combine_kernel(CombineArgs a) {
  __shared__ float sm[8][32], ss[8][32];
  const int rl = threadIdx.x & 31;
  const int part = threadIdx.x >> 5;
  const int r = blockIdx.x * 32 + rl;
  const float ninf = -__builtin_inff();
  float M = ninf, S = 0.f;
  if (r < a.rows) {
    // kU tiles per round, loaded before any of them is merged, so that a round costs one
    // memory latency instead of kU
    constexpr int kU = 8;
    for (int j0 = part; j0 < a.tiles_n; j0 += 8 * kU) {
      float m[kU], s[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int j = j0 + 8 * u;
        const bool in = j < a.tiles_n;
        m[u] = in ? a.pm[(int64_t)j * a.pstride + r] : ninf;
        s[u] = in ? a.ps[(int64_t)j * a.pstride + r] : 0.f;
      }
      float Mn = M;
#pragma unroll
      for (int u = 0; u < kU; ++u) Mn = fmaxf(Mn, m[u]);
      if (Mn == ninf) continue;                     // nothing but empty partials so far
      float Sn = M == ninf ? 0.f : S * fast_exp(M - Mn);
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (m[u] != ninf) Sn += s[u] * fast_exp(m[u] - Mn);
      M = Mn;
      S = Sn;
    }
  }
  sm[part][rl] = M;
  ss[part][rl] = S;
  __syncthreads();
  if (part != 0 || r >= a.rows) return;
  float MM = ninf;
  for (int p = 0; p < 8; ++p) MM = fmaxf(MM, sm[p][rl]);
  float SS = 0.f;
  for (int p = 0; p < 8; ++p)
    if (sm[p][rl] != ninf) SS += ss[p][rl] * fast_exp(sm[p][rl] - MM);
  const float lse = MM + fast_log(SS);
  const int64_t tv = a.t[r];
  a.lse[r] = lse;
  if (a.ign.skip(tv)) {                 // ignored token: no loss
    a.loss_rows[r] = 0.f;
    return;
  }
  const bool ok = tv >= 0 && tv < a.V;
  a.loss_rows[r] = ok ? lse - a.zt[r] : __builtin_nanf("");
  if (!ok) atomicOr(a.flag, 1);
}

// ---------------------------------------------------------------------------
// G = (exp(z - lse) - onehot) / N, in place over the buffer of z - M (M: the row's tile
// maximum), as exp((z - M) - (lse - M)); zero in the padding columns
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dlogits_kernel(DlogitsArgs a) {
  // Work items are (row group, vocabulary tile): kRows rows x 256 columns, one 16-byte chunk per
  // thread, so a block reads its rows' tile maxima as one short contiguous run and each row's
  // chunks as one contiguous 512-byte (bf16) or 1 KiB (fp32) span.  Tiles vary fastest.
  constexpr int E = Elem<T>::E;
  constexpr int kChunks = kTile / E;          // chunks per row of a tile
  constexpr int kRows = 256 / kChunks;        // rows per work item
  const int tiles = (int)(a.ldz / kTile);
  const int64_t items = (int64_t)((a.rows + kRows - 1) / kRows) * tiles;
  T* Z = static_cast<T*>(a.z);
  const float scale = a.scale->grad;
  const int tr = threadIdx.x / kChunks;
  const int tc = threadIdx.x % kChunks;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int tile = (int)(it % tiles);
    const int r = (int)(it / tiles) * kRows + tr;
    if (r >= a.rows) continue;
    const int c0 = tile * kTile + tc * E;
    // the buffer holds z - M (M: the row's maximum over the tile, its LSE partial)
    const float l = a.lse[r] - a.pm[(int64_t)tile * a.pstride + r];
    const int64_t tv = a.t[r];
    const bool counted = !a.ign.skip(tv);   // an ignored token's row of G is zero
    u32x4* p = reinterpret_cast<u32x4*>(Z + (int64_t)r * a.ldz + c0);
    u32x4 v = *p;
    T* e = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const int col = c0 + k;
      float g = 0.f;
      if (counted && col < a.V) {
        g = fast_exp(to_f32<T>(e[k]) - l);
        if (col == tv) g -= 1.f;
        g *= scale;
      }
      e[k] = from_f32<T>(g);
    }
    *p = v;
  }
}

// ---------------------------------------------------------------------------
// dx_c = G W (split over the vocabulary when the tile count is low)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void dx_kernel(DxArgs a) {
  const ClockSpan span(a.clk);
  __shared__ __attribute__((aligned(16))) char smem[kDeepRingBytes];
  const int tiles = a.tiles_m * a.tiles_n;
  const int L = xcd_remap(blockIdx.x, tiles * a.splits);
  const int split = L / tiles;
  const int rem = L - split * tiles;
  int tm, tn;
  grouped_tile(rem, a.tiles_m, a.tiles_n, kGroupM, tm, tn);
  const int m0 = tm * kTile, n0 = tn * kTile;   // tokens, hidden units
  const int ks = split * a.k_per_split;
  const int ke = (int)min((int64_t)ks + a.k_per_split, a.ldg);
  constexpr int ES = (int)sizeof(T);

  Operand<T, false> C;   // columns: W as [v][h] (hidden contiguous)
  Operand<T, true> R;    // rows: G as [token][v]
  C.init(static_cast<const T*>(a.W), a.H, n0, a.H, (uint32_t)((int64_t)a.V * a.H * ES));
  R.init(static_cast<const T*>(a.g), a.ldg, m0, a.rows, (uint32_t)((int64_t)a.rows * a.ldg * ES));
  f32x16 acc[kColBlocks][4];
  gemm_tile_balanced<T>(acc, smem, C, R, ks, ke, threadIdx.x);

  const Frag f = frag_coords();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int grow = m0 + f.row(j);
    if (grow >= a.rows) continue;
#pragma unroll
    for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + f.col0(i, q);
        if (col >= a.H) continue;
        const f32x4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        const int64_t o = (int64_t)grow * a.H + col;
        if (a.splits > 1) {
          *reinterpret_cast<f32x4*>(a.part + split * a.part_stride + o) = v;
        } else if (a.dx_fp32) {
          f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(a.dx) + o);
          *p = a.accumulate ? *p + v : v;
        } else {
          u32x2* p = reinterpret_cast<u32x2*>(static_cast<bf16_t*>(a.dx) + o);
          f32x4 w = v;
          if (a.accumulate) {
            const u32x2 old = *p;
            w[0] += bf16_to_f32(old[0] & 0xffffu);
            w[1] += bf16_to_f32(old[0] >> 16);
            w[2] += bf16_to_f32(old[1] & 0xffffu);
            w[3] += bf16_to_f32(old[1] >> 16);
          }
          *p = u32x2{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3])};
        }
      }
  }
}

__global__ __launch_bounds__(256) void dx_reduce_kernel(DxReduceArgs a) {
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < a.count;
       i += (int64_t)gridDim.x * blockDim.x * 4) {
    f32x4 s = *reinterpret_cast<const f32x4*>(a.part + i);
    for (int k = 1; k < a.splits; ++k) s += *reinterpret_cast<const f32x4*>(a.part + k * a.part_stride + i);
    if (a.dx_fp32) {
      f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(a.dx) + i);
      *p = a.accumulate ? *p + s : s;
    } else {
      u32x2* p = reinterpret_cast<u32x2*>(static_cast<bf16_t*>(a.dx) + i);
      if (a.accumulate) {
        const u32x2 old = *p;
        s[0] += bf16_to_f32(old[0] & 0xffffu);
        s[1] += bf16_to_f32(old[0] >> 16);
        s[2] += bf16_to_f32(old[1] & 0xffffu);
        s[3] += bf16_to_f32(old[1] >> 16);
      }
      *p = u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
    }
  }
}

// ---------------------------------------------------------------------------
// dW (+)= G^T x_c
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void dw_kernel(DwArgs a) {
  const ClockSpan span(a.clk);
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x;
  const int L = xcd_remap(blockIdx.x, a.tiles_m * a.tiles_n);
  int tm, tn;
  grouped_tile(L, a.tiles_m, a.tiles_n, kGroupM, tm, tn);
  const int m0 = tm * kTile, n0 = tn * kTile;   // vocabulary ids, hidden units
  constexpr int ES = (int)sizeof(T);

  Operand<T, false> C;   // columns: x_c as [token][h]
  Operand<T, false> R;   // rows: G as [token][v]
  C.init(static_cast<const T*>(a.x), a.H, n0, a.H, (uint32_t)((int64_t)a.rows * a.H * ES));
  R.init(static_cast<const T*>(a.g), a.ldg, m0, (int)a.ldg, (uint32_t)((int64_t)a.rows * a.ldg * ES));
  f32x16 acc[kColBlocks][4];
  gemm_tile<T>(acc, smem, C, R, 0, a.rows, threadIdx.x);

  const Frag f = frag_coords();
  if (a.dw_fp32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = m0 + f.row(j);
      if (v >= a.V) continue;
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int h = n0 + f.col0(i, q);
          if (h >= a.H) continue;
          f32x4 val{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(a.dW) + (int64_t)v * a.H + h);
          if (a.accumulate) val += *p;
          *p = val;
        }
    }
    return;
  }
  // bf16 dW: the 256 x 256 tile goes through the (now free) LDS ring as 256 rows of 512 bytes,
  // 16-byte chunk c of row r at chunk c ^ (r % 32), so that HBM sees full-line copies (2 rows
  // per 1 KiB copy) instead of 8-byte accesses that each touch 32 rows: the old tile comes in
  // by direct-to-LDS copies, each lane adds its accumulators in place, full rows go out.
  const i32x4 rs = make_rsrc(a.dW, (uint32_t)((int64_t)a.V * a.H * 2));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  constexpr int kPerWave = kTile * kTile * 2 / 1024 / kWaves;
  auto block_off = [&](int b, int& r) -> uint32_t {   // global byte offset of this lane's chunk
    r = 2 * b + (lane >> 5);
    const int c = (lane & 31) ^ (r & 31);
    const int v = m0 + r;
    return (v < a.V && n0 + 8 * c < a.H) ? ((uint32_t)v * (uint32_t)a.H + (uint32_t)n0) * 2u + (uint32_t)c * 16u : kOOB;
  };
  if (a.accumulate) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      int r;
      dma16(rs, smem + (wave * kPerWave + i) * 1024, block_off(wave * kPerWave + i, r));
    }
    phase_barrier<true, false>();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = f.row(j);
#pragma unroll
    for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = f.col0(i, q) >> 3;
        u32x2* s = reinterpret_cast<u32x2*>(smem + r * 512 + ((c ^ (r & 31)) << 4) + 8 * (f.lane >> 5));
        f32x4 val{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if (a.accumulate) {
          const u32x2 old = *s;
          val[0] += bf16_to_f32(old[0] & 0xffffu);
          val[1] += bf16_to_f32(old[0] >> 16);
          val[2] += bf16_to_f32(old[1] & 0xffffu);
          val[3] += bf16_to_f32(old[1] >> 16);
        }
        *s = u32x2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
      }
  }
  phase_barrier<false, true>();
  bf16_t* dW = static_cast<bf16_t*>(a.dW);
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int b = wave * kPerWave + i;
    int r;
    const uint32_t off = block_off(b, r);
    if (off != kOOB)
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dW) + off) = *reinterpret_cast<const u32x4*>(smem + b * 1024 + 16 * lane);
  }
}

// ---------------------------------------------------------------------------
// loss = sum_n loss_n / N, fixed summation order (bitwise repeatable)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void finalize_kernel(FinalizeArgs a) {
  __shared__ double part[1024];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < a.n; i += 1024) s += (double)a.loss_rows[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *a.loss = (float)(part[0] / a.scale->denom);
}

// ---------------------------------------------------------------------------
// per-call normalisation: count the tokens whose target is not ignored (fixed order, one
// block), then 1 / count (mean) or 1 (sum).  With no token counted a mean is 0 / 0 = NaN and
// every dlogits row is zero, as for the mean cross-entropy of an all-ignored batch.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void scale_kernel(ScaleArgs a) {
  __shared__ long long part[1024];
  long long c = 0;
  for (int64_t i = threadIdx.x; i < a.n; i += 1024) c += a.ign.skip(a.t[i]) ? 0 : 1;
  part[threadIdx.x] = c;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double denom = a.sum ? 1.0 : (double)part[0];
    a.out->grad = (float)(1.0 / denom);
    a.out->pad = 0.f;
    a.out->denom = denom;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline int grid_elementwise(int64_t work, int per_block) {
  int64_t b = (work + per_block - 1) / per_block;
  if (b > 256 * 16) b = 256 * 16;
  if (b < 1) b = 1;
  return (int)b;
}

hipError_t launch_logits(In in, const LogitsArgs& a, hipStream_t s) {
  const int grid = a.tiles_m * a.tiles_n;
  if (in == In::BF16) hipLaunchKernelGGL(logits_lse_kernel<bf16_t>, dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(logits_lse_kernel<float>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lse_combine_kernel, dim3((a.rows + 31) / 32), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dlogits(In in, const DlogitsArgs& a, hipStream_t s) {
  const int E = in == In::BF16 ? 8 : 4;
  const int grid = grid_elementwise(a.ldz / E * a.rows, 256);   // one 16-byte chunk per thread
  if (in == In::BF16) hipLaunchKernelGGL(dlogits_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(dlogits_kernel<float>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dx(In in, const DxArgs& a, hipStream_t s) {
  const int grid = a.tiles_m * a.tiles_n * a.splits;
  if (in == In::BF16) hipLaunchKernelGGL(dx_kernel<bf16_t>, dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(dx_kernel<float>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dx_reduce(const DxReduceArgs& a, hipStream_t s) {
  const int grid = grid_elementwise(a.count / 4, 256);
  hipLaunchKernelGGL(dx_reduce_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dw(In in, const DwArgs& a, hipStream_t s) {
  const int grid = a.tiles_m * a.tiles_n;
  if (in == In::BF16) hipLaunchKernelGGL(dw_kernel<bf16_t>, dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(dw_kernel<float>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scale(const ScaleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(scale_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace flce
