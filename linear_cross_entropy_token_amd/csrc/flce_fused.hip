// Fused FLCE variant, pass 2, for gfx950 (bf16 inputs).
//
// Pass 1 (logits_lse without the logits store, then lse_combine) leaves the
// per-token log-sum-exp.  Pass 2 never writes a logits or dlogits tensor:
// for each (256-token, 256-vocabulary) tile a workgroup
//   1. recomputes z = x_tile W_tile^T on the MFMA engine (contraction over H),
//   2. forms G = (exp(z - lse) - onehot(t)) * scale (1/N for the page's mean;
//      zero rows for ignored tokens) and keeps it in LDS as a
//      256 x 256 bf16 tile (the dlogits of the FLCE page's step 2, held
//      on-chip as the "Unsloth deep architecture" page's streaming CE kernel
//      does),
//   3. for every 256-wide slice of the hidden dimension, multiplies the LDS
//      tile by the matching W slice (dx partial, contraction over the tile's
//      vocabulary) and by the matching x slice (dW partial, contraction over
//      the tile's tokens), streaming those operands through a 2 x 16 KiB
//      direct-to-LDS ring, and adds the partials into fp32 accumulators with
//      global fp32 atomics (the reduction by atomic adds that page names).
// The recomputation costs one extra forward GEMM (8 N H V flops instead of
// 6 N H V) and every dx / dW element receives one atomic add per vocabulary
// tile / token tile.
#include "flce_device.hpp"
#include "flce_internal.hpp"

namespace flce {

// LDS layout of the dlogits tile: 256 token rows x 512 bytes; 16-byte chunk c of
// row r sits at chunk c ^ swz_g(r).  Conflict-free (128- and 256-byte banking)
// both for 16-byte k-major reads (dx) and for transposing reads (dW).
__device__ __forceinline__ int swz_g(int r) {
  return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 10 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 2 : 0) ^ ((r & 16) ? 16 : 0);
}
__device__ __forceinline__ int g_off(int row, int chunk) { return row * 512 + ((chunk ^ swz_g(row)) << 4); }

// dx rows operand: token mnb + l % 32, k = vocabulary 16 ks + 8 (l / 32) .. +7
__device__ __forceinline__ u32x4 g_frag_k(const char* g, int mnb, int ks, int lane) {
  const int row = mnb + (lane & 31);
  const int c = 2 * ks + (lane >> 5);
  return *reinterpret_cast<const u32x4*>(g + g_off(row, c));
}

// dW rows operand: vocabulary mnb + l % 32, k = token 16 ks + 8 (l / 32) .. +7.  Issued as inline
// asm (the transposing-read builtin makes the compiler wait for every copy in flight first);
// gemm_stream waits for these reads before its MFMAs.
__device__ __forceinline__ u32x4 g_frag_t(const char* g, int mnb, int ks, int lane) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const int r = 16 * ks + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int v = mnb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int byte = (v & 7) * 2;
  const uint32_t a0 = (uint32_t)(uintptr_t)(const lds_i16x4*)(g + g_off(r, v >> 3) + byte);
  const uint32_t a1 = (uint32_t)(uintptr_t)(const lds_i16x4*)(g + g_off(r + 4, v >> 3) + byte);
  u32x2 l2, h2;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(l2) : "v"(a0));
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(h2) : "v"(a1));
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

constexpr int kStreamBytes = 16384;   // one 32-row mn-major slice of a 256-wide operand

// acc = sum over the tile's 256 k of S[k][col] * rows(row, k), S streamed 32 k-rows at a time.
// MFMA roles are swapped relative to the tile engine: the rows operand is the MFMA's A input,
// so register rg of block (i, j) in lane l holds
//   row = 32 j + 8 (rg / 4) + 4 (l / 32) + rg % 4,   col = 32 i + l % 32,
// i.e. the 32 lanes of a half-wave hold 32 consecutive columns of one row, and each atomic
// instruction of the epilogue touches two 128-byte lines.
constexpr int kStreamBPW = 16 / kWaves;   // 1 KiB DMA blocks per wave per streamed slice

template <class RowsFrag>
__device__ __forceinline__ void gemm_stream(f32x16 (&acc)[kColBlocks][4], char* ring,
                                            const Operand<bf16_t, false, kStreamBPW>& S, int k_end,
                                            RowsFrag rows_frag) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rowb = (wave / kWaveCols) * 128;
  const int colb = (wave % kWaveCols) * (kTile / kWaveCols);
#pragma unroll
  for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  S.issue(ring, 0, k_end, wave);
  for (int kt = 0; kt < 8; ++kt) {
    phase_barrier<true, false>();
    if (kt + 1 < 8) S.issue(ring + ((kt + 1) & 1) * kStreamBytes, (kt + 1) * 32, k_end, wave);
    const char* st = ring + (kt & 1) * kStreamBytes;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 a[kColBlocks], b[4];
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i) a[i] = read_frag<bf16_t, false, true>(st, colb + 32 * i, s, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = rows_frag(rowb + 32 * j, 2 * kt + s, lane);
      lgkm_wait();   // the transposing reads are asm: the compiler does not wait for them
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma<bf16_t>(b[j], a[i], acc[i][j]);
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void fused_bwd_kernel(FusedArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes + 2 * kStreamBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int L = xcd_remap(blockIdx.x, a.tiles_m * a.tiles_n);
  const int tm = L % a.tiles_m;
  const int tn = L / a.tiles_m;
  const int m0 = tm * kTile;   // tokens (within the chunk)
  const int n0 = tn * kTile;   // vocabulary ids
  const bf16_t* X = static_cast<const bf16_t*>(a.x);
  const bf16_t* W = static_cast<const bf16_t*>(a.W);

  // 1. z tile (columns: vocabulary, rows: tokens)
  f32x16 acc[kColBlocks][4];
  {
    Operand<bf16_t, true> C, R;
    C.init(W, a.H, n0, a.V, (uint32_t)((int64_t)a.V * a.H * 2));
    R.init(X, a.H, m0, a.rows, (uint32_t)((int64_t)a.rows * a.H * 2));
    gemm_tile_interleaved<bf16_t>(acc, smem, C, R, 0, a.H);
  }

  // 2. dlogits tile into LDS (bf16)
  char* g = smem;
  const float gscale = a.scale->grad;
  const Frag f = frag_coords();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = f.row(j);
    const int tok = m0 + row;
    const int64_t tv = tok < a.rows ? a.t[tok] : -1;
    const bool rok = tok < a.rows && !a.ign.skip(tv);   // an ignored token's row of G is zero
    const float l = rok ? a.lse[tok] : 0.f;
#pragma unroll
    for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c0 = f.col0(i, q);
        float gv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = n0 + c0 + e;
          float x = 0.f;
          if (rok && v < a.V) {
            x = fast_exp(acc[i][j][4 * q + e] - l);
            if (v == tv) x -= 1.f;
            x *= gscale;
          }
          gv[e] = x;
        }
        *reinterpret_cast<u32x2*>(g + g_off(row, c0 >> 3) + (c0 & 7) * 2) =
            u32x2{pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};
      }
  }
  __syncthreads();

  // 3. dx and dW partials for every 256-wide hidden slice
  char* ring = smem + kSmemBytes;
  const int kv = min(kTile, a.V - n0);      // valid vocabulary rows of the tile
  const int kt_ = min(kTile, a.rows - m0);  // valid token rows of the tile
  const uint32_t row_bytes = (uint32_t)a.H * 4u;
  const i32x4 dx_rsrc = make_rsrc(a.dx_acc, (uint32_t)((int64_t)a.rows * a.H * 4));
  const i32x4 dw_rsrc = make_rsrc(a.dw_acc, (uint32_t)((int64_t)a.V * a.H * 4));
  for (int hb = 0; hb < a.tiles_h; ++hb) {
    const int h0 = hb * kTile;
    // Lane-dependent atomic offsets are formed here from an opaque copy of the lane id, so the
    // compiler cannot hoist 128 of them over the loop; the per-register row offsets are
    // wave-uniform and travel in the scalar offset.
    int ol = lane;
    asm volatile("" : "+v"(ol));
    const int row_l = f.rowb + 4 * (ol >> 5);   // + 32 j + 8 (rg / 4) + rg % 4
    {
      Operand<bf16_t, false, kStreamBPW> S;           // W[n0 + v][h0 + h], contraction over v
      S.init(W + (int64_t)n0 * a.H, a.H, h0, a.H, (uint32_t)((int64_t)kv * a.H * 2));
      gemm_stream(acc, ring, S, kv, [&](int mnb, int ks, int ln) { return g_frag_k(g, mnb, ks, ln); });
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i) {
        const int h = h0 + f.colb + 32 * i + (ol & 31);
        if (h >= a.H) continue;
        const uint32_t vbase = (uint32_t)(m0 + row_l) * row_bytes + (uint32_t)h * 4u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int rg = 0; rg < 16; ++rg) {
            const int r = 32 * j + 8 * (rg >> 2) + (rg & 3);
            if (m0 + row_l + r < a.rows)
              llvm_amdgcn_raw_buffer_atomic_fadd_f32(acc[i][j][rg], dx_rsrc, (int)vbase, (int)((uint32_t)r * row_bytes), 0);
          }
      }
    }
    {
      Operand<bf16_t, false, kStreamBPW> S;           // x[m0 + token][h0 + h], contraction over tokens
      S.init(X + (int64_t)m0 * a.H, a.H, h0, a.H, (uint32_t)((int64_t)kt_ * a.H * 2));
      gemm_stream(acc, ring, S, kt_, [&](int mnb, int ks, int ln) { return g_frag_t(g, mnb, ks, ln); });
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i) {
        const int h = h0 + f.colb + 32 * i + (ol & 31);
        if (h >= a.H) continue;
        const uint32_t vbase = (uint32_t)(n0 + row_l) * row_bytes + (uint32_t)h * 4u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int rg = 0; rg < 16; ++rg) {
            const int r = 32 * j + 8 * (rg >> 2) + (rg & 3);
            if (n0 + row_l + r < a.V)
              llvm_amdgcn_raw_buffer_atomic_fadd_f32(acc[i][j][rg], dw_rsrc, (int)vbase, (int)((uint32_t)r * row_bytes), 0);
          }
      }
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(FillArgs a) {
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < a.n;
       i += (int64_t)gridDim.x * blockDim.x * 4)
    *reinterpret_cast<f32x4*>(a.p + i) = f32x4{0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(CastArgs a) {
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < a.n;
       i += (int64_t)gridDim.x * blockDim.x * 4) {
    f32x4 v = *reinterpret_cast<const f32x4*>(a.src + i);
    u32x2* p = reinterpret_cast<u32x2*>(static_cast<bf16_t*>(a.dst) + i);
    if (a.accumulate) {
      const u32x2 old = *p;
      v[0] += bf16_to_f32(old[0] & 0xffffu);
      v[1] += bf16_to_f32(old[0] >> 16);
      v[2] += bf16_to_f32(old[1] & 0xffffu);
      v[3] += bf16_to_f32(old[1] >> 16);
    }
    *p = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

static inline int grid_for(int64_t n4) {
  int64_t b = (n4 + 255) / 256;
  if (b > 256 * 16) b = 256 * 16;
  return (int)(b < 1 ? 1 : b);
}

hipError_t launch_fused_bwd(const FusedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fused_bwd_kernel, dim3(a.tiles_m * a.tiles_n), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill_zero(const FillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(a.n / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const CastArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid_for(a.n / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace flce
