// HIP kernels of the token-chunked FLCE path for gfx950.
//
// Per token chunk (the four steps of the core idea of the "Fused Linear
// Cross-Entropy" page, 42jerrykim.github.io):
//   logits_lse   z = x_c W^T on MFMA; the epilogue reduces each row of the
//                256-wide vocabulary tile to (max, sum exp(z - max)) with
//                half-wave butterflies, picks up the target logit, and stores
//                z into the chunk buffer (online-softmax statistics as on the
//                "Unsloth deep architecture" page, streaming CE kernel).
//   lse_combine  lse_n = M + ln sum_j s_j e^(m_j - M) over the vocab tiles,
//                per-row loss lse_n - z[n, t_n].
//   dlogits      G = (exp(z - lse) - onehot(t)) / N written over z
//                (softmax - one_hot in the same buffer, step 2).
//   dx           dx_c = G W (contraction over the vocabulary, split-K).
//   dw           dW (+)= G^T x_c (contraction over the chunk's tokens).
// and once per call: finalize, loss = sum_n loss_n / N (deterministic).
#include "flce_device.hpp"
#include "flce_internal.hpp"

namespace flce {

constexpr int BM = kTileM;
constexpr int BN = kTileN;
constexpr int kSmemBytes = 2 * (BM + BN) * kRowBytes;   // 128 KiB: two k-slice stages

// ---------------------------------------------------------------------------
// logits + LSE partials + target gather (+ z store)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void logits_lse_kernel(LogitsArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x;
  const int L = xcd_remap(blockIdx.x, a.tiles_m * a.tiles_n);
  const int tm = L % a.tiles_m;
  const int tn = L / a.tiles_m;
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const T* X = static_cast<const T*>(a.x);
  const T* W = static_cast<const T*>(a.W);

  f32x16 acc[BM / 64][BN / 64];
  gemm_mainloop<T, BM, BN, KMajorLoader<T, BM>, KMajorLoader<T, BN>>(
      acc, smem, 0, a.H,
      [&](KMajorLoader<T, BM>& l, int k0) { l.load(X, a.H, m0, a.rows, k0, a.H, tid); },
      [&](KMajorLoader<T, BN>& l, int k0) { l.load(W, a.H, n0, a.V, k0, a.H, tid); });

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  float* red = reinterpret_cast<float*>(smem);                 // [4][BM]: max wn0, max wn1, sum wn0, sum wn1
  int* trel = reinterpret_cast<int*>(smem + 4 * BM * sizeof(float));
  if (tid < BM) {
    const int r = m0 + tid;
    int rel = -1;
    if (r < a.rows) {
      const int64_t d = a.t[r] - (int64_t)n0;
      rel = (d >= 0 && d < BN) ? (int)d : -1;
    }
    trel[tid] = rel;
  }
  __syncthreads();

  const float ninf = -__builtin_inff();
  T* Z = static_cast<T*>(a.z);
#pragma unroll
  for (int i = 0; i < BM / 64; ++i) {
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) {
      const int row = wm * (BM / 2) + 32 * i + 8 * (rg >> 2) + 4 * (lane >> 5) + (rg & 3);
      const int grow = m0 + row;
      float mx = ninf;
#pragma unroll
      for (int j = 0; j < BN / 64; ++j) {
        const int col = wn * (BN / 2) + 32 * j + (lane & 31);
        if (n0 + col < a.V) mx = fmaxf(mx, acc[i][j][rg]);
      }
      mx = half_max(mx);
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < BN / 64; ++j) {
        const int col = wn * (BN / 2) + 32 * j + (lane & 31);
        if (n0 + col < a.V) s += fast_exp(acc[i][j][rg] - mx);
      }
      s = half_sum(s);
      if ((lane & 31) == 0) {
        red[wn * BM + row] = mx;
        red[(2 + wn) * BM + row] = s;
      }
      if (grow < a.rows) {
        const int tr = trel[row];
#pragma unroll
        for (int j = 0; j < BN / 64; ++j) {
          const int col = wn * (BN / 2) + 32 * j + (lane & 31);
          if (col == tr) a.zt[grow] = acc[i][j][rg];
          if (Z != nullptr && n0 + col < a.V) Z[(int64_t)grow * a.ldz + n0 + col] = from_f32<T>(acc[i][j][rg]);
        }
      }
    }
  }
  __syncthreads();
  if (tid < BM && m0 + tid < a.rows) {
    const float M0 = red[tid], M1 = red[BM + tid];
    const float S0 = red[2 * BM + tid], S1 = red[3 * BM + tid];
    const float M = fmaxf(M0, M1);
    const float S = (M0 == ninf ? 0.f : S0 * fast_exp(M0 - M)) + (M1 == ninf ? 0.f : S1 * fast_exp(M1 - M));
    a.pm[(int64_t)tn * a.pstride + m0 + tid] = M;
    a.ps[(int64_t)tn * a.pstride + m0 + tid] = S;
  }
}

// ---------------------------------------------------------------------------
// per-row combine of the vocabulary-tile partials
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lse_combine_kernel(CombineArgs a) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= a.rows) return;
  const float ninf = -__builtin_inff();
  float M = ninf;
  for (int j = 0; j < a.tiles_n; ++j) M = fmaxf(M, a.pm[(int64_t)j * a.pstride + r]);
  float S = 0.f;
  for (int j = 0; j < a.tiles_n; ++j) {
    const float m = a.pm[(int64_t)j * a.pstride + r];
    if (m != ninf) S += a.ps[(int64_t)j * a.pstride + r] * fast_exp(m - M);
  }
  const float lse = M + fast_log(S);
  const int64_t tv = a.t[r];
  const bool ok = tv >= 0 && tv < a.V;
  a.lse[r] = lse;
  a.loss_rows[r] = ok ? lse - a.zt[r] : __builtin_nanf("");
  if (!ok) atomicOr(a.flag, 1);
}

// ---------------------------------------------------------------------------
// G = (exp(z - lse) - onehot) / N, in place, zero in the padding columns
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dlogits_kernel(DlogitsArgs a) {
  constexpr int E = Elem<T>::E;
  const int64_t per_row = a.ldz / E;
  const int64_t total = per_row * a.rows;
  T* Z = static_cast<T*>(a.z);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(idx / per_row);
    const int c0 = (int)(idx - (int64_t)r * per_row) * E;
    const float l = a.lse[r];
    const int64_t tv = a.t[r];
    u32x4* p = reinterpret_cast<u32x4*>(Z + (int64_t)r * a.ldz + c0);
    u32x4 v = *p;
    T* e = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const int col = c0 + k;
      float g = 0.f;
      if (col < a.V) {
        g = fast_exp(to_f32<T>(e[k]) - l);
        if (col == tv) g -= 1.f;
        g *= a.inv_n;
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
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x;
  const int tiles = a.tiles_m * a.tiles_n;
  const int L = xcd_remap(blockIdx.x, tiles * a.splits);
  const int split = L / tiles;
  const int rem = L - split * tiles;
  const int tn = rem % a.tiles_n;
  const int tm = rem / a.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int ks = split * a.k_per_split;
  const int ke = min((int64_t)ks + a.k_per_split, a.ldg);
  const int kw = min(ke, a.V);
  const T* G = static_cast<const T*>(a.g);
  const T* W = static_cast<const T*>(a.W);

  f32x16 acc[BM / 64][BN / 64];
  gemm_mainloop<T, BM, BN, KMajorLoader<T, BM>, MNMajorLoader<T, BN>>(
      acc, smem, ks, ke,
      [&](KMajorLoader<T, BM>& l, int k0) { l.load(G, a.ldg, m0, a.rows, k0, ke, tid); },
      [&](MNMajorLoader<T, BN>& l, int k0) { l.load(W, a.H, n0, a.H, k0, kw, tid); });

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < BM / 64; ++i)
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) {
      const int grow = m0 + wm * (BM / 2) + 32 * i + 8 * (rg >> 2) + 4 * (lane >> 5) + (rg & 3);
      if (grow >= a.rows) continue;
#pragma unroll
      for (int j = 0; j < BN / 64; ++j) {
        const int col = n0 + wn * (BN / 2) + 32 * j + (lane & 31);
        if (col >= a.H) continue;
        const float v = acc[i][j][rg];
        const int64_t o = (int64_t)grow * a.H + col;
        if (a.splits > 1) {
          a.part[split * a.part_stride + o] = v;
        } else if (a.dx_fp32) {
          static_cast<float*>(a.dx)[o] = v;
        } else {
          static_cast<bf16_t*>(a.dx)[o] = f32_to_bf16(v);
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
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.dx) + i) = s;
    } else {
      bf16_t* o = static_cast<bf16_t*>(a.dx) + i;
      uint32_t lo = f32_to_bf16(s[0]) | ((uint32_t)f32_to_bf16(s[1]) << 16);
      uint32_t hi = f32_to_bf16(s[2]) | ((uint32_t)f32_to_bf16(s[3]) << 16);
      reinterpret_cast<uint32_t*>(o)[0] = lo;
      reinterpret_cast<uint32_t*>(o)[1] = hi;
    }
  }
}

// ---------------------------------------------------------------------------
// dW (+)= G^T x_c
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void dw_kernel(DwArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x;
  const int L = xcd_remap(blockIdx.x, a.tiles_m * a.tiles_n);
  const int tn = L % a.tiles_n;
  const int tm = L / a.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const T* G = static_cast<const T*>(a.g);
  const T* X = static_cast<const T*>(a.x);

  f32x16 acc[BM / 64][BN / 64];
  gemm_mainloop<T, BM, BN, MNMajorLoader<T, BM>, MNMajorLoader<T, BN>>(
      acc, smem, 0, a.rows,
      [&](MNMajorLoader<T, BM>& l, int k0) { l.load(G, a.ldg, m0, (int)a.ldg, k0, a.rows, tid); },
      [&](MNMajorLoader<T, BN>& l, int k0) { l.load(X, a.H, n0, a.H, k0, a.rows, tid); });

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < BM / 64; ++i)
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) {
      const int v = m0 + wm * (BM / 2) + 32 * i + 8 * (rg >> 2) + 4 * (lane >> 5) + (rg & 3);
      if (v >= a.V) continue;
#pragma unroll
      for (int j = 0; j < BN / 64; ++j) {
        const int h = n0 + wn * (BN / 2) + 32 * j + (lane & 31);
        if (h >= a.H) continue;
        const int64_t o = (int64_t)v * a.H + h;
        float val = acc[i][j][rg];
        if (a.dw_fp32) {
          float* p = static_cast<float*>(a.dW) + o;
          if (a.accumulate) val += *p;
          *p = val;
        } else {
          bf16_t* p = static_cast<bf16_t*>(a.dW) + o;
          if (a.accumulate) val += bf16_to_f32(*p);
          *p = f32_to_bf16(val);
        }
      }
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
  if (threadIdx.x == 0) *a.loss = (float)(part[0] / (double)a.n);
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
  hipLaunchKernelGGL(lse_combine_kernel, dim3((a.rows + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dlogits(In in, const DlogitsArgs& a, hipStream_t s) {
  const int E = in == In::BF16 ? 8 : 4;
  const int grid = grid_elementwise(a.ldz / E * a.rows, 256);
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

}  // namespace flce
