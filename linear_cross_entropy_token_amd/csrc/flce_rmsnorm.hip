// RMSNorm in front of the LM head, for gfx950 (the final normalisation of the
// "Unsloth deep architecture" page, section on RMSNorm and its backward as one
// kernel: RMS(h) = sqrt(mean_k h_k^2 + eps), x = h / RMS(h) * gamma; the
// backward keeps only h and one rstd = 1 / RMS per row and produces dh and
// dgamma together).
//
// Used per token chunk by flce_rmsnorm_forward_backward: the forward writes the
// chunk's x (input dtype, one rounding) and rstd into the workspace; the FLCE
// chunk turns x into the chunk's fp32 dL/dx; the backward turns that into dh
// rows and per-block dgamma partials, which a fixed-order column sum folds into
// an fp32 dgamma accumulator.  All three are memory-bound row kernels: 16-byte
// vector accesses, fp32 arithmetic, block reductions through LDS.
#include "flce_device.hpp"
#include "flce_internal.hpp"

namespace flce {

constexpr int kRmsThreads = 256;

template <typename T> struct Vec;   // one 16-byte chunk of T
template <> struct Vec<bf16_t> {
  static constexpr int E = 8;
  typedef u32x4 raw;
  static __device__ __forceinline__ void to_f32(raw r, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(r[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(r[i] >> 16);
    }
  }
  static __device__ __forceinline__ raw from_f32(const float (&v)[8]) {
    return raw{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
};
template <> struct Vec<float> {
  static constexpr int E = 4;
  typedef f32x4 raw;
  static __device__ __forceinline__ void to_f32(raw r, float (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r[i];
  }
  static __device__ __forceinline__ raw from_f32(const float (&v)[4]) { return raw{v[0], v[1], v[2], v[3]}; }
};

template <typename T>
__device__ __forceinline__ void load_f32(const T* p, float (&v)[Vec<T>::E]) {
  Vec<T>::to_f32(*reinterpret_cast<const typename Vec<T>::raw*>(p), v);
}

// Sum over the block (256 threads = 4 waves); every thread gets the total.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();   // red is free (a previous call's readers are done)
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------------------------
// forward: one block per row
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kRmsThreads) void rms_fwd_kernel(RmsFwdArgs a) {
  __shared__ float red[4];
  constexpr int E = Vec<T>::E;
  const int r = blockIdx.x;
  const int nc = a.H / E;   // 16-byte chunks per row (H % 8 == 0)
  const T* h = static_cast<const T*>(a.h) + (int64_t)r * a.H;
  const T* g = static_cast<const T*>(a.gamma);
  float ss = 0.f;
  for (int c = threadIdx.x; c < nc; c += kRmsThreads) {
    float v[E];
    load_f32(h + c * E, v);
#pragma unroll
    for (int e = 0; e < E; ++e) ss += v[e] * v[e];
  }
  ss = block_sum(ss, red);
  const float rstd = 1.0f / sqrtf(ss / (float)a.H + a.eps);
  T* x = static_cast<T*>(a.x) + (int64_t)r * a.H;
  for (int c = threadIdx.x; c < nc; c += kRmsThreads) {
    float v[E], w[E];
    load_f32(h + c * E, v);
    load_f32(g + c * E, w);
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = v[e] * rstd * w[e];
    *reinterpret_cast<typename Vec<T>::raw*>(x + c * E) = Vec<T>::from_f32(v);
  }
  if (threadIdx.x == 0) a.rstd[r] = rstd;
}

// ---------------------------------------------------------------------------
// backward: kRmsRowsPerBlock rows per block; the block's dgamma partial sits in
// LDS (one fp32 per column, each column owned by one thread, so no atomics)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kRmsThreads) void rms_bwd_kernel(RmsBwdArgs a) {
  extern __shared__ float dg[];   // [H]
  __shared__ float red[4];
  constexpr int E = Vec<T>::E;
  const int nc = a.H / E;
  const T* g = static_cast<const T*>(a.gamma);
  for (int c = threadIdx.x; c < nc; c += kRmsThreads)
#pragma unroll
    for (int e = 0; e < E; ++e) dg[c * E + e] = 0.f;
  const int r0 = blockIdx.x * kRmsRowsPerBlock;
  const int r1 = min(r0 + kRmsRowsPerBlock, a.rows);
  const float inv_h = 1.0f / (float)a.H;
  for (int r = r0; r < r1; ++r) {
    const float* dx = a.dx + (int64_t)r * a.H;
    const T* h = static_cast<const T*>(a.h) + (int64_t)r * a.H;
    const float rstd = a.rstd[r];
    float s = 0.f;   // sum_k dx_k g_k h_k
    for (int c = threadIdx.x; c < nc; c += kRmsThreads) {
      float hv[E], gv[E];
      load_f32(h + c * E, hv);
      load_f32(g + c * E, gv);
      const float* d = dx + c * E;
#pragma unroll
      for (int e = 0; e < E; ++e) s += d[e] * gv[e] * hv[e];
    }
    s = block_sum(s, red);
    const float k = rstd * rstd * s * inv_h;
    for (int c = threadIdx.x; c < nc; c += kRmsThreads) {
      float hv[E], gv[E], out[E];
      load_f32(h + c * E, hv);
      load_f32(g + c * E, gv);
      const float* d = dx + c * E;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        out[e] = rstd * (d[e] * gv[e] - hv[e] * k);
        dg[c * E + e] += d[e] * hv[e] * rstd;
      }
      const int64_t o = (int64_t)r * a.H + c * E;
      if (a.dh_fp32) {
        float* p = static_cast<float*>(a.dh) + o;
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          f32x4 v{out[e], out[e + 1], out[e + 2], out[e + 3]};
          if (a.accumulate) v += *reinterpret_cast<const f32x4*>(p + e);
          *reinterpret_cast<f32x4*>(p + e) = v;
        }
      } else {
        bf16_t* p = static_cast<bf16_t*>(a.dh) + o;
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          float w0 = out[e], w1 = out[e + 1], w2 = out[e + 2], w3 = out[e + 3];
          if (a.accumulate) {
            const u32x2 old = *reinterpret_cast<const u32x2*>(p + e);
            w0 += bf16_to_f32(old[0] & 0xffffu);
            w1 += bf16_to_f32(old[0] >> 16);
            w2 += bf16_to_f32(old[1] & 0xffffu);
            w3 += bf16_to_f32(old[1] >> 16);
          }
          *reinterpret_cast<u32x2*>(p + e) = u32x2{pack_bf16x2(w0, w1), pack_bf16x2(w2, w3)};
        }
      }
    }
  }
  float* part = a.part + (int64_t)blockIdx.x * a.H;
  for (int c = threadIdx.x; c < nc; c += kRmsThreads)
#pragma unroll
    for (int e = 0; e < E; e += 4)
      *reinterpret_cast<f32x4*>(part + c * E + e) =
          f32x4{dg[c * E + e], dg[c * E + e + 1], dg[c * E + e + 2], dg[c * E + e + 3]};
}

// acc[k] += sum over blocks of part[b][k] in a fixed order (bitwise repeatable): a block takes 32
// columns; its 8 row groups each sum every 8th partial row (coalesced 128-byte row segments),
// then group 0 adds the 8 group sums in order.
constexpr int kReduceCols = 32, kReduceGroups = 8;
__global__ __launch_bounds__(kReduceCols * kReduceGroups) void rms_reduce_kernel(RmsReduceArgs a) {
  __shared__ float grp[kReduceGroups][kReduceCols];
  const int c = threadIdx.x % kReduceCols;
  const int rg = threadIdx.x / kReduceCols;
  const int k = blockIdx.x * kReduceCols + c;
  float s = 0.f;
  if (k < a.H)
    for (int b = rg; b < a.nblk; b += kReduceGroups) s += a.part[(int64_t)b * a.H + k];
  grp[rg][c] = s;
  __syncthreads();
  if (rg == 0 && k < a.H) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < kReduceGroups; ++g) t += grp[g][c];
    a.acc[k] += t;
  }
}

hipError_t launch_rms_fwd(In in, const RmsFwdArgs& a, hipStream_t s) {
  if (in == In::BF16) hipLaunchKernelGGL(rms_fwd_kernel<bf16_t>, dim3(a.rows), dim3(kRmsThreads), 0, s, a);
  else hipLaunchKernelGGL(rms_fwd_kernel<float>, dim3(a.rows), dim3(kRmsThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rms_bwd(In in, const RmsBwdArgs& a, hipStream_t s) {
  const int nblk = (a.rows + kRmsRowsPerBlock - 1) / kRmsRowsPerBlock;
  const size_t lds = (size_t)a.H * sizeof(float);
  if (in == In::BF16) hipLaunchKernelGGL(rms_bwd_kernel<bf16_t>, dim3(nblk), dim3(kRmsThreads), lds, s, a);
  else hipLaunchKernelGGL(rms_bwd_kernel<float>, dim3(nblk), dim3(kRmsThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_rms_reduce(const RmsReduceArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(rms_reduce_kernel, dim3((a.H + kReduceCols - 1) / kReduceCols),
                     dim3(kReduceCols * kReduceGroups), 0, s, a);
  return hipGetLastError();
}

}  // namespace flce
