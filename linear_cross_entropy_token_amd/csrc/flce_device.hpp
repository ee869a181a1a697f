// Device-side building blocks of the FLCE kernels for gfx950 (MI355X).
//
// Every dense contraction of the path (logits = x W^T, dx = G W, dW = G^T x)
// runs on one MFMA tile engine: a 256-thread workgroup (4 wave64s in a 2x2
// arrangement) owns a BM x BN output tile, walks the contraction in 128-byte
// k-slices (64 bf16 or 32 fp32 values) staged through LDS with two buffers,
// and accumulates in fp32 registers with v_mfma_f32_32x32x16_bf16 (bf16
// inputs) or v_mfma_f32_32x32x2_f32 (fp32 inputs).
//
// LDS holds both operands "k-contiguous": one 128-byte row per output row
// (A) or column (B), made of eight 16-byte chunks, each chunk holding the
// consecutive k-values one lane feeds to an MFMA.  Chunk c of row r is
// stored at chunk position c ^ swz(r), which keeps the 16-byte accesses of
// every 8-lane group on distinct banks for the MFMA reads and for both
// loaders' writes.
//
// Operands that are stored k-contiguous in HBM (x and W for the logits, G for
// dx) are copied chunk by chunk.  Operands stored with the contraction index
// as the *row* (W for dx; G and x for dW) are read as E x E blocks (E rows of
// one 16-byte chunk, E = 16 / sizeof(T)), transposed in registers and
// written as E k-contiguous chunks, so every global read stays a coalesced
// 16-byte load.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

typedef uint16_t bf16_t;   // bf16 storage (raw bits)

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;          // one LDS operand row = one k-slice
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Elem;
template <> struct Elem<bf16_t> { static constexpr int E = 8; };   // values per 16-byte chunk
template <> struct Elem<float>  { static constexpr int E = 4; };

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {   // round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return f32_to_bf16(f); }
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float fast_log(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// Butterfly reductions over the 32 lanes of one half-wave (lane bit 5 fixed).
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Global -> register -> LDS loaders for one BMN x (one k-slice) operand tile.
// ---------------------------------------------------------------------------

// Operand stored [MN][K] with K contiguous (row stride ld elements).
// Requires k_end % E == 0 (chunk-granular k bound) and 16-byte aligned rows.
template <typename T, int BMN>
struct KMajorLoader {
  static constexpr int E = Elem<T>::E;
  static constexpr int PER = BMN * 8 / kThreads;   // 16-byte chunks per thread
  u32x4 r[PER];

  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int mn0, int mn_end,
                                       int k0, int k_end, int tid) {
    const int c = tid & 7;
    const int k = k0 + c * E;
    const bool kok = k < k_end;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int mn = mn0 + (tid >> 3) + 32 * p;
      if (kok && mn < mn_end) {
        r[p] = *reinterpret_cast<const u32x4*>(base + (int64_t)mn * ld + k);
      } else {
        r[p] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int row = (tid >> 3) + 32 * p;
      *reinterpret_cast<u32x4*>(lds + lds_off(row, tid & 7)) = r[p];
    }
  }
};

// Operand stored [K][MN] with MN contiguous (row stride ld elements): the
// contraction index is the row.  Requires mn_end % E == 0; k bound is exact.
template <typename T, int BMN>
struct MNMajorLoader {
  static constexpr int E = Elem<T>::E;
  static constexpr int MNC = BMN / E;                    // 16-byte chunks across MN
  static constexpr int PER = 8 * MNC / kThreads;         // E x E blocks per thread
  static_assert(PER >= 1, "tile too small for the transposing loader");
  u32x4 r[PER][E];

  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int mn0, int mn_end,
                                       int k0, int k_end, int tid) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int b = tid + kThreads * q;
      const int mc = b % MNC;
      const int kg = b / MNC;
      const int mn = mn0 + mc * E;
      const bool mnok = mn < mn_end;
#pragma unroll
      for (int rr = 0; rr < E; ++rr) {
        const int k = k0 + kg * E + rr;
        if (mnok && k < k_end) {
          r[q][rr] = *reinterpret_cast<const u32x4*>(base + (int64_t)k * ld + mn);
        } else {
          r[q][rr] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int b = tid + kThreads * q;
      const int mc = b % MNC;
      const int kg = b / MNC;
      if constexpr (E == 8) {
        // 8x8 transpose of 16-bit values: out[j] holds column j of the block.
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u32x4 o;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const uint32_t a = r[q][2 * qd][j >> 1];
            const uint32_t c = r[q][2 * qd + 1][j >> 1];
            o[qd] = (j & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
          }
          *reinterpret_cast<u32x4*>(lds + lds_off(mc * 8 + j, kg)) = o;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x4 o{r[q][0][j], r[q][1][j], r[q][2][j], r[q][3][j]};
          *reinterpret_cast<u32x4*>(lds + lds_off(mc * 4 + j, kg)) = o;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA on one LDS stage.  Wave w of the 2x2 arrangement owns rows
// wm*(BM/2) .. +BM/2 and columns wn*(BN/2) .. +BN/2 as TM x TN blocks of 32x32.
// Output element (row, col) of block (i, j), register rg of lane l:
//   row = 32 i + 8 (rg / 4) + 4 (l / 32) + rg % 4,   col = 32 j + l % 32.
// ---------------------------------------------------------------------------
template <typename T, int TM, int TN>
__device__ __forceinline__ void mma_stage(f32x16 (&acc)[TM][TN], const char* As, const char* Bs,
                                          int arow0, int brow0, int lane) {
  const int lr = lane & 31;
  const int hi = lane >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = 2 * s + hi;
    u32x4 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = *reinterpret_cast<const u32x4*>(As + lds_off(arow0 + 32 * i + lr, c));
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = *reinterpret_cast<const u32x4*>(Bs + lds_off(brow0 + 32 * j + lr, c));
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (Elem<T>::E == 8) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                              __builtin_bit_cast(bf16x8, b[j]),
                                                              acc[i][j], 0, 0, 0);
        } else {
          const f32x4 af = __builtin_bit_cast(f32x4, a[i]);
          const f32x4 bf = __builtin_bit_cast(f32x4, b[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[e], acc[i][j], 0, 0, 0);
        }
      }
    }
  }
}

// Double-buffered main loop over k-slices [k_begin, k_end).
template <typename T, int BM, int BN, class LA, class LB, class FA, class FB>
__device__ __forceinline__ void gemm_mainloop(f32x16 (&acc)[BM / 64][BN / 64], char* smem,
                                              int k_begin, int k_end, FA&& loadA, FB&& loadB) {
  constexpr int TM = BM / 64, TN = BN / 64;
  constexpr int BK = kRowBytes / (int)sizeof(T);
  constexpr int STAGE = (BM + BN) * kRowBytes;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int arow0 = (wave >> 1) * (BM / 2);
  const int brow0 = (wave & 1) * (BN / 2);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  LA la;
  LB lb;
  const int nk = (k_end - k_begin + BK - 1) / BK;
  if (nk <= 0) return;
  loadA(la, k_begin);
  loadB(lb, k_begin);
  la.store(smem, tid);
  lb.store(smem + BM * kRowBytes, tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE;
    char* nxt = smem + ((kt + 1) & 1) * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      loadA(la, k_begin + (kt + 1) * BK);
      loadB(lb, k_begin + (kt + 1) * BK);
    }
    mma_stage<T, TM, TN>(acc, cur, cur + BM * kRowBytes, arow0, brow0, lane);
    if (more) {
      la.store(nxt, tid);
      lb.store(nxt + BM * kRowBytes, tid);
    }
    __syncthreads();
  }
}

// Maps the hardware workgroup index to a logical tile index so that each of
// the 8 XCDs (workgroups are dealt to XCDs round-robin) works on one
// contiguous range of logical tiles, whose operands then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int xcd = bid & 7;
  const int local = bid >> 3;
  const int base = total >> 3;
  const int rem = total & 7;
  return xcd * base + (xcd < rem ? xcd : rem) + local;
}

}  // namespace flce
