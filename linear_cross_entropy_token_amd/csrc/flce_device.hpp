// Device-side building blocks of the FLCE kernels for gfx950 (MI355X).
//
// Every dense contraction of the path (logits = x W^T, dx = G W, dW = G^T x)
// runs on one MFMA tile engine:
//  * a 512-thread workgroup (8 wave64s, 2 x 4) owns a 256 x 256 output tile;
//    each wave owns 128 x 64 as 2 x 4 blocks of 32 x 32 accumulated in fp32
//    by v_mfma_f32_32x32x16_bf16 (bf16 inputs) or v_mfma_f32_32x32x2_f32
//    (fp32 inputs);
//  * the contraction is walked in k-slices of 128 bytes per operand row
//    (64 bf16 / 32 fp32, one full cache line per k-major row) through an
//    LDS ring: operand tiles are copied HBM -> LDS by buffer_load ... lds
//    (direct-to-LDS DMA, no VGPR staging) ahead of the MFMAs that consume
//    them; out-of-range rows/columns come back as zeros from the buffer
//    range check, so ragged edges need no branches.  (Measured on MI355X:
//    full-line requests beat half-line requests with more stages.)
//  * the two waves of each SIMD run a ping-pong schedule: one multiplies a
//    whole k-slice from registers while the other reads the next fragments
//    from LDS and issues copies.  gemm_tile uses a 2-stage ring (2 x 64 KiB);
//    gemm_tile_balanced uses all 160 KiB (3 slots for one operand, 2 for the
//    other) so that each phase carries half a slice of copies.
//  * an operand stored with the contraction index contiguous ("k-major": x
//    and W for the logits, G for dx) is kept k-major in LDS and read with
//    ds_read_b128; an operand whose contraction index is the ROW ("mn-major":
//    W for dx, G and x for dW) is kept mn-major in LDS and read with the
//    gfx950 transposing read ds_read_b64_tr_b16, so no operand is ever
//    transposed in HBM or in registers.
//
// MFMA roles: the MFMA's A input is the operand that indexes the OUTPUT
// COLUMNS and its B input the one that indexes the output rows.  Register
// rg of block (i, j) in lane l then holds
//   col = 32 i + 8 (rg / 4) + 4 (l / 32) + rg % 4,   row = 32 j + l % 32,
// so each lane owns runs of 4 consecutive columns of one row: epilogue loads
// and stores are 8- or 16-byte vectors and row reductions stay in registers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce_internal.hpp"

namespace flce {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef uint16_t bf16_t;   // bf16 storage (raw bits)

// Eight waves (two per SIMD) per 256 x 256 tile, each owning 128 rows x 64 columns
// (128 accumulator registers + 96 fragment registers for one k-slice); the two waves of a
// SIMD alternate between multiplying and reading LDS (the ping-pong schedule of gemm_tile).
constexpr int kWaves = 8;                           // waves per workgroup (2 rows x kWaveCols)
constexpr int kWaveCols = kWaves / 2;
constexpr int kColBlocks = 256 / kWaveCols / 32;    // 32-column MFMA blocks per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 256;             // output tile is kTile x kTile
constexpr int kStages = 2;                          // LDS ring depth
constexpr int kSliceBytes = kSliceBytesABI;         // bytes of one k-major operand row per slice
constexpr int kOpBytes = kTile * kSliceBytes;       // one operand's part of a stage (32 KiB)
constexpr int kStageBytes = 2 * kOpBytes;
constexpr int kSmemBytes = kStages * kStageBytes;   // 128 KiB
constexpr int kBlocksPerWave = kOpBytes / 1024 / kWaves; // 1 KiB DMA blocks per wave per operand and slice
constexpr int kSteps = kSliceBytes / 32;            // MFMA k-steps per slice
constexpr int kRowsPerBlock = 1024 / kSliceBytes;   // k-major rows per 1 KiB DMA block
constexpr int kLanesPerRow = kSliceBytes / 16;
constexpr uint32_t kOOB = 0xFFFFFF00u; // buffer offset beyond every valid range -> zeros
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Elem;
template <> struct Elem<bf16_t> { static constexpr int E = 8; };   // values per 16-byte chunk
template <> struct Elem<float>  { static constexpr int E = 4; };
template <typename T> constexpr int slice_k() { return kSliceBytes / (int)sizeof(T); }

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {   // round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}
template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return f32_to_bf16(f); }
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float fast_log(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// ---------------------------------------------------------------------------
// Buffer resources and direct-to-LDS copies.
// ---------------------------------------------------------------------------
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(
    i32x4 rsrc, __attribute__((address_space(3))) uint32_t* lds, int size, int voffset,
    int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// No-return fp32 atomic add through a raw buffer (vector memory, added in L2).
extern "C" __device__ float llvm_amdgcn_raw_buffer_atomic_fadd_f32(float v, i32x4 rsrc, int voffset, int soffset,
                                                                   int aux) __asm("llvm.amdgcn.raw.buffer.atomic.fadd.f32");

// Raw buffer over [base, base + bytes): reads at offsets >= bytes return zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int32_t)(uint32_t)(a & 0xffffffffu);
  r[1] = (int32_t)(uint32_t)((a >> 32) & 0xffffu);
  r[2] = (int32_t)bytes;
  r[3] = 0x00020000;
  return r;
}

// Lane l's 16 bytes at buffer offset voff land at lds + 16 l (lds is wave-uniform).
__device__ __forceinline__ void dma16(i32x4 rsrc, char* lds, uint32_t voff) {
  llvm_amdgcn_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) uint32_t*)lds, 16,
                                  (int)voff, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS layouts (bank-conflict-free for 128- and 256-byte-per-clock banking).
// k-major: 256 rows x 128 B; 16-byte chunk c of row r sits at chunk c ^ swz_k(r).
// mn-major (bf16): 64 k-rows x 512 B; 32-byte granule g of row r sits at g ^ swz_mn(r).
// mn-major (fp32): 32 k-rows x 1 KiB, unswizzled.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz_k(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }
__device__ __forceinline__ int swz_mn(int r) { return ((r & 1) ? 5 : 0) ^ (r & 2); }

// One operand: 256 indices along its "mn" dimension by one k-slice per stage, copied as
// 8 x BPW blocks of 1 KiB (BPW per wave).  KMAJOR: stored [mn][k] (k contiguous); otherwise
// stored [k][mn] (mn contiguous).  With BPW < kBlocksPerWave an mn-major slice holds fewer
// k-rows (2 per block for bf16).  All fields are wave-uniform (scalar registers); each
// lane's offsets are recomputed per slice, which costs a few VALU instructions and leaves
// the vector registers to accumulators and fragments (measured 4-6% faster on dx and dW
// than keeping per-lane offsets in registers).
template <typename T, bool KMAJOR, int BPW = kBlocksPerWave>
struct Operand {
  static constexpr bool kKMajor = KMAJOR;
  static constexpr int E = Elem<T>::E;
  static constexpr int ES = (int)sizeof(T);
  i32x4 rsrc;
  uint32_t ld_bytes;    // bytes per stored row
  int mn0, mn_end;      // first mn index of the tile; valid mn extent

  // ld: row stride (elements); rows beyond the buffer's bytes read as zero.
  __device__ __forceinline__ void init(const T* ptr, int64_t ld, int mn0_, int mn_end_, uint32_t bytes) {
    rsrc = make_rsrc(ptr, bytes);
    ld_bytes = (uint32_t)(ld * ES);
    mn0 = mn0_;
    mn_end = mn_end_;
  }

  // Copies the slice starting at contraction index k0 (k < k_end valid) into lds_op.
  // Offsets are 32-bit: every valid byte of the buffer lies below 2^32.  `lane`: the calling
  // lane (0..63), passed in so that callers decide where lane-dependent values are formed.
  __device__ __forceinline__ void issue(char* lds_op, int k0, int k_end, int wave, int lane) const {
#pragma unroll
    for (int i = 0; i < BPW; ++i) issue_block(lds_op, k0, k_end, wave * BPW + i, lane);
  }

  // Blocks vw * N .. vw * N + N - 1 of the slice (one wave of a group of 4 copying the whole slice).
  template <int N>
  __device__ __forceinline__ void issue_part(char* lds_op, int k0, int k_end, int vw, int lane) const {
#pragma unroll
    for (int i = 0; i < N; ++i) issue_block(lds_op, k0, k_end, vw * N + i, lane);
  }

  // 1 KiB block b (0 .. 8 BPW - 1) of the slice at k0.
  __device__ __forceinline__ void issue_block(char* lds_op, int k0, int k_end, int b, int lane) const {
    {
      int mn, kpos;
      uint32_t off;
      if constexpr (KMAJOR) {
        const int row = kRowsPerBlock * b + lane / kLanesPerRow;
        const int c = (lane % kLanesPerRow) ^ swz_k(row);
        mn = mn0 + row;
        kpos = k0 + c * E;
        off = (uint32_t)mn * ld_bytes + (uint32_t)kpos * ES;
      } else if constexpr (ES == 2) {
        const int row = 2 * b + (lane >> 5);
        const int p = lane & 31;
        const int c = (((p >> 1) ^ swz_mn(row)) << 1) | (p & 1);
        mn = mn0 + c * E;
        kpos = k0 + row;
        off = (uint32_t)kpos * ld_bytes + (uint32_t)mn * ES;
      } else {
        mn = mn0 + lane * E;
        kpos = k0 + b;
        off = (uint32_t)kpos * ld_bytes + (uint32_t)mn * ES;
      }
      dma16(rsrc, lds_op + b * 1024, (mn < mn_end && kpos < k_end) ? off : kOOB);
    }
  }
};

// Fragment of one 32-index block for k-step s (16 bf16 / 8 fp32 k-values; kSteps per slice):
// lane l supplies index mnb + l % 32 and the k-values 8 (l / 32) .. +7 (bf16) / 4 (l / 32) .. +3 (fp32).
//
// ASM (bf16 mn-major only): issue the transposing reads as inline assembly.  The compiler
// treats the transposing-read builtin as possibly aliasing every direct-to-LDS copy still in
// flight and inserts a wait for all of them (vmcnt(0)) before it, which stalls a wave that
// has just issued the next slice's copies for the whole copy latency (measured: dx 15%, dW 8%
// slower).  The ping-pong loops order copies and reads with their own waits and barriers and
// wait for these reads (lgkmcnt(0)) before the MFMAs use them, so the asm form is exact there;
// loops that rely on compiler-inserted waits must use the builtin.
template <typename T, bool KMAJOR, bool ASM = false>
__device__ __forceinline__ u32x4 read_frag(const char* op, int mnb, int s, int lane) {
  if constexpr (KMAJOR) {
    const int row = mnb + (lane & 31);
    const int c = 2 * s + (lane >> 5);
    return *reinterpret_cast<const u32x4*>(op + row * kSliceBytes + ((c ^ swz_k(row)) << 4));
  } else if constexpr (sizeof(T) == 2) {
    const int r = 16 * s + 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int g = (mnb >> 4) + ((lane >> 4) & 1);
    const int byte = 8 * (lane & 3);
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const lds_i16x4* p0 = (const lds_i16x4*)(op + r * 512 + ((g ^ swz_mn(r)) << 5) + byte);
    const lds_i16x4* p1 = (const lds_i16x4*)(op + (r + 4) * 512 + ((g ^ swz_mn(r + 4)) << 5) + byte);
    if constexpr (ASM) {   // p1 = p0 + 4 rows: swz_mn depends on r % 4 only
      const uint32_t a0 = (uint32_t)(uintptr_t)p0;
      u32x2 l2, h2;
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(l2) : "v"(a0));
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:2048" : "=v"(h2) : "v"(a0));
      return u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  } else {
    const int mn = mnb + (lane & 31);
    const int k = 8 * s + 4 * (lane >> 5);
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = *reinterpret_cast<const uint32_t*>(op + (k + e) * 1024 + mn * 4);
    return v;
  }
}

template <typename T>
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    const f32x4 af = __builtin_bit_cast(f32x4, a);
    const f32x4 bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[e], c, 0, 0, 0);
    return c;
  }
}

// Joins the workgroup barrier after this wave's outstanding copies (vmcnt) and/or LDS reads
// (lgkmcnt) have completed.  One asm statement between two scheduling barriers, so the compiler
// moves no instruction (memory access or MFMA) across it; the plain barrier carries no fence.
template <bool VM, bool LGKM>
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (VM && LGKM) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (VM) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (LGKM) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Waits for this wave's LDS reads; no instruction moves across it.
__device__ __forceinline__ void lgkm_wait() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// acc[i][j] += sum over k in [k_begin, k_end) of C[col 32i + ..][k] * R[row 32j + ..][k] for the
// wave's 128 x 64 part of the tile.  C and R fill their halves of each LDS stage.
//
// Ping-pong schedule.  The two waves of a SIMD (wave w and w + 4) take turns: in each phase
// (one barrier interval) one of them runs the 4 x kColBlocks x 4 MFMAs of a whole k-slice from
// registers while the other reads its fragments of the next slice from LDS and issues
// copies, so the matrix core never waits for the LDS pipe of its own wave.  With phases
// numbered from 0, waves 0-3 read slice kt in phase 2kt and multiply in 2kt+1; waves 4-7
// read it in 2kt+1 and multiply in 2kt+2.  Slice kt+1 is copied into the other stage
// during phase 2kt (both readers of the slice it replaces finished by phase 2kt-1): waves
// 0-3 copy their share after reading slice kt, waves 4-7 before multiplying slice kt-1, and
// every wave waits for its copies at the end of phase 2kt+1.  There are 2 nk + 1 phases per
// tile.
//
// SWAP exchanges the MFMA's A and B inputs (the row operand becomes A): register rg of block
// (i, j) in lane l then holds
//   row = 32 j + 8 (rg / 4) + 4 (l / 32) + rg % 4,   col = 32 i + l % 32,
// so the 32 lanes of a half-wave hold 32 consecutive columns of one row (the layout for
// epilogues that issue one atomic per element: each instruction touches two cache lines).
template <typename T, class OpC, class OpR, bool SWAP = false>
__device__ __forceinline__ void gemm_tile(f32x16 (&acc)[kColBlocks][4], char* smem, const OpC& C, const OpR& R,
                                          int k_begin, int k_end, int tid) {
  static_assert(kStages == 2 && kWaves == 8, "the ping-pong schedule pairs the waves of a SIMD over two stages");
  constexpr int BK = slice_k<T>();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar address arithmetic
  const int rowb = (wave / kWaveCols) * 128;
  const int colb = (wave % kWaveCols) * (kTile / kWaveCols);
#pragma unroll
  for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int nk = (k_end - k_begin + BK - 1) / BK;
  auto issue = [&](int kt) {
    char* st = smem + (kt % kStages) * kStageBytes;
    const int k0 = k_begin + kt * BK;
    C.issue(st, k0, k_end, wave, lane);
    R.issue(st + kOpBytes, k0, k_end, wave, lane);
  };
  u32x4 fa[kSteps][kColBlocks], fb[kSteps][4];
  auto read = [&](int kt) {
    const char* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i) fa[s][i] = read_frag<T, OpC::kKMajor, true>(st, colb + 32 * i, s, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[s][j] = read_frag<T, OpR::kKMajor, true>(st + kOpBytes, rowb + 32 * j, s, lane);
    }
  };
  auto multiply = [&]() {
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = SWAP ? mfma<T>(fb[s][j], fa[s][i], acc[i][j]) : mfma<T>(fa[s][i], fb[s][j], acc[i][j]);
  };
  if (nk > 0) issue(0);
  phase_barrier<true, false>();                 // slice 0 resident
  if (wave < kWaves / 2) {
    for (int kt = 0; kt < nk; ++kt) {
      read(kt);                                 // phase 2kt
      lgkm_wait();
      if (kt + 1 < nk) issue(kt + 1);
      phase_barrier<false, false>();
      multiply();                               // phase 2kt + 1
      phase_barrier<true, false>();
    }
    phase_barrier<false, false>();              // phase 2nk
  } else {
    if (1 < nk) issue(1);                       // phase 0
    phase_barrier<false, false>();
    for (int kt = 0; kt < nk; ++kt) {
      read(kt);                                 // phase 2kt + 1
      phase_barrier<true, true>();
      if (kt + 2 < nk) issue(kt + 2);           // phase 2kt + 2
      multiply();
      phase_barrier<false, false>();
    }
  }
  __syncthreads();   // LDS free for the epilogue
}

// Joins the barrier once this wave's copies have landed, except (keep8) the 8 it issued last.
__device__ __forceinline__ void vm_barrier_keep8(bool keep8) {
  __builtin_amdgcn_sched_barrier(0);
  if (keep8) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// gemm_tile over all 160 KiB of LDS: the column operand C in a 3-slot ring, the row operand R
// in a 2-slot ring, and the copies of each slice split between the two wave groups so that
// every phase carries half a slice of them, issued by the group that is reading (its matrix
// core is busy with the other group's MFMAs).  Phases as in gemm_tile: waves 0-3 read slice m
// in phase 2m and multiply it in 2m+1, waves 4-7 read it in 2m+1 and multiply it in 2m+2.
//   * waves 0-3, after reading slice m, copy R(m+1) (8 blocks each) into R slot (m+1) % 2,
//     whose previous slice m-1 was last read in phase 2m-1; they wait for it at the end of
//     phase 2m+1, one phase before its first reader;
//   * waves 4-7, after reading slice m, copy C(m+2) (8 blocks each) into C slot (m+2) % 3,
//     whose previous slice m-1 was last read in phase 2m-1; they wait for it at the end of
//     phase 2m+3 (keeping only the newer C(m+3) in flight), so C's copies get two phases.
// Measured against gemm_tile at the Llama-3 chunk: logits -11%, dx -3%; dW (both operands
// read with transposing reads, so its read phases are the longest) stays on gemm_tile.
constexpr int kDeepRingBytes = 5 * kOpBytes;   // 160 KiB
template <typename T, class OpC, class OpR, bool SWAP = false>
__device__ __forceinline__ void gemm_tile_balanced(f32x16 (&acc)[kColBlocks][4], char* smem, const OpC& C,
                                                   const OpR& R, int k_begin, int k_end, int tid) {
  static_assert(kWaves == 8 && kBlocksPerWave == 4, "two groups of 4 waves; 8 blocks per wave copy a slice");
  constexpr int BK = slice_k<T>();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vw = wave & 3;                       // position inside the wave group
  const int rowb = (wave / kWaveCols) * 128;
  const int colb = (wave % kWaveCols) * (kTile / kWaveCols);
#pragma unroll
  for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int nk = (k_end - k_begin + BK - 1) / BK;
  char* ringR = smem + 3 * kOpBytes;
  auto slot_c = [&](int kt) { return smem + (kt % 3) * kOpBytes; };
  auto slot_r = [&](int kt) { return ringR + (kt & 1) * kOpBytes; };
  u32x4 fa[kSteps][kColBlocks], fb[kSteps][4];
  auto read = [&](int kt) {
    const char* sc = slot_c(kt);
    const char* sr = slot_r(kt);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i) fa[s][i] = read_frag<T, OpC::kKMajor, true>(sc, colb + 32 * i, s, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[s][j] = read_frag<T, OpR::kKMajor, true>(sr, rowb + 32 * j, s, lane);
    }
  };
  auto multiply = [&]() {
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = SWAP ? mfma<T>(fb[s][j], fa[s][i], acc[i][j]) : mfma<T>(fa[s][i], fb[s][j], acc[i][j]);
  };
  if (nk > 0) {                                  // slice 0: every wave copies its share
    C.issue(slot_c(0), k_begin, k_end, wave, lane);
    R.issue(slot_r(0), k_begin, k_end, wave, lane);
  }
  if (wave < kWaves / 2) {
    vm_barrier_keep8(false);                     // slice 0 resident
    for (int m = 0; m < nk; ++m) {
      read(m);                                   // phase 2m
      lgkm_wait();
      if (m + 1 < nk) R.template issue_part<8>(slot_r(m + 1), k_begin + (m + 1) * BK, k_end, vw, lane);
      phase_barrier<false, false>();
      multiply();                                // phase 2m + 1
      vm_barrier_keep8(false);                   // R(m+1) resident
    }
    phase_barrier<false, false>();               // phase 2nk
  } else {
    if (1 < nk) C.template issue_part<8>(slot_c(1), k_begin + BK, k_end, vw, lane);
    vm_barrier_keep8(1 < nk);                    // slice 0 resident; C(1) may be in flight
    phase_barrier<false, false>();               // phase 0
    for (int m = 0; m < nk; ++m) {
      read(m);                                   // phase 2m + 1
      lgkm_wait();
      if (m + 2 < nk) C.template issue_part<8>(slot_c(m + 2), k_begin + (m + 2) * BK, k_end, vw, lane);
      vm_barrier_keep8(m + 2 < nk);              // C(m+1) resident
      multiply();                                // phase 2m + 2
      phase_barrier<false, false>();
    }
  }
  __syncthreads();   // LDS free for the epilogue
}

// Output coordinates of accumulator (i, j, q) in this lane: the 4 consecutive
// columns col0 .. col0 + 3 of one row (see the engine header).
struct Frag {
  int rowb, colb, lane;
  __device__ __forceinline__ int row(int j) const { return rowb + 32 * j + (lane & 31); }
  __device__ __forceinline__ int col0(int i, int q) const { return colb + 32 * i + 8 * q + 4 * (lane >> 5); }
};
__device__ __forceinline__ Frag frag_coords(int tid) {
  const int wave = tid >> 6;
  return Frag{(wave / kWaveCols) * 128, (wave % kWaveCols) * (kTile / kWaveCols), tid & 63};
}
__device__ __forceinline__ Frag frag_coords() { return frag_coords(threadIdx.x); }

// The thread's id through an empty asm statement: values derived from it are formed where this is
// called and cannot be hoisted above it (kernels that run several tile products in a loop use it
// so that each product's lane-dependent addresses stay out of the registers of the others).
__device__ __forceinline__ int opaque_tid() {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  return tid;
}

// Logical tile L -> (tm, tn): tiles walk m fastest inside groups of gm m-tiles that sweep
// all n, so the 32 tiles one XCD runs at a time form a gm x (32 / gm) block whose operand
// slices are shared in that XCD's L2 (4 x 8 needs 12 tile-slices of operands per k-step
// instead of 2 x 16's 18).
__device__ __forceinline__ void grouped_tile(int L, int TM, int TN, int gm, int& tm, int& tn) {
  const int per_group = gm * TN;
  const int g = L / per_group;
  const int first = g * gm;
  const int rows = min(TM - first, gm);
  const int r = L - g * per_group;
  tm = first + r % rows;
  tn = r / rows;
}
constexpr int kGroupM = 4;

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

// Adds the workgroup's lifetime, from construction to the end of its scope, to clk[0] in
// shader-clock ticks (s_memtime) and to clk[1] in 100 MHz real-time ticks (s_memrealtime) when clk
// is set: summed over the workgroups of a launch, their ratio is the shader clock it ran at.
struct ClockSpan {
  unsigned long long* clk;
  uint64_t t0, r0;
  __device__ explicit ClockSpan(unsigned long long* c) : clk(c), t0(0), r0(0) {
    if (clk != nullptr) {
      t0 = __builtin_amdgcn_s_memtime();
      r0 = __builtin_amdgcn_s_memrealtime();
    }
  }
  __device__ ~ClockSpan() {
    if (clk != nullptr && threadIdx.x == 0) {
      const uint64_t t1 = __builtin_amdgcn_s_memtime();
      const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
      atomicAdd(clk, (unsigned long long)(t1 - t0));
      atomicAdd(clk + 1, (unsigned long long)(r1 - r0));
    }
  }
};

}  // namespace flce
