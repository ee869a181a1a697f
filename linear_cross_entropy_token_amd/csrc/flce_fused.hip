// Fused FLCE variant, pass 2, for gfx950 (bf16 inputs), and the small elementwise kernels the
// fused path uses (accumulator clearing, fp32 -> bf16 output casts).
//
// Pass 1 (logits_lse without the logits store, then lse_combine) leaves the per-token
// log-sum-exp.  Pass 2 recomputes the logits block by block, turns them into dlogits in the
// recompute's epilogue and adds the dx and dW contributions into fp32 accumulators (the reduction
// by atomic adds that the "Unsloth deep architecture" page's streaming CE kernel uses); no [chunk, V]
// logits tensor is ever written.  The recomputation costs one extra forward product (8 N H V flops
// instead of 6 N H V).
#include "flce_device.hpp"
#include "flce_internal.hpp"

namespace flce {

// ---------------------------------------------------------------------------
// Pass 2.  Each add of a 256 x 256 partial tile into dx or dW costs one fp32 atomic per element, and
// an atomic cannot complete in an XCD's L2 (the eight L2s are not coherent with each other), so it
// travels to the memory side: a kernel that added one partial per (token tile, vocabulary tile)
// pair would make 2 rows V H / 256 adds per launch.  Here the plane is cut into blocks of bt x bv
// tiles (planned per launch, e.g. 32 x 42: 8192 tokens x 10,752 vocabulary ids, ~36x fewer adds),
// done in steps of two kernels (the dealing of blocks and items is StepPlan's, flce_internal.hpp):
//   Z (fused_z_kernel): each logits tile of the step's blocks is recomputed (contraction over H on
//     the tile engine) and turned into dlogits G = (exp(z - lse) - onehot) * scale, stored bf16 in
//     the block's slot (the dlogits tile of the FLCE page's step 2, for a block of tiles; slots are
//     workspace and are overwritten by the next step);
//   P (fused_p_kernel): for every 256-wide slice of H, the block's dx tiles (slot rows times W) and
//     dW tiles (slot columns times x) are formed on the same engine and added into the fp32
//     accumulators with atomics (the reduction by atomic adds of the "Unsloth deep architecture"
//     page's streaming CE kernel).
// The kernel boundary orders the slots' writes before their reads.  A group of workgroups (one
// XCD's) works on one block at a time, so each slot row or column that a product reads is fetched
// once into the XCD's L2 for the group's products of it (one per 256-wide slice of H).
// ---------------------------------------------------------------------------

// Adds a 256 x 256 fp32 tile in the SWAP accumulator layout into out[(row0 + r) H + col0 + c] with
// one atomic per element; rows >= row_end and columns >= H are skipped.
__device__ __forceinline__ void atomic_add_tile(const f32x16 (&acc)[kColBlocks][4], const i32x4& rsrc, int row0,
                                                int row_end, int col0, int H) {
  // lane-dependent offsets from an opaque copy of the thread id, so that the compiler does not
  // hoist 128 of them; the per-register row offsets are wave-uniform and go in the scalar offset
  const int tid = opaque_tid();
  const Frag f = frag_coords(tid);
  const int ol = tid & 63;
  const uint32_t row_bytes = (uint32_t)H * 4u;
  const int row_l = f.rowb + 4 * (ol >> 5);   // + 32 j + 8 (rg / 4) + rg % 4
#pragma unroll
  for (int i = 0; i < kColBlocks; ++i) {
    const int col = col0 + f.colb + 32 * i + (ol & 31);
    if (col >= H) continue;
    const uint32_t vbase = (uint32_t)(row0 + row_l) * row_bytes + (uint32_t)col * 4u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int rg = 0; rg < 16; ++rg) {
        const int r = 32 * j + 8 * (rg >> 2) + (rg & 3);
        if (row0 + row_l + r < row_end)
          llvm_amdgcn_raw_buffer_atomic_fadd_f32(acc[i][j][rg], rsrc, (int)vbase, (int)((uint32_t)r * row_bytes), 0);
      }
  }
}

// Stores a 256 x 256 fp32 tile in the engine's default accumulator layout (each lane holds runs of 4
// consecutive columns of one row) into out[(row0 + r) H + col0 + c] as bf16 (round to nearest even),
// adding the bf16 value already there when `add`: 8-byte loads and stores.  Rows >= row_end and
// columns >= H are skipped (H is a multiple of 8).  For tiles with exactly one producer.
__device__ __forceinline__ void store_tile_bf16(const f32x16 (&acc)[kColBlocks][4], bf16_t* out, int row0,
                                                int row_end, int col0, int H, bool add) {
  const Frag f = frag_coords(opaque_tid());
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = row0 + f.row(j);
    if (row >= row_end) continue;
#pragma unroll
    for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = col0 + f.col0(i, q);
        if (col >= H) continue;
        u32x2* p = reinterpret_cast<u32x2*>(out + (int64_t)row * H + col);
        f32x4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if (add) {
          const u32x2 old = *p;
          v[0] += bf16_to_f32(old[0] & 0xffffu);
          v[1] += bf16_to_f32(old[0] >> 16);
          v[2] += bf16_to_f32(old[1] & 0xffffu);
          v[3] += bf16_to_f32(old[1] >> 16);
        }
        *p = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  }
}

__global__ __launch_bounds__(kThreads, 1) void fused_z_kernel(FusedStepArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kDeepRingBytes];
  const StepPlan& sp = a.sp;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = L / sp.gsize, pos = L - grp * sp.gsize;
  const int gld = sp.bv * kTile;   // bf16 elements per slot row
  const bf16_t* X = static_cast<const bf16_t*>(a.x);
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  int seen = 0;   // items of the group's earlier blocks
  for (int j = grp; j < sp.count; j += sp.groups) {
    int mt0, vt0, nt, nv;
    step_block(sp, j, mt0, vt0, nt, nv);
    const int n = z_items(nt, nv);
    bf16_t* G = reinterpret_cast<bf16_t*>(a.slots + (int64_t)j * a.slot_bytes);
    int q = (pos - seen) % sp.gsize;
    if (q < 0) q += sp.gsize;
    for (; q < n; q += sp.gsize) {
      int mi, nj;
      grid_item(q, nt, nv, 4, mi, nj);
      const int m0 = (mt0 + mi) * kTile, n0 = (vt0 + nj) * kTile;   // first token, first vocabulary id
      f32x16 acc[kColBlocks][4];
      {
        Operand<bf16_t, true> C, R;   // columns: W rows (vocabulary), rows: x rows (tokens)
        C.init(W, a.H, n0, a.V, (uint32_t)((int64_t)a.V * a.H * 2));
        R.init(X, a.H, m0, a.rows, (uint32_t)((int64_t)a.rows * a.H * 2));
        gemm_tile_balanced<bf16_t>(acc, smem, C, R, 0, a.H, opaque_tid());
      }
      // G tile into LDS as 256 rows of 512 bytes, 16-byte chunk c of row r at c ^ (r % 32)
      const int tid = opaque_tid();
      const Frag f = frag_coords(tid);
      const int lane = tid & 63;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = f.row(jj);
        const int tok = m0 + row;
        const int64_t tv = tok < a.rows ? a.t[tok] : -1;
        const bool rok = tok < a.rows && !a.ign.skip(tv);   // an ignored token's row of G is zero
        const float l = rok ? a.lse[tok] : 0.f;
        const float gscale = a.scale->grad;
#pragma unroll
        for (int i = 0; i < kColBlocks; ++i)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int c0 = f.col0(i, qq);
            float gv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = n0 + c0 + e;
              float g = 0.f;
              if (rok && v < a.V) {
                g = fast_exp(acc[i][jj][4 * qq + e] - l);
                if (v == tv) g -= 1.f;
                g *= gscale;
              }
              gv[e] = g;
            }
            *reinterpret_cast<u32x2*>(smem + row * 512 + (((c0 >> 3) ^ (row & 31)) << 4) + 8 * (lane >> 5)) =
                u32x2{pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};
          }
      }
      phase_barrier<false, true>();   // the G tile visible in LDS
      // full 512-byte rows out to the slot: rows mi*256 + r, columns nj*256 ..
      constexpr int kPerWave = kTile * kTile * 2 / 1024 / kWaves;
      const int ln = opaque_tid() & 63;
#pragma unroll
      for (int k = 0; k < kPerWave; ++k) {
        const int b = wave * kPerWave + k;
        const int r = 2 * b + (ln >> 5);
        const int c = (ln & 31) ^ (r & 31);
        *reinterpret_cast<u32x4*>(G + (int64_t)(mi * kTile + r) * gld + nj * kTile + 8 * c) =
            *reinterpret_cast<const u32x4*>(smem + b * 1024 + 16 * ln);
      }
      phase_barrier<true, true>();    // stores complete, LDS free for the next product
    }
    seen += n;
  }
}

__global__ __launch_bounds__(kThreads, 1) void fused_p_kernel(FusedStepArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kDeepRingBytes];
  const StepPlan& sp = a.sp;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = L / sp.gsize, pos = L - grp * sp.gsize;
  const int gld = sp.bv * kTile;
  const uint32_t gbytes = (uint32_t)a.slot_bytes;
  const bf16_t* X = static_cast<const bf16_t*>(a.x);
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  int seen = 0;
  for (int j = grp; j < sp.count; j += sp.groups) {
    int mt0, vt0, nt, nv;
    step_block(sp, j, mt0, vt0, nt, nv);
    const int n = p_items(sp, nt, nv);
    const bf16_t* G = reinterpret_cast<const bf16_t*>(a.slots + (int64_t)j * a.slot_bytes);
    const int tok0 = mt0 * kTile, voc0 = vt0 * kTile;
    const int ntok = min(nt * kTile, a.rows - tok0), nvoc = min(nv * kTile, a.V - voc0);
    int q = (pos - seen) % sp.gsize;
    if (q < 0) q += sp.gsize;
    for (; q < n; q += sp.gsize) {
      f32x16 acc[kColBlocks][4];
      if (q < nt * sp.th) {   // dx rows tok0 + mi*256 .. = G rows x W, contraction over the block's ids
        int mi, hb;
        grid_item(q, nt, sp.th, 4, mi, hb);
        Operand<bf16_t, false> C;   // columns: W[voc0 + v][h0 + h]
        Operand<bf16_t, true> R;    // rows: G[mi*256 + token][v]
        C.init(W + (int64_t)voc0 * a.H, a.H, hb * kTile, a.H, (uint32_t)((int64_t)nvoc * a.H * 2));
        R.init(G, gld, mi * kTile, ntok, gbytes);
        gemm_tile_balanced<bf16_t, Operand<bf16_t, false>, Operand<bf16_t, true>, true>(acc, smem, C, R, 0, nvoc,
                                                                                  opaque_tid());
        atomic_add_tile(acc, make_rsrc(a.dx_acc, (uint32_t)((int64_t)a.rows * a.H * 4)), tok0 + mi * kTile, a.rows,
                        hb * kTile, a.H);
      } else {                // dW rows voc0 + nj*256 .. = G columns^T x, contraction over the block's tokens
        int nj, hb;
        grid_item(q - nt * sp.th, nv, sp.th, 4, nj, hb);
        Operand<bf16_t, false> C;   // columns: x[tok0 + token][h0 + h]
        Operand<bf16_t, false> R;   // rows: G[token][nj*256 + v]
        C.init(X + (int64_t)tok0 * a.H, a.H, hb * kTile, a.H, (uint32_t)((int64_t)ntok * a.H * 2));
        R.init(G, gld, nj * kTile, nvoc, gbytes);
        if (a.dw_owned) {   // the block holds every token of the launch: this is the tile's only product
          gemm_tile<bf16_t>(acc, smem, C, R, 0, ntok, opaque_tid());
          store_tile_bf16(acc, static_cast<bf16_t*>(a.dw_out), voc0 + nj * kTile, a.V, hb * kTile, a.H, a.dw_add != 0);
        } else {
          gemm_tile<bf16_t, Operand<bf16_t, false>, Operand<bf16_t, false>, true>(acc, smem, C, R, 0, ntok,
                                                                           opaque_tid());
          atomic_add_tile(acc, make_rsrc(a.dw_acc, (uint32_t)((int64_t)a.V * a.H * 4)), voc0 + nj * kTile, a.V,
                          hb * kTile, a.H);
        }
      }
    }
    seen += n;
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

hipError_t launch_fused_step(const FusedStepArgs& a, hipStream_t s) {
  const int grid = a.sp.groups * a.sp.gsize;
  hipLaunchKernelGGL(fused_z_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fused_p_kernel, dim3(grid), dim3(kThreads), 0, s, a);
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
