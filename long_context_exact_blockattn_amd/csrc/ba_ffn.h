// Blockwise feedforward: the SwiGLU feedforward of a block of query rows,
//   hidden = silu(x W1^T) * (x W3^T),   out = hidden W2^T,
// as two GEMM launches per block (Ring Attention summary, Summary: each host
// computes attention and the feedforward for its query block, block by block;
// the blockwise parallel transformer computes the feedforward per block so the
// hidden activation of the whole sequence never exists, Key points).
//
// gemm_nt_kernel: C = A B^T with A [M, K] and B [N, K] row-major (a linear
// layer's [out, in] weights), bf16 in, fp32 accumulation, bf16 out.  Work item
// = 256 output rows x 256 rows of B ("virtual" B rows); 8 waves, each 64 rows x
// 128 virtual B rows (2 x 4 accumulators of v_mfma_f32_32x32x16_bf16, computed
// transposed as in the attention kernels so that one lane holds one output
// row).  K advances 64 at a time through double-buffered LDS tiles filled by
// direct global->LDS loads into the swizzled layout of ba_common.h.
//   EPI_STORE  : B = W2; the 256 virtual rows are 256 output columns.
//   EPI_SWIGLU : the virtual rows of wave column wn are 64 rows of W1 followed
//                by the same 64 rows of W3, so every wave holds matching W1
//                and W3 accumulators and writes silu(A W1^T) * (A W3^T) for 64
//                output columns (128 per item).
#pragma once

#include "ba_common.h"
#include "ba_schedule.h"

namespace ba {

enum { EPI_STORE = 0, EPI_SWIGLU = 1 };

struct GemmArgs {
  const bf16* a;   // [M, K]
  const bf16* b;   // [N, K]: W2 (STORE) or W1 (SWIGLU)
  const bf16* b3;  // [N, K]: W3 (SWIGLU)
  bf16* c;         // [M, n_out]
  int64_t M;
  int32_t K, n_out;
  int32_t tiles_m, tiles_n;
  int64_t n_items;
};

constexpr int kGemmThreads = 512;
constexpr int kGemmBM = 256;
constexpr int kGemmBK = 64;
constexpr int kGemmGroupM = 4;

template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_nt_kernel(GemmArgs g) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = kGemmBM, BK = kGemmBK;
  constexpr int NW = kGemmThreads / 64;
  constexpr int TILE = BM * BK;            // elements of one A or B tile
  constexpr int CPR = BK / 8;              // 16-byte chunks per tile row
  constexpr int NPI = TILE / 8 / kGemmThreads;  // direct loads per thread per tile
  constexpr int STEP = 64 * NW / CPR;      // tile rows between a thread's loads
  static_assert(STEP == 64, "the loader assumes the swizzle repeats every STEP rows and 64-row groups");
  // separate arrays: each has its own alias scope (see the forward kernel)
  __shared__ __attribute__((aligned(16))) bf16 sA0[TILE], sA1[TILE], sB0[TILE], sB1[TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int hl = lane >> 5, l32 = lane & 31;

  // Item order: groups of kGemmGroupM row tiles, each group walking every
  // column tile; with the XCD remap the 32 items an XCD runs at once span 4 row
  // tiles x 8 column tiles, so their A and B slices are shared in that XCD's L2
  // (the kernel is bound by L2-miss traffic into LDS, not by the matrix cores).
  const int64_t item = xcd_remap(blockIdx.x, g.n_items);
  const int64_t per_group = (int64_t)kGemmGroupM * g.tiles_n;
  const int64_t first_m = (item / per_group) * kGemmGroupM;
  const int gsz = (int)((g.tiles_m - first_m) < kGemmGroupM ? (g.tiles_m - first_m) : kGemmGroupM);
  const int64_t within = item % per_group;
  const int tn = (int)(within / gsz);
  const int64_t m0 = (first_m + within % gsz) * BM;
  const int n0 = tn * (EPI == EPI_SWIGLU ? 128 : 256);  // first output column of the item

  // loader: thread slot ci = (p*NW + wave)*64 + lane holds tile row ci / CPR
  const int ld_row0 = (wave * 64 + lane) / CPR;
  const int ld_col = 8 * (((wave * 64 + lane) % CPR) ^ swz<BK>(ld_row0));
  // 32-bit element offsets from uniform bases (the host keeps every operand
  // under 2^31 elements)
  unsigned a_src[NPI], b_src[NPI];
#pragma unroll
  for (int p = 0; p < NPI; ++p) {
    const int r = ld_row0 + p * STEP;
    int64_t ar = m0 + r;
    ar = ar < g.M ? ar : g.M - 1;  // ragged last tile re-reads the last row; its stores are dropped
    a_src[p] = (unsigned)(ar * g.K + ld_col);
    if (EPI == EPI_SWIGLU) {
      // ld_row0 < 64 = STEP, so row r is in 64-row group p: W1 for even p, W3 for odd,
      // output columns n0 + 64 (p / 2) + ld_row0
      b_src[p] = (unsigned)((int64_t)(n0 + 64 * (p >> 1) + ld_row0) * g.K + ld_col);
    } else {
      b_src[p] = (unsigned)((int64_t)(n0 + r) * g.K + ld_col);
    }
  }
  // buffer loads: scalar bases, per-lane byte offsets fixed for the item and
  // the K position in the scalar offset (the host keeps every operand under
  // 2^31 elements, so byte offsets fit in 32 bits)
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, 0xFFFFFFFFu);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b, 0xFFFFFFFFu);
  const __amdgpu_buffer_rsrc_t rb3 = make_rsrc(EPI == EPI_SWIGLU ? g.b3 : g.b, 0xFFFFFFFFu);
  auto issue = [&](bf16* sa, bf16* sb, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NPI; ++p) {
      buf2lds16(ra, 2u * a_src[p], 2u * k0, sa + (p * NW + wave) * 512);
      buf2lds16((EPI == EPI_SWIGLU && (p & 1)) ? rb3 : rb, 2u * b_src[p], 2u * k0, sb + (p * NW + wave) * 512);
    }
  };

  // LDS offsets: the swizzle depends on the row mod 16 only, so row blocks
  // 32 apart differ by a constant; one register per k step
  int kx[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) kx[kk] = tile_off<BK>(l32, 16 * kk + 8 * hl);
  const int a_row0 = 64 * wm * BK, b_row0 = 128 * wn * BK;
  f32x16 acc[2][4];
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      acc[ib][jb] = f32x16{};
      // in accumulator registers from the start: with vector registers the
      // compiler gives the MFMAs results separate from their inputs and keeps
      // two copies of every accumulator
      asm volatile("" : "+a"(acc[ib][jb]));
    }

  // fragments of k step kk+1 are read while the MFMAs of kk run (two register
  // sets; the fences stop the compiler from reading further ahead)
  auto step = [&](const bf16* sa, const bf16* sb) __attribute__((always_inline)) {
    bf16x8 af[2][2], bfr[2][4];
    auto read = [&](int kk, int set) __attribute__((always_inline)) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) af[set][ib] = *(const bf16x8*)(sa + a_row0 + 32 * ib * BK + kx[kk]);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) bfr[set][jb] = *(const bf16x8*)(sb + b_row0 + 32 * jb * BK + kx[kk]);
    };
    read(0, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) read(kk + 1, (kk + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) acc[ib][jb] = mfma32(bfr[kk & 1][jb], af[kk & 1][ib], acc[ib][jb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = g.K / BK;
  issue(sA0, sB0, 0);
  wait_vmem();
  __syncthreads();
  for (int t = 0; t < nk; t += 2) {
    if (t + 1 < nk) issue(sA1, sB1, (t + 1) * BK);
    step(sA0, sB0);
    wait_vmem();
    __syncthreads();
    if (t + 1 >= nk) break;
    if (t + 2 < nk) issue(sA0, sB0, (t + 2) * BK);
    step(sA1, sB1);
    wait_vmem();
    __syncthreads();
  }

  // epilogue: lane l32 of accumulator block (ib, jb) is output row 64wm + 32ib + l32;
  // register r is virtual B row 32jb + 8(r/4) + 4hl + r%4 of the wave's 128
#pragma unroll
  for (int ib = 0; ib < 2; ++ib) {
    const int64_t row = m0 + 64 * wm + 32 * ib + l32;
    if (row >= g.M) continue;
    bf16* crow = g.c + row * g.n_out;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = acc[ib][jb][4 * q + e];
            const float s = z / (1.f + exp2_hw(-z * kLog2e));
            hv[e] = (bf16)(s * acc[ib][jb + 2][4 * q + e]);
          }
          *(bf16x4*)(crow + n0 + 64 * wn + 32 * jb + 8 * q + 4 * hl) = hv;
        }
    } else {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (bf16)acc[ib][jb][4 * q + e];
          *(bf16x4*)(crow + n0 + 128 * wn + 32 * jb + 8 * q + 4 * hl) = ov;
        }
    }
  }
#endif
}

}  // namespace ba
