// Standalone merge of partial (O, LSE) pairs, elementwise over query rows.
//
// Combination rule (the order-independent blockwise combination of the Ring
// Attention summary, Summary): with La, Lb the log-sum-exps of two disjoint key
// sets, L = log(e^La + e^Lb) and O = e^(La-L) O_a + e^(Lb-L) O_b; a pair with
// L = -inf contributes nothing (its O is never read), two such pairs give
// (0, -inf).  HBM-bound: one thread handles 8 consecutive elements of a row.
#pragma once

#include "ba_common.h"

namespace ba {

struct MergeArgs {
  float* o_acc;
  float* lse_acc;
  const void* o_part;
  const float* lse_part;
  bf16* o_final;
  int64_t s_b, s_s, s_h;
  int64_t Sq;
  int32_t Hq, D, part_f32;
  int64_t n_threads;
};

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= a.n_threads) return;
  const int cpr = a.D / 8;
  const int64_t rowid = g / cpr;
  const int c = (int)(g % cpr);
  const int h = (int)(rowid % a.Hq);
  const int64_t s = (rowid / a.Hq) % a.Sq;
  const int64_t b = rowid / ((int64_t)a.Hq * a.Sq);
  const int64_t li = (b * a.Hq + h) * a.Sq + s;
  const int64_t off = b * a.s_b + s * a.s_s + h * a.s_h + 8 * c;

  const float la2 = a.lse_acc[li] * kLog2e;
  const float lb2 = a.lse_part[li] * kLog2e;
  const float M = fmaxf(la2, lb2);
  float wa = 0.f, wb = 0.f, L2 = -INFINITY;
  if (M != -INFINITY) {
    const float ea = exp2_hw(la2 - M);
    const float eb = exp2_hw(lb2 - M);
    const float tot = ea + eb;
    L2 = M + log2_hw(tot);
    wa = ea / tot;
    wb = eb / tot;
  }
  float out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = 0.f;
  if (wa > 0.f) {
    const f32x4 x0 = *(const f32x4*)(a.o_acc + off);
    const f32x4 x1 = *(const f32x4*)(a.o_acc + off + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { out[e] = wa * x0[e]; out[4 + e] = wa * x1[e]; }
  }
  if (wb > 0.f) {
    float y[8];
    if (a.part_f32) {
      const f32x4 y0 = *(const f32x4*)((const float*)a.o_part + off);
      const f32x4 y1 = *(const f32x4*)((const float*)a.o_part + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { y[e] = y0[e]; y[4 + e] = y1[e]; }
    } else {
      const bf16x8 yb = *(const bf16x8*)((const bf16*)a.o_part + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (float)yb[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = __builtin_fmaf(wb, y[e], out[e]);
  }
  *(f32x4*)(a.o_acc + off) = f32x4{out[0], out[1], out[2], out[3]};
  *(f32x4*)(a.o_acc + off + 4) = f32x4{out[4], out[5], out[6], out[7]};
  // All D/8 threads of a row sit in one wavefront (D/8 divides 64), so every
  // one of them has read lse_acc[li] before this store executes.
  if (c == 0) a.lse_acc[li] = L2 * kLn2;
  if (a.o_final) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)out[e];
    *(bf16x8*)(a.o_final + off) = r;
  }
#endif
}

// Final bf16 store of rows a ring step does not reach: o_final = bf16(o_acc)
// (round to nearest even) for rows [0, rows) of every (batch, head); the
// running pair itself is left as it is.  HBM-bound like the merge: one thread
// converts 8 consecutive elements, consecutive threads consecutive memory.
struct StoreArgs {
  const float* o_acc;
  bf16* o_final;
  int64_t s_b, s_s, s_h;
  int64_t rows;
  int32_t Hq, D;
  int64_t n_threads;
};

__global__ __launch_bounds__(256) void store_final_kernel(StoreArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= a.n_threads) return;
  const int cpr = a.D / 8;
  const int64_t rowid = g / cpr;
  const int c = (int)(g % cpr);
  const int h = (int)(rowid % a.Hq);
  const int64_t s = (rowid / a.Hq) % a.rows;
  const int64_t b = rowid / ((int64_t)a.Hq * a.rows);
  const int64_t off = b * a.s_b + s * a.s_s + h * a.s_h + 8 * c;
  const f32x4 x0 = *(const f32x4*)(a.o_acc + off);
  const f32x4 x1 = *(const f32x4*)(a.o_acc + off + 4);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) { r[e] = (bf16)x0[e]; r[4 + e] = (bf16)x1[e]; }
  *(bf16x8*)(a.o_final + off) = r;
#endif
}

}  // namespace ba
