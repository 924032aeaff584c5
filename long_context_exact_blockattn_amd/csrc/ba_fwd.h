// Forward kernel: one ring step of exact blockwise attention (or S2-Attn).
//
// Work item = (batch, query head, tile of BM = 128 query rows); 4 waves, each
// owning 32 query rows.  Key/value tiles of BN = 64 rows stream through a
// double-buffered LDS ring filled by direct global->LDS loads (no staging
// registers); the tile loop is unrolled by two so both buffers sit at fixed
// LDS addresses.  Scores and outputs use v_mfma_f32_32x32x16_bf16 in the
// TRANSPOSED form, S^T = K Q^T and O^T += V^T P^T, so that one lane holds the
// scores of ONE query row: the row max and row sum of the online softmax are
// in-lane reductions plus a single exchange between the two lane halves.
//
// Online softmax (Milakov & Gimelshein's online normaliser, cited by the Ring
// Attention summary's references): running max m and sum l per row, in base 2
// with tau*log2(e) folded into one FMA; m is only raised when a tile's (base-2)
// max exceeds it by more than 8, so the O rescale is rare; a fully masked row
// keeps m = -inf and l = 0 without producing NaN.  The epilogue turns (acc, m,
// l) into the chunk's partial pair and, in ACCUMULATE mode, merges it into the
// running pair (O_acc, LSE_acc) in fp32 -- the order-independent combination of
// the Ring Attention summary (Summary).
#pragma once

#include "ba_common.h"
#include "ba_schedule.h"

namespace ba {

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  void* o;          // fp32 or bf16 [B,Sq,Hq,D]
  float* lse;       // [B,Hq,Sq]
  bf16* o_final;    // nullable bf16 [B,Sq,Hq,D]
  int64_t qs_b, qs_s, qs_h;  // element strides of query-shaped tensors
  int64_t ks_b, ks_s, ks_h;  // element strides of key-shaped tensors
  int64_t Sq, Sk, q_pos0, k_pos0;
  int32_t B, Hq, Hkv, grp;
  int32_t causal, accumulate, o_f32;
  int32_t s2_group, s2_shift_head0;
  float scale_log2;  // tau * log2(e)
  int64_t n_qtiles;  // query tiles per (batch, head)
  int64_t n_ranks;   // of which launched: the n_ranks longest (the rest have no allowed key)
  int64_t n_items;
};

// One 32-row query block per wave, two waves per SIMD.  The loops below are
// written over kFwdQB blocks per wave: with two, every K or V fragment read
// from LDS would feed two MFMAs (half the LDS bytes per MFMA), but the ~380
// live registers that takes leave one wave per SIMD, which measures about half
// as fast.
constexpr int kFwdQB = 1;
constexpr int kFwdThreads = 256;
constexpr int kFwdBM = (kFwdThreads / 64) * 32 * kFwdQB;
constexpr int kFwdBN = 64;

template <int D>
__global__ __launch_bounds__(kFwdThreads, 2 / kFwdQB) void fwd_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = kFwdBM, BN = kFwdBN, QB = kFwdQB;
  constexpr int NW = kFwdThreads / 64;       // waves
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int NPI = BN * CPR / (64 * NW);  // direct-load instructions per wave per tensor
  constexpr int KK = D / 16;                 // MFMA k-steps over D
  constexpr int DB = D / 32;                 // 32-wide blocks of D in the output
  constexpr int TILE = BN * D;               // elements per tile
  // K0, V0, K1, V1 tiles (swizzled), as separate arrays: the compiler then sees
  // that a direct load into one buffer cannot alias LDS reads of another and
  // does not wait for the prefetch before reading the current tile.
  __shared__ __attribute__((aligned(16))) bf16 sK0[TILE], sV0[TILE], sK1[TILE], sV1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;   // lane half
  const int l32 = lane & 31;

  // ---- work item
  const int64_t pid = xcd_remap(blockIdx.x, a.n_items);
  const int64_t bh = pid / a.n_ranks;
  const int64_t w = pid % a.n_ranks;
  const int b = (int)(bh / a.Hq);
  const int h = (int)(bh % a.Hq);
  const int kvh = h / a.grp;
  Sched sc;
  sc.Sq = a.Sq; sc.Sk = a.Sk; sc.q_pos0 = a.q_pos0; sc.k_pos0 = a.k_pos0;
  sc.causal = a.causal; sc.s2_group = a.s2_group;
  sc.s2_shift = (a.s2_group > 0 && h >= a.s2_shift_head0) ? a.s2_group / 2 : 0;
  sc.BM = BM; sc.BN = BN;
  const QTile qt = make_qtile(sc, qtile_of_rank(sc, a.n_qtiles, w));
  const bool empty = qt.kt_end <= qt.kt_begin;
  if (empty && a.accumulate && a.o_final == nullptr) return;

  // rows of this lane: block qb holds tile row wave*32*QB + qb*32 + l32
  int rloc[QB];
  bool row_ok[QB];
  float m_run[QB], l_run[QB];
  f32x16 oacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    rloc[qb] = wave * 32 * QB + qb * 32 + l32;
    row_ok[qb] = rloc[qb] < qt.rows;
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[qb][i] = f32x16{};
  }
  const int64_t wave_cmin = qt.cpos0 + wave * 32 * QB;  // coordinate of the wave's first row
  const int64_t wave_cmax = wave_cmin + 32 * QB - 1;

  if (!empty) {
    // ---- resident query fragments: B operand of S^T = K Q^T
    bf16x8 qf[QB][KK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const bf16* qp = a.q + (int64_t)b * a.qs_b + (qt.row0 + rloc[qb]) * a.qs_s + (int64_t)h * a.qs_h + 8 * hl;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qf[qb][kk] = row_ok[qb] ? *(const bf16x8*)(qp + 16 * kk) : bf16x8{};
    }

    // ---- per-lane offsets, computed once
    // K fragment (row l32 of a 32-key block, chunk 2kk+hl); the second block adds 32*D
    int k_off[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) k_off[kk] = tile_off<D>(l32, 16 * kk + 8 * hl);
    // V^T fragment, read transposed: rows k0 (+16kc) and k0 + 8 (+16kc), columns dcol
    const int gi = lane & 15;
    const int k0 = 4 * hl + (gi >> 2);
    int v_off[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dcol = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
      v_off[db][0] = tile_off<D>(k0, dcol);
      v_off[db][1] = tile_off<D>(k0 + 8, dcol);
    }
    // direct loads: lane fills slot ci of the tile with row r, chunk c of the source
    int g_row[NPI], g_col[NPI];
#pragma unroll
    for (int p = 0; p < NPI; ++p) {
      const int ci = (p * NW + wave) * 64 + lane;
      g_row[p] = ci / CPR;
      g_col[p] = 8 * ((ci % CPR) ^ swz<D>(ci / CPR));
    }
    const bf16* kbase = a.k + (int64_t)b * a.ks_b + (int64_t)kvh * a.ks_h;
    const bf16* vbase = a.v + (int64_t)b * a.ks_b + (int64_t)kvh * a.ks_h;
    const int ks_s = (int)a.ks_s;
    unsigned g_off[NPI];  // byte offset of this lane's chunk inside a full tile
#pragma unroll
    for (int p = 0; p < NPI; ++p) g_off[p] = 2u * (unsigned)(g_row[p] * ks_s + g_col[p]);

    auto issue_tile = [&](bf16* kdst, bf16* vdst, int64_t kt) {
      const KTile t = make_ktile(sc, kt);
      const bf16* kt_base = kbase + t.row0 * a.ks_s;
      const bf16* vt_base = vbase + t.row0 * a.ks_s;
      const int last = (int)t.rows - 1;
      if (last == BN - 1) {  // full tile: scalar base + the fixed per-lane offsets
        // the resource spans exactly the tile's rows: (BN - 1) strides plus one row
        const unsigned bytes = 2u * (unsigned)((BN - 1) * ks_s + D);
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(kt_base, bytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vt_base, bytes);
#pragma unroll
        for (int p = 0; p < NPI; ++p) {
          buf2lds16(krs, g_off[p], 0u, kdst + (p * NW + wave) * 512);
          buf2lds16(vrs, g_off[p], 0u, vdst + (p * NW + wave) * 512);
        }
        return;
      }
#pragma unroll
      for (int p = 0; p < NPI; ++p) {
        const int r = g_row[p] < last ? g_row[p] : last;  // ragged tail re-reads the last row
        const unsigned off = (unsigned)(r * ks_s + g_col[p]);
        g2lds16(kt_base + off, kdst + (p * NW + wave) * 512);
        g2lds16(vt_base + off, vdst + (p * NW + wave) * 512);
      }
    };

    // one key tile from a fixed buffer
    auto tile_step = [&](const bf16* Ks, const bf16* Vs, int64_t kt) {
      const KTile t = make_ktile(sc, kt);
      if (a.causal && t.cpos0 > wave_cmax) return;  // every key after every row of this wave
      // ---- S^T = K Q^T  (two 32-key blocks; each K fragment feeds QB MFMAs)
      f32x16 s[QB][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 kf = *(const bf16x8*)(Ks + kb * 32 * D + k_off[kk]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][kb] = mfma32(kf, qf[qb][kk], kk == 0 ? f32x16{} : s[qb][kb]);
        }
      }
      // ---- mask: keys past the chunk's end or (causal) after this lane's row
      const bool need_mask = (t.rows < BN) || (a.causal && t.cpos0 + BN - 1 > wave_cmin);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          // last allowed key index of this lane's row in block qb, in 32 bits
          int lim = (int)t.rows - 1;
          if (a.causal) {
            int64_t c = wave_cmin + 32 * qb - t.cpos0;  // >= -32*QB for an active wave
            c = c > BN ? BN : c;
            const int cl = (int)c + l32;
            lim = cl < lim ? cl : lim;
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
              s[qb][kb][r] = key <= lim ? s[qb][kb][r] : -INFINITY;
            }
        }
      }
      // ---- online softmax (base 2), per query block
      bf16x8 pf[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        mx = halves_max(mx);
        // The running max moves only when a tile's max exceeds it by more than 8
        // (base 2): p = 2^(s - m) then stays <= 256, far inside the fp32 and bf16
        // ranges, and the O rescale below is skipped on almost every tile.
        const float mx2 = mx * a.scale_log2;
        const float m_new = (mx2 > m_run[qb] + 8.f) ? mx2 : m_run[qb];
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float m_old = m_run[qb];
        float rsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_hw(__builtin_fmaf(s[qb][kb][r], a.scale_log2, -m_use));
            rsum += p;
            pf[qb][kb * 2 + (r >> 3)][r & 7] = (bf16)p;
          }
        // alpha = 2^(m_old - m_use) differs from 1 only where the running max moved
        // (or where it was -inf, with O and l still 0): the rescale is decided on
        // the max alone and the exponential stays off the common path
        if (__any(m_new != m_old)) {
          const float al = exp2_hw(m_old - m_use);
          l_run[qb] = l_run[qb] * al + rsum;
#pragma unroll
          for (int i = 0; i < DB; ++i) oacc[qb][i] *= al;
        } else {
          l_run[qb] = l_run[qb] + rsum;
        }
        m_run[qb] = m_new;
      }
      // ---- O^T += V^T P^T ; V^T operand read transposed from the [key][d] tile,
      // each fragment feeding QB MFMAs
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16x4 v0 = lds_read_tr16(Vs + 16 * kc * D + v_off[db][0]);
          const bf16x4 v1 = lds_read_tr16(Vs + 16 * kc * D + v_off[db][1]);
          const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma32(vf, pf[qb][kc], oacc[qb][db]);
        }
      }
    };

    bf16* const K0 = sK0;
    bf16* const V0 = sV0;
    bf16* const K1 = sK1;
    bf16* const V1 = sV1;
    issue_tile(K0, V0, qt.kt_begin);
    wait_vmem();
    __syncthreads();
    for (int64_t kt = qt.kt_begin; kt < qt.kt_end; kt += 2) {
      if (kt + 1 < qt.kt_end) issue_tile(K1, V1, kt + 1);
      tile_step(K0, V0, kt);
      wait_vmem();
      __syncthreads();
      if (kt + 1 >= qt.kt_end) break;
      if (kt + 2 < qt.kt_end) issue_tile(K0, V0, kt + 2);
      tile_step(K1, V1, kt + 1);
      wait_vmem();
      __syncthreads();
    }
  }

  // ---- epilogue, per query block: partial pair of this chunk, optional merge
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = halves_sum(l_run[qb]);
    const bool has = l_tot > 0.f;
    const float lse2_c = has ? m_run[qb] + log2_hw(l_tot) : -INFINITY;
    const float inv_l = has ? 1.f / l_tot : 0.f;
    if (!row_ok[qb]) continue;
    const int64_t row = qt.row0 + rloc[qb];
    const int64_t lse_idx = ((int64_t)b * a.Hq + h) * a.Sq + row;
    const int64_t obase = (int64_t)b * a.qs_b + row * a.qs_s + (int64_t)h * a.qs_h + 4 * hl;
    float ca = 0.f, cc = inv_l, L2 = lse2_c;
    if (a.accumulate) {
      const float la2 = a.lse[lse_idx] * kLog2e;
      const float M = fmaxf(la2, lse2_c);
      if (M == -INFINITY) {
        ca = 0.f; cc = 0.f; L2 = -INFINITY;
      } else {
        const float wa = exp2_hw(la2 - M);
        const float wc = exp2_hw(lse2_c - M);
        const float tot = wa + wc;
        L2 = M + log2_hw(tot);
        ca = wa / tot;
        cc = wc / tot * inv_l;
      }
    }
    const bool write_state = !(a.accumulate && empty);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t off = obase + 32 * db + 8 * g;
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = cc * oacc[qb][db][4 * g + e];
        if (a.accumulate && ca > 0.f) {
          const f32x4 prev = *(const f32x4*)((const float*)a.o + off);
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = __builtin_fmaf(ca, prev[e], val[e]);
        }
        if (write_state) {
          if (a.o_f32) {
            *(f32x4*)((float*)a.o + off) = val;
          } else {
            bf16x4 bv;
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[e] = (bf16)val[e];
            *(bf16x4*)((bf16*)a.o + off) = bv;
          }
        }
        if (a.o_final) {
          bf16x4 bv;
#pragma unroll
          for (int e = 0; e < 4; ++e) bv[e] = (bf16)val[e];
          *(bf16x4*)(a.o_final + off) = bv;
        }
      }
    }
    if (write_state && hl == 0) a.lse[lse_idx] = L2 * kLn2;
  }
#endif
}

}  // namespace ba
