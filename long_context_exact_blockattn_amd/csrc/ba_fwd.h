// Forward kernel: one ring step of exact blockwise attention (or S2-Attn).
//
// Work item = (batch, query head, tile of BM = 256 query rows); 8 waves, each
// owning 32 query rows, one workgroup per CU.  Key/value tiles of BN = 64 rows
// stream through LDS filled by direct global->LDS loads (no staging
// registers).  Scores and outputs use v_mfma_f32_32x32x16_bf16 in the
// TRANSPOSED form, S^T = K Q^T and O^T += V^T P^T, so that one lane holds the
// scores of ONE query row: the row max and row sum of the online softmax are
// in-lane reductions plus a single exchange between the two lane halves.
//
// Two wave groups share every SIMD: group A (waves 0-3) and group B (waves
// 4-7) run the same three steps per key tile -- the score MFMAs, the softmax
// (vector ALU only), the P V MFMAs -- but skewed by half a tile between the
// workgroup's barriers.  Between two barriers (interval j) group A runs P V of
// tile j-1 and the scores of tile j (matrix cores), then the softmax of tile j
// (vector ALU); group B runs the softmax of tile j-1, then P V of tile j-1 and
// the scores of tile j.  So on every SIMD one wave's softmax runs beside the
// other wave's MFMAs, which the hardware executes concurrently; each softmax
// is kept free of MFMAs, because the waves issue in order and an MFMA waiting
// for the busy matrix core would hold the rest of the softmax back.  Group A
// carries P across a barrier, group B the scores.  Key tiles sit in two
// K buffers (tile j in K[j mod 2]) and four V buffers (V[j mod 4]): the loads
// of tile j+1 are issued at the start of interval j, when V[(j+1) mod 4] (tile
// j-3) and K[(j+1) mod 2] (tile j-1) have been read by both groups.
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

#include <type_traits>

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
  int64_t qs_b, qs_s, qs_h;  // element strides of q
  int64_t ks_b, ks_s, ks_h;  // element strides of k and v
  int64_t os_b, os_s, os_h;  // element strides of o and o_final
  int64_t Sq, Sk, q_pos0, k_pos0;
  int32_t B, Hq, Hkv, grp;
  int32_t causal, accumulate, o_f32;
  int32_t s2_group, s2_shift_head0;
  float scale_log2;  // tau * log2(e)
  int64_t n_qtiles;  // query tiles per (batch, head)
  int64_t n_ranks;   // of which launched: the n_ranks longest (the rest have no allowed key)
  int64_t n_items;
  int64_t hx;        // heads interleaved per XCD (qitem_of_pid), 0 for head-major order
};

constexpr int kFwdWaves = 8;
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr int kFwdBM = 32 * kFwdWaves;
constexpr int kFwdBN = 64;
constexpr int kFwdSlotsPerXcd = 32;  // one workgroup per CU, 32 CUs per XCD

template <int D>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = kFwdBM, BN = kFwdBN;
  constexpr int NW = kFwdWaves;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int NPI = BN * CPR / (64 * NW);  // direct-load instructions per wave per tensor
  constexpr int KK = D / 16;                 // MFMA k-steps over D
  constexpr int DB = D / 32;                 // 32-wide blocks of D in the output
  constexpr int TILE = BN * D;               // elements per tile
  static_assert(NPI >= 1, "every wave loads part of a tile");
  // K0, K1, V0..V3 tiles (swizzled), as separate arrays: the compiler then sees that a
  // direct load into one buffer cannot alias LDS reads of another and does not wait for
  // the prefetch before reading the current tile.  E0, E1 only widen the epilogue's stage
  // (one array per wave).
  __shared__ __attribute__((aligned(16))) bf16 sK0[TILE], sK1[TILE], sV0[TILE], sV1[TILE], sV2[TILE],
      sV3[TILE], sE0[TILE], sE1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grp_b = wave >= NW / 2;  // waves w and w + 4 share a SIMD
  const int hl = lane >> 5;           // lane half
  const int l32 = lane & 31;

  // ---- work item
  int64_t bh, w;
  qitem_of_pid(xcd_remap(blockIdx.x, a.n_items), a.n_ranks, a.hx, bh, w);
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

  // this lane's row: tile row wave*32 + l32
  const int rloc = wave * 32 + l32;
  const bool row_ok = rloc < qt.rows;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  const int64_t wave_cmin = qt.cpos0 + wave * 32;  // coordinate of the wave's first row
  const int64_t wave_cmax = wave_cmin + 31;

  if (!empty) {
    // ---- resident query fragments: B operand of S^T = K Q^T
    bf16x8 qf[KK];
    {
      const bf16* qp = a.q + (int64_t)b * a.qs_b + (qt.row0 + rloc) * a.qs_s + (int64_t)h * a.qs_h + 8 * hl;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[kk] = row_ok ? *(const bf16x8*)(qp + 16 * kk) : bf16x8{};
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
    const bf16* kbase = a.k + (int64_t)b * a.ks_b + (int64_t)kvh * a.ks_h;
    const bf16* vbase = a.v + (int64_t)b * a.ks_b + (int64_t)kvh * a.ks_h;
    const int ks_s = (int)a.ks_s;
    unsigned g_off[NPI];  // byte offset of this lane's chunk inside a full tile
#pragma unroll
    for (int p = 0; p < NPI; ++p) {
      const int ci = (p * NW + wave) * 64 + lane;
      g_off[p] = 2u * (unsigned)((ci / CPR) * ks_s + 8 * ((ci % CPR) ^ swz<D>(ci / CPR)));
    }

    auto issue_tile = [&](bf16* kdst, bf16* vdst, int64_t kt) {
      const KTile t = make_ktile(sc, kt);
      const bf16* kt_base = kbase + t.row0 * a.ks_s;
      const bf16* vt_base = vbase + t.row0 * a.ks_s;
      // the resource spans exactly the tile's valid rows ((rows - 1) strides plus one row):
      // lanes of a ragged tile's missing rows read past its end and get zeros (masked later)
      const unsigned bytes = 2u * (unsigned)(((int)t.rows - 1) * ks_s + D);
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(kt_base, bytes);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vt_base, bytes);
#pragma unroll
      for (int p = 0; p < NPI; ++p) buf2lds16(krs, g_off[p], 0u, kdst + (p * NW + wave) * 512);
#pragma unroll
      for (int p = 0; p < NPI; ++p) buf2lds16(vrs, g_off[p], 0u, vdst + (p * NW + wave) * 512);
    };

    // Per-wave tile thresholds, once per item: the key coordinate of tile kt is c0 + kt*BN
    // (make_ktile), so from act_end on no key of a tile is allowed for any row of this wave
    // (causal) and from mask_from on a tile needs the mask (causal diagonal, or the chunk's
    // ragged last tile).  Per interval the tests are then two scalar compares, in 32 bits
    // relative to the item's first tile (64-bit signed compares go to the vector ALU).
    constexpr int LBN = __builtin_ctz(BN);
    static_assert((1 << LBN) == BN, "floor division by BN as a shift");
    const int64_t c0 = a.s2_group > 0 ? 0 : a.k_pos0;
    const int64_t act_end = a.causal ? ((wave_cmax - c0) >> LBN) + 1 : INT64_MAX;
    int64_t mask_from = a.causal ? ((wave_cmin - c0 + 1) >> LBN) : INT64_MAX;
    if (a.s2_group == 0 && a.Sk % BN != 0) {
      const int64_t last = ceil_div(a.Sk, BN) - 1;
      mask_from = last < mask_from ? last : mask_from;
    }
    // Intervals j = 0 .. T (T = the item's key tiles); tile j is tile kt_begin + j
    const int64_t kt0 = qt.kt_begin;
    const int T = (int)(qt.kt_end - qt.kt_begin);
    auto rel = [&](int64_t kt) __attribute__((always_inline)) {
      const int64_t r = kt - kt0;
      return (int)(r < 0 ? 0 : (r > T + 1 ? T + 1 : r));
    };
    const int act_rel = rel(act_end), mask_rel = rel(mask_from);
    // whether this wave has any allowed key in tile j (causal: not every key after every row)
    auto active = [&](int j) __attribute__((always_inline)) { return j < act_rel; };

    f32x16 s[2];   // S^T of the wave's 32 rows x the tile's two 32-key blocks
    bf16x8 pf[4];  // P in bf16, B operand of the P V MFMAs (k-step kc = keys 16kc..16kc+15)

    // ---- S^T = K Q^T: the two 32-key blocks' fragments of k-step kk + 2 are read while
    // the MFMAs of k-step kk run (three fragment sets live)
    auto scores = [&](const bf16* Ks) __attribute__((always_inline)) {
      bf16x8 kf[3][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        kf[j][0] = *(const bf16x8*)(Ks + k_off[j]);
        kf[j][1] = *(const bf16x8*)(Ks + 32 * D + k_off[j]);
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 2 < KK) {
          kf[(kk + 2) % 3][0] = *(const bf16x8*)(Ks + k_off[kk + 2]);
          kf[(kk + 2) % 3][1] = *(const bf16x8*)(Ks + 32 * D + k_off[kk + 2]);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(kf[kk % 3][kb], qf[kk], kk == 0 ? f32x16{} : s[kb]);
      }
      // keep that order: 4 reads, then per k-step 2 reads (k-step + 2) before 2 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 2 < KK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    };

    // ---- mask of tile j: keys past the chunk's end or (causal) after this lane's row
    auto mask = [&](int j) __attribute__((always_inline)) {
      if (j >= mask_rel) {
        const KTile t = make_ktile(sc, kt0 + j);
        // last allowed key index of this lane's row, in 32 bits
        int lim = (int)t.rows - 1;
        if (a.causal) {
          int64_t c = wave_cmin - t.cpos0;  // >= -32 for an active wave
          c = c > BN ? BN : c;
          const int cl = (int)c + l32;
          lim = cl < lim ? cl : lim;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            s[kb][r] = key <= lim ? s[kb][r] : -INFINITY;
          }
      }
    };

    // ---- online softmax (base 2): scores -> P, running max / sum, rare O rescale.  With
    // DEFER (group A, whose P V of this tile comes after the next barrier) the rescale of O is
    // left to the start of that P V phase, right before the MFMAs that accumulate into O: at
    // the end of the softmax, the compiler merged the rescaled and the untouched accumulator
    // by copying all 64 of its registers out and back on every tile.
    float al_pend = 1.f;  // pending O factor (DEFER), per lane; 1 where the max did not move
    bool resc_pend = false;  // whether any lane of the wave has a pending factor (uniform)
    auto softmax = [&](auto defer) __attribute__((always_inline)) {
      constexpr bool DEFER = decltype(defer)::value;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = halves_max(mx);
      // The running max moves only when a tile's max exceeds it by more than 8
      // (base 2): p = 2^(s - m) then stays <= 256, far inside the fp32 and bf16
      // ranges, and the O rescale below is skipped on almost every tile.
      const float mx2 = mx * a.scale_log2;
      const float m_new = (mx2 > m_run + 8.f) ? mx2 : m_run;
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float m_old = m_run;
      float rsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_hw(__builtin_fmaf(s[kb][r], a.scale_log2, -m_use));
          rsum += p;
          pf[kb * 2 + (r >> 3)][r & 7] = (bf16)p;
        }
      // alpha = 2^(m_old - m_use) differs from 1 only where the running max moved
      // (or where it was -inf, with O and l still 0): the rescale is decided on
      // the max alone and the exponential stays off the common path
      if (__any(m_new != m_old)) {
        const float al = exp2_hw(m_old - m_use);
        l_run = l_run * al + rsum;
        if (DEFER) {
          al_pend = al;
          resc_pend = true;
        } else {
#pragma unroll
          for (int i = 0; i < DB; ++i) oacc[i] *= al;
        }
      } else {
        l_run = l_run + rsum;
      }
      m_run = m_new;
    };

    // ---- O^T += V^T P^T ; V^T operand read transposed from the [key][d] tile
    auto pv = [&](const bf16* Vs) __attribute__((always_inline)) {
      if (resc_pend) {
#pragma unroll
        for (int i = 0; i < DB; ++i) oacc[i] *= al_pend;
        resc_pend = false;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16x4 v0 = lds_read_tr16(Vs + 16 * kc * D + v_off[db][0]);
          const bf16x4 v1 = lds_read_tr16(Vs + 16 * kc * D + v_off[db][1]);
          const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = mfma32(vf, pf[kc], oacc[db]);
        }
      }
    };

    // Each group runs its own copy of the loop, so what one group keeps across a barrier (P
    // for A, the scores for B) is not live in the other's.  Both copies pass the same barriers.
    auto run = [&](auto group_b) __attribute__((always_inline)) {
      constexpr bool GB = decltype(group_b)::value;
      auto interval = [&](int j, const bf16* Kc, const bf16* Vp, bf16* Kn, bf16* Vn) __attribute__((always_inline)) {
        if (j + 1 < T) issue_tile(Kn, Vn, kt0 + j + 1);
        const bool prev = j >= 1 && active(j - 1);
        const bool cur = j < T && active(j);
        if (!GB) {
          if (prev) pv(Vp);
          if (cur) {
            scores(Kc);
            __builtin_amdgcn_sched_barrier(0);
            mask(j);
            softmax(std::true_type{});
          }
        } else {
          if (prev) {
            mask(j - 1);
            softmax(std::false_type{});
            // the softmax stays pure vector work: an MFMA issued among it would stall the
            // rest of it while the other group's MFMAs hold the matrix core
            __builtin_amdgcn_sched_barrier(0);
            pv(Vp);
          }
          if (cur) scores(Kc);
        }
        wait_vmem();
        __syncthreads();
      };
      // K slot j mod 2, V slot j mod 4: unrolled by four so every buffer is a fixed address
      for (int j = 0;; j += 4) {
        interval(j, sK0, sV3, sK1, sV1);
        if (j + 1 > T) break;
        interval(j + 1, sK1, sV0, sK0, sV2);
        if (j + 2 > T) break;
        interval(j + 2, sK0, sV1, sK1, sV3);
        if (j + 3 > T) break;
        interval(j + 3, sK1, sV2, sK0, sV0);
        if (j + 4 > T) break;
      }
    };
    issue_tile(sK0, sV0, kt0);
    wait_vmem();
    __syncthreads();
    if (grp_b)
      run(std::true_type{});
    else
      run(std::false_type{});
  }

  // ---- epilogue: the chunk's partial pair (acc / l, m + log2 l), merged in ACCUMULATE
  // mode into the running pair.  Rows pass through LDS so that global memory is read and
  // written in whole lines (in the MFMA layout one 16-byte access per lane touches 32
  // rows): after the loop's last barrier every buffer is free, and wave w stages its 32
  // rows x D fp32 in array w (32*4D bytes = one tile of BN x D bf16).  In the stage, row
  // r's 16-byte piece c sits at slot c ^ (r mod D/4) of the row, so the MFMA-layout
  // accesses (32 rows, one piece each) spread over the banks; the direct loads and the
  // copy-out walk the stage linearly, 1 KB (whole rows) per instruction.
  constexpr int SPR = D / 4;               // 16-byte pieces per staged row
  constexpr int NIO = 32 * SPR / 64;       // linear 1 KB steps per wave
  const float l_tot = halves_sum(l_run);
  const bool has = l_tot > 0.f;
  const float lse2_c = has ? m_run + log2_hw(l_tot) : -INFINITY;
  const float inv_l = has ? 1.f / l_tot : 0.f;
  const int64_t wrows = qt.rows - (int64_t)wave * 32;
  if (wrows <= 0) return;
  const int vr = wrows < 32 ? (int)wrows : 32;  // rows of this wave inside the tile
  float* const stage = (float*)(wave == 0   ? sK0
                                : wave == 1 ? sK1
                                : wave == 2 ? sV0
                                : wave == 3 ? sV1
                                : wave == 4 ? sV2
                                : wave == 5 ? sV3
                                : wave == 6 ? sE0
                                            : sE1);
  const int64_t gbase = (int64_t)b * a.os_b + (qt.row0 + (int64_t)wave * 32) * a.os_s + (int64_t)h * a.os_h;
  const int64_t lse_idx = ((int64_t)b * a.Hq + h) * a.Sq + qt.row0 + rloc;
  const bool write_state = !(a.accumulate && empty);
  float ca = 0.f, cc = inv_l, L2 = lse2_c;
  if (a.accumulate) {
    // the running output's rows, straight into the stage (rows past the tile read zeros)
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc((const float*)a.o + gbase, 4u * (unsigned)((vr - 1) * (int)a.os_s + D));
#pragma unroll
    for (int i = 0; i < NIO; ++i) {
      const int u = i * 64 + lane, r = u / SPR, c = (u % SPR) ^ (r & (SPR - 1));
      buf2lds16(rs, 4u * (unsigned)(r * (int)a.os_s + 4 * c), 0u, stage + 256 * i);
    }
    const float la = row_ok ? a.lse[lse_idx] : -INFINITY;
    wait_vmem();
    // a row whose running LSE is -inf gets weight 0 and its stale values are not used
    const float la2 = la * kLog2e;
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
  // merge in the MFMA layout: lane (row l32, half hl) holds pieces 8db + 2g + hl
  auto stage_at = [&](int db, int g) __attribute__((always_inline)) {
    const int c = 8 * db + 2 * g + hl;
    return stage + 4 * (l32 * SPR + (c ^ (l32 & (SPR - 1))));
  };
  f32x4 prev[DB][4];
  if (a.accumulate) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) prev[db][g] = *(const f32x4*)stage_at(db, g);
  }
  const bool use_prev = a.accumulate && ca > 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        val[e] = cc * oacc[db][4 * g + e];
        val[e] = use_prev ? __builtin_fmaf(ca, prev[db][g][e], val[e]) : val[e];
      }
      *(f32x4*)stage_at(db, g) = val;
    }
  }
  // the copy-out reads pieces other lanes of the wave wrote
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  f32x4 outv[NIO];
#pragma unroll
  for (int i = 0; i < NIO; ++i) outv[i] = *(const f32x4*)(stage + 4 * (i * 64 + lane));
#pragma unroll
  for (int i = 0; i < NIO; ++i) {
    const int u = i * 64 + lane, r = u / SPR, c = (u % SPR) ^ (r & (SPR - 1));
    const f32x4 v = outv[i];
    if (r < vr) {
      const int64_t go = gbase + (int64_t)r * a.os_s + 4 * c;
      bf16x4 bv;
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[e] = (bf16)v[e];
      if (write_state) {
        if (a.o_f32)
          *(f32x4*)((float*)a.o + go) = v;
        else
          *(bf16x4*)((bf16*)a.o + go) = bv;
      }
      if (a.o_final) *(bf16x4*)(a.o_final + go) = bv;
    }
  }
  if (write_state && hl == 0 && row_ok) a.lse[lse_idx] = L2 * kLn2;
#endif
}

}  // namespace ba
