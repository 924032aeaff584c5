// Backward kernels: gradient of <dO, O> for one ring step (one key/value chunk).
//
// With S = tau Q K^T, P = exp(S - LSE) (LSE of the FINAL output, all chunks),
// dP = dO V^T and dS = P (dP - delta), delta_i = sum_d dO_id O_id:
//   dV = P^T dO,  dK = tau dS^T Q,  dQ = tau dS K.
// The pages train with exact attention (project page "How It Works"; LongLoRA
// and Ring Attention summaries) without printing the gradient; this is the
// analytic one.  Three kernels, no atomics:
//   delta_kernel  rowsum(dO * O) -> delta                            (HBM-bound)
//   dkdv_kernel   key/value-stationary: each lane owns one key; S, dP, and the
//                 dV, dK contractions over the query tiles the mask allows;
//                 GQA sums the group's query heads inside the item
//   dq_kernel     query-stationary: each lane owns one query row; S, dP and
//                 dQ over the key tiles the mask allows, then dq_acc += tau dQ
// Every MFMA is v_mfma_f32_32x32x16_bf16 with operands arranged as in the
// forward kernel (see ba_fwd.h): the stationary side is the B operand held in
// registers; tiles of the streamed side sit in the swizzled LDS layout of
// ba_common.h, filled by direct global->LDS loads and read directly for
// contractions over D, through ds_read_b64_tr_b16 for contractions over the
// streamed rows.
#pragma once

#include "ba_common.h"
#include "ba_schedule.h"

namespace ba {

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  float* delta;
  float* dq_acc;
  void* dk;
  void* dv;
  bf16* dq_final;
  int64_t qs_b, qs_s, qs_h;  // element strides of q
  int64_t ks_b, ks_s, ks_h;  // element strides of k, v, dk, dv
  int64_t os_b, os_s, os_h;  // element strides of o, dout, dq_acc, dq_final
  int64_t Sq, Sk, q_pos0, k_pos0;
  int32_t B, Hq, Hkv, grp;
  int32_t causal, s2_group, s2_shift_head0;
  int32_t dkv_f32, finalize;
  float scale, scale_log2;
  int64_t n_tiles;  // query tiles (dq_kernel) or key tiles (dkdv_kernel) per head
  int64_t n_ranks;  // dq_kernel: of the query tiles, the n_ranks longest are launched (the rest
                    // have no allowed key and, unless finalizing, nothing to do)
  int64_t n_items;
  int64_t hx;       // dq_kernel: heads interleaved per XCD (qitem_of_pid), 0 for head-major
};

constexpr int kDqBM = 128;   // query rows per dq item (4 waves x 32)
constexpr int kDqSlotsPerXcd = 64;  // two dq workgroups per CU, 32 CUs per XCD
constexpr int kDqBN = 64;    // key rows per streamed tile
constexpr int kKvBN = 128;   // keys per dkdv item (4 waves x 32)
constexpr int kKvBM = 64;    // query rows per streamed tile
constexpr int kBwdThreads = 256;
constexpr int kKvThreads = 512;  // dkdv: 4 key blocks x 2 waves

__device__ __forceinline__ Sched bwd_sched(const BwdArgs& a, int head, int BM, int BN) {
  Sched sc;
  sc.Sq = a.Sq; sc.Sk = a.Sk; sc.q_pos0 = a.q_pos0; sc.k_pos0 = a.k_pos0;
  sc.causal = a.causal; sc.s2_group = a.s2_group;
  sc.s2_shift = (a.s2_group > 0 && head >= a.s2_shift_head0) ? a.s2_group / 2 : 0;
  sc.BM = BM; sc.BN = BN;
  return sc;
}

// Direct loads of one R-row tile into the swizzled LDS layout: slot ci of the
// tile gets row ci / CPR, chunk (ci % CPR) ^ swz(row) of the source.  Rows past
// the end of a ragged tile re-read its last valid row (masked by the caller).
template <int D, int R, int THREADS = kBwdThreads>
struct TileLoader {
  static constexpr int CPR = D / 8;
  static constexpr int NW = THREADS / 64;
  static constexpr int NPI = R * CPR / (64 * NW);
  static constexpr int STEP = 64 * NW / CPR;  // rows between consecutive instructions
  // Slot ci = (p*NW + wave)*64 + lane is row ci / CPR = row0 + p*STEP; the row's
  // swizzle depends on row mod 16 only and STEP is a multiple of 16, so the
  // source chunk is the same for every instruction.
  int row0, col;
  __device__ __forceinline__ void init(int wave, int lane) {
    const int ci = wave * 64 + lane;
    row0 = ci / CPR;
    col = 8 * ((ci % CPR) ^ swz<D>(row0));
  }
  // src points at row 0 of the tile; rows are `stride` elements apart.  Buffer loads over a
  // resource spanning exactly the tile's valid rows: lanes of a ragged tile's missing rows
  // read past its end and get zeros (masked by the caller).
  __device__ __forceinline__ void issue(const bf16* src, int stride, int rows, bf16* dst, int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, 2u * (unsigned)((rows - 1) * stride + D));
#pragma unroll
    for (int p = 0; p < NPI; ++p)
      buf2lds16(rs, 2u * (unsigned)((row0 + p * STEP) * stride + col), 0u, dst + (p * NW + wave) * 512);
#endif
  }
};
static_assert(TileLoader<128, 64>::STEP % 16 == 0 && TileLoader<64, 64>::STEP % 16 == 0 &&
                  TileLoader<128, 64, kKvThreads / 2>::STEP % 16 == 0 &&
                  TileLoader<64, 64, kKvThreads / 2>::STEP % 16 == 0,
              "the loader assumes the swizzle repeats every STEP rows");

#if defined(__HIP_DEVICE_COMPILE__)
// bf16x8 MFMA operand from two transposing 8-byte LDS reads
__device__ __forceinline__ bf16x8 tr_pair(const bf16* base, int off0, int off1) {
  const bf16x4 x0 = lds_read_tr16(base + off0);
  const bf16x4 x1 = lds_read_tr16(base + off1);
  return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
}
#endif

// ---------------------------------------------------------------- delta = rowsum(dO * O)
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a, int64_t n_threads) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int CPR = D / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rowid = g / CPR;
  const int c = (int)(g % CPR);
  float acc = 0.f;
  int64_t b = 0, s = 0;
  int h = 0;
  if (g < n_threads) {
    h = (int)(rowid % a.Hq);
    s = (rowid / a.Hq) % a.Sq;
    b = rowid / ((int64_t)a.Hq * a.Sq);
    const int64_t off = b * a.os_b + s * a.os_s + (int64_t)h * a.os_h + 8 * c;
    const bf16x8 x = *(const bf16x8*)(a.dout + off);
    const bf16x8 y = *(const bf16x8*)(a.o + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
  }
  // CPR consecutive lanes of one wavefront hold one row
#pragma unroll
  for (int m = CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (g < n_threads && c == 0) a.delta[(b * a.Hq + h) * a.Sq + s] = acc;
#endif
}

// ---------------------------------------------------------------- dQ (query-stationary)
template <int D>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = kDqBM, BN = kDqBN;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BN * D;
  __shared__ __attribute__((aligned(16))) bf16 smem[4 * TILE];  // K0, V0, K1, V1 (swizzled)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, l32 = lane & 31;

  int64_t bh, w;
  qitem_of_pid(xcd_remap(blockIdx.x, a.n_items), a.n_ranks, a.hx, bh, w);
  const int b = (int)(bh / a.Hq);
  const int h = (int)(bh % a.Hq);
  const int kvh = h / a.grp;
  const Sched sc = bwd_sched(a, h, BM, BN);
  const QTile qt = make_qtile(sc, qtile_of_rank(sc, a.n_tiles, w));
  const bool empty = qt.kt_end <= qt.kt_begin;
  if (empty && !a.finalize) return;

  const int rloc = wave * 32 + l32;
  const bool row_ok = rloc < qt.rows;
  const int64_t row = qt.row0 + rloc;
  const int64_t wave_cmin = qt.cpos0 + wave * 32;
  const int64_t wave_cmax = wave_cmin + 31;
  const int64_t lse_idx = ((int64_t)b * a.Hq + h) * a.Sq + row;
  const int64_t qoff = (int64_t)b * a.qs_b + row * a.qs_s + (int64_t)h * a.qs_h;
  const int64_t ooff = (int64_t)b * a.os_b + row * a.os_s + (int64_t)h * a.os_h;

  f32x16 dqacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dqacc[i] = f32x16{};

  if (!empty) {
    const float lse2 = row_ok ? a.lse[lse_idx] * kLog2e : INFINITY;
    const float dlt = row_ok ? a.delta[lse_idx] : 0.f;
    bf16x8 qf[KK], df[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[kk] = row_ok ? *(const bf16x8*)(a.q + qoff + 16 * kk + 8 * hl) : bf16x8{};
      df[kk] = row_ok ? *(const bf16x8*)(a.dout + ooff + 16 * kk + 8 * hl) : bf16x8{};
    }
    // per-lane LDS offsets: direct reads (row l32, chunk 2kk+hl) and transposed reads
    int n_off[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) n_off[kk] = tile_off<D>(l32, 16 * kk + 8 * hl);
    const int gi = lane & 15;
    const int r0 = 4 * hl + (gi >> 2);
    int t_off[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dcol = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
      t_off[db][0] = tile_off<D>(r0, dcol);
      t_off[db][1] = tile_off<D>(r0 + 8, dcol);
    }
    TileLoader<D, BN> ld;
    ld.init(wave, lane);
    const bf16* kbase = a.k + (int64_t)b * a.ks_b + (int64_t)kvh * a.ks_h;
    const bf16* vbase = a.v + (int64_t)b * a.ks_b + (int64_t)kvh * a.ks_h;
    const int ks_s = (int)a.ks_s;
    auto issue = [&](bf16* kd, bf16* vd, int64_t kt) {
      const KTile t = make_ktile(sc, kt);
      ld.issue(kbase + t.row0 * a.ks_s, ks_s, (int)t.rows, kd, wave);
      ld.issue(vbase + t.row0 * a.ks_s, ks_s, (int)t.rows, vd, wave);
    };

    // Per-wave tile thresholds, once per item, relative to the item's first key tile (32-bit
    // scalar compares per tile; 64-bit signed compares go to the vector ALU): the key
    // coordinate of tile kt is c0 + kt*BN (make_ktile), so from act_end on every key of a tile
    // comes after every row of this wave (causal), and from mask_from on a tile needs the mask
    // (causal diagonal, or the chunk's ragged last tile).
    constexpr int LBN = __builtin_ctz(BN);
    static_assert((1 << LBN) == BN, "floor division by BN as a shift");
    const int64_t kt_b = qt.kt_begin;
    const int T = (int)(qt.kt_end - qt.kt_begin);
    const int64_t c0 = a.s2_group > 0 ? 0 : a.k_pos0;
    const int64_t act_end = a.causal ? ((wave_cmax - c0) >> LBN) + 1 : INT64_MAX;
    int64_t mask_from = a.causal ? ((wave_cmin - c0 + 1) >> LBN) : INT64_MAX;
    if (a.s2_group == 0 && a.Sk % BN != 0) {
      const int64_t last = ceil_div(a.Sk, BN) - 1;
      mask_from = last < mask_from ? last : mask_from;
    }
    auto rel = [&](int64_t kt) {
      const int64_t r = kt - kt_b;
      return (int)(r < 0 ? 0 : (r > T + 1 ? T + 1 : r));
    };
    const int act_rel = rel(act_end), mask_rel = rel(mask_from);

    auto tile_step = [&](const bf16* Ks, const bf16* Vs, int j) {
      if (j >= act_rel) return;  // every key after every row of this wave
      const bool need_mask = j >= mask_rel;
      int lim = BN;
      if (need_mask) {
        const KTile t = make_ktile(sc, kt_b + j);
        lim = (int)t.rows - 1;
        if (a.causal) {
          int64_t c = wave_cmin - t.cpos0;
          c = c > BN ? BN : c;
          const int cl = (int)c + l32;
          lim = cl < lim ? cl : lim;
        }
      }
      f32x16 s[2], dp[2];
      bf16x8 dsf[2][2];
      auto scores = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          s[kb] = mfma32(*(const bf16x8*)(Ks + kb * 32 * D + n_off[kk]), qf[kk], kk == 0 ? f32x16{} : s[kb]);
          dp[kb] = mfma32(*(const bf16x8*)(Vs + kb * 32 * D + n_off[kk]), df[kk], kk == 0 ? f32x16{} : dp[kb]);
        }
      };
      // keys past the tile's valid rows or (causal) after this lane's row get a score of
      // -inf, so that P = 0 there: only the scores branch on the mask, and both kinds of
      // tile share one MFMA schedule (with two paths, the compiler copies the whole dQ
      // accumulator to merge them)
      auto mask = [&](int kb) __attribute__((always_inline)) {
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            s[kb][r] = key <= lim ? s[kb][r] : -INFINITY;
          }
        }
      };
      auto make_ds = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_hw(__builtin_fmaf(s[kb][r], a.scale_log2, -lse2));
          dsf[kb][r >> 3][r & 7] = (bf16)(p * (dp[kb][r] - dlt));
        }
      };
      // dQ^T += K^T dS^T: K^T operand read transposed from the [key][d] tile
      // (strict: the reads stay two MFMAs ahead; not where another block's vector work is
      // interleaved with these MFMAs)
      auto accumulate = [&](int kb, bool strict) __attribute__((always_inline)) {
        bf16x8 tf[3];
        auto rdt = [&](int j) __attribute__((always_inline)) {
          const int db = j >> 1, c2 = j & 1;
          tf[j % 3] = tr_pair(Ks + (kb * 32 + 16 * c2) * D, t_off[db][0], t_off[db][1]);
        };
        rdt(0);
        rdt(1);
#pragma unroll
        for (int j = 0; j < 2 * DB; ++j) {
          if (j + 2 < 2 * DB) rdt(j + 2);
          if (strict) __builtin_amdgcn_sched_barrier(0);
          dqacc[j >> 1] = mfma32(tf[j % 3], dsf[kb][j & 1], dqacc[j >> 1]);
          if (strict) __builtin_amdgcn_sched_barrier(0);
        }
      };
      // each 32-key block's vector work runs between the MFMAs of the next step (block 1's
      // scores, then block 0's dQ)
      scores(0);
      __builtin_amdgcn_sched_barrier(0);
      mask(0);
      __builtin_amdgcn_sched_barrier(0);
      scores(1);
      make_ds(0);
      for (int j = 0; j < 2 * KK; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);  // four VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      mask(1);
      __builtin_amdgcn_sched_barrier(0);
      accumulate(0, false);
      make_ds(1);
      for (int j = 0; j < 2 * DB; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x402, 8, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      accumulate(1, true);
    };

    bf16* K0 = smem;
    bf16* V0 = smem + TILE;
    bf16* K1 = smem + 2 * TILE;
    bf16* V1 = smem + 3 * TILE;
    issue(K0, V0, kt_b);
    wait_vmem();
    __syncthreads();
    for (int j = 0; j < T; j += 2) {
      if (j + 1 < T) issue(K1, V1, kt_b + j + 1);
      tile_step(K0, V0, j);
      wait_vmem();
      __syncthreads();
      if (j + 1 >= T) break;
      if (j + 2 < T) issue(K0, V0, kt_b + j + 2);
      tile_step(K1, V1, j + 1);
      wait_vmem();
      __syncthreads();
    }
  }

  if (!row_ok) return;
  const int64_t obase = ooff + 4 * hl;
  // the lane's dq_acc row is read whole before any store: one memory round trip
  // for the wave instead of one per 16-byte piece
  f32x4 prev[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) prev[db][g] = *(const f32x4*)(a.dq_acc + obase + 32 * db + 8 * g);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t off = obase + 32 * db + 8 * g;
      f32x4 val = prev[db][g];
      if (!empty) {
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = __builtin_fmaf(a.scale, dqacc[db][4 * g + e], val[e]);
        *(f32x4*)(a.dq_acc + off) = val;
      }
      if (a.finalize) {
        bf16x4 bv;
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = (bf16)val[e];
        *(bf16x4*)(a.dq_final + off) = bv;
      }
    }
  }
#endif
}

// ---------------------------------------------------------------- dK, dV (key/value-stationary)
// Eight waves: each 32-key block of the item is owned by a PAIR of waves that
// share a SIMD.  The P wave holds K and computes S, P = exp(S - LSE) and
// dV += P^T dO; the dS wave holds V and computes dP = dO V^T, dS = P (dP -
// delta) and dK += dS^T Q, taking P from the P wave through LDS (bf16, in the
// accumulator layout both waves share: lane = key, register = query).  The dS
// wave's dP accumulator starts at -delta, so its MFMAs leave dP - delta and dS
// costs one product per element.  Each
// tile of 64 query rows has two phases per wave: the score / dP MFMAs (with
// the softmax on the P wave), then the two gradient contractions.  The phases
// are skewed by one tile: between two barriers every wave runs phase 2 of
// tile j - 1 and then phase 1 of tile j, so the dS wave's second phase (the
// heavier one: dS on the vector ALU, then dK) overlaps the P wave's first
// phase (the softmax) instead of following it.  One barrier per tile; three
// tile buffers (tile j + 1 loads while tiles j - 1 and j are read) and two P
// buffers.  Each wave keeps one stationary operand and one accumulator set,
// so two waves fit on a SIMD and each one's VALU work runs under the other's
// MFMAs.  The P waves issue every tile load: both waves of a pair leave the
// same barrier, and loads issued by both would hold both at issue while the
// SIMD's matrix core idles.
template <int D>
__global__ __launch_bounds__(kKvThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = kKvBM, BN = kKvBN;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BM * D;
  constexpr int NKB = BN / 32;  // key blocks = wave pairs
  // three buffers, each a Q tile followed by a dO tile (swizzled); separate
  // arrays so prefetches into one buffer do not make the compiler wait before
  // reading the others
  __shared__ __attribute__((aligned(16))) bf16 sT0[2 * TILE], sT1[2 * TILE], sT2[2 * TILE];
  __shared__ __attribute__((aligned(16))) float stat[3][2][BM];  // [buffer][lse*log2e, -delta][row]
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][NKB][2][2][64];  // [parity][key block][qb][half][lane]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, l32 = lane & 31;
  const int kblk = wave % NKB;
  const bool pwave = wave < NKB;  // P / dV wave; otherwise dP / dS / dK wave

  const int64_t pid = xcd_remap(blockIdx.x, a.n_items);
  const int64_t bkv = pid / a.n_tiles;
  const int64_t w = pid % a.n_tiles;
  const int b = (int)(bkv / a.Hkv);
  const int kvh = (int)(bkv % a.Hkv);
  const int h0 = kvh * a.grp;
  const Sched sc = bwd_sched(a, h0, BM, BN);  // every head of the group shares the shift
  const KVItem it = make_kv_item(sc, ktile_of_rank(sc, a.n_tiles, w));

  const int kloc = kblk * 32 + l32;
  const bool key_ok = kloc < it.krows;
  const int64_t krow = it.krow0 + kloc;
  const int64_t kcpos = it.kcpos0 + kloc;
  const int64_t wave_kmin = it.kcpos0 + kblk * 32;
  const int64_t wave_kmax = wave_kmin + 31;
  const int64_t koff = (int64_t)b * a.ks_b + krow * a.ks_s + (int64_t)kvh * a.ks_h;

  // stationary operand: K rows (P wave) or V rows (dS wave)
  bf16x8 sf[KK];
  {
    const bf16* src = pwave ? a.k : a.v;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sf[kk] = key_ok ? *(const bf16x8*)(src + koff + 16 * kk + 8 * hl) : bf16x8{};
  }
  f32x16 acc[DB];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  const int64_t nqt = it.qt_end > it.qt_begin ? it.qt_end - it.qt_begin : 0;
  const int n_iter = (int)(nqt * a.grp);  // query tiles x heads of the group (32-bit loop control)
  if (n_iter > 0) {
    int n_off[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) n_off[kk] = tile_off<D>(l32, 16 * kk + 8 * hl);
    const int gi = lane & 15;
    const int r0 = 4 * hl + (gi >> 2);
    int t_off[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dcol = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
      t_off[db][0] = tile_off<D>(r0, dcol);
      t_off[db][1] = tile_off<D>(r0 + 8, dcol);
    }
    // only the four P waves load tiles (8 direct loads each per tile): a burst of loads
    // holds its wave at issue for hundreds of cycles, and the P wave, with the lighter
    // phases, has that slack while its dS partner on the same SIMD goes on with its MFMAs
    TileLoader<D, BM, kKvThreads / 2> ld;
    ld.init(wave, lane);
    const int qs_s = (int)a.qs_s;
    const int os_s = (int)a.os_s;
    // tiles run over the group's heads, each over the query tiles [qt_begin, qt_end); the
    // loads and the compute each keep their own position (no divisions per tile)
    struct Pos {
      int head;
      int64_t qtile;
    };
    auto advance = [&](Pos& p) {
      if (++p.qtile == it.qt_end) {
        p.qtile = it.qt_begin;
        ++p.head;
      }
    };
    Pos pos_load{h0, it.qt_begin}, pos_comp{h0, it.qt_begin};
    // stage a tile: LSE and delta by ordinary loads (issued first, written to LDS
    // only after the interval's compute), Q and dO by direct loads
    float st_l = INFINITY, st_d = 0.f;
    bool st_ok = false;
    auto issue = [&](bf16* qd) {
      const int hh = pos_load.head;
      const QTile t = make_qtile(sc, pos_load.qtile);
      advance(pos_load);
      if (tid < BM) {
        st_ok = tid < t.rows;
        const int64_t li = ((int64_t)b * a.Hq + hh) * a.Sq + t.row0 + (st_ok ? tid : 0);
        st_l = a.lse[li];
        st_d = a.delta[li];
      }
      const int64_t qbase = (int64_t)b * a.qs_b + t.row0 * a.qs_s + (int64_t)hh * a.qs_h;
      const int64_t obase = (int64_t)b * a.os_b + t.row0 * a.os_s + (int64_t)hh * a.os_h;
      if (pwave) {
        ld.issue(a.q + qbase, qs_s, (int)t.rows, qd, wave);
        ld.issue(a.dout + obase, os_s, (int)t.rows, qd + TILE, wave);
      }
    };
    auto put_stats = [&](int buf) {
      if (tid < BM) {
        stat[buf][0][tid] = st_ok ? st_l * kLog2e : INFINITY;
        stat[buf][1][tid] = st_ok ? -st_d : 0.f;
      }
    };

    // state of the tile between its two phases: which query blocks the mask
    // leaves active and S (P wave) or dP (dS wave)
    bool act[2] = {false, false};
    f32x16 x[2];

    // ---- phase 1: S^T = K Q^T (P wave) or dP^T = V dO^T (dS wave), 32 queries per
    // block (fragments read one pair of k-steps ahead of the MFMAs that use them);
    // the P wave then forms P and hands it to the dS wave through pbuf[par]
    auto phase1 = [&](const bf16* QDs, int sbuf, int par) __attribute__((always_inline)) {
      const QTile t = make_qtile(sc, pos_comp.qtile);
      advance(pos_comp);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) act[qb] = !(a.causal && wave_kmin > t.cpos0 + qb * 32 + 31);
      const float* lse_s = stat[sbuf][0];
      const float* ndel_s = stat[sbuf][1];
      const bf16* Xs = QDs + (pwave ? 0 : TILE);
      auto contract = [&](int qb, bool strict) __attribute__((always_inline)) {
        bf16x8 fr[2][2];
        auto rd = [&](int kk2, int set) __attribute__((always_inline)) {
          fr[set][0] = *(const bf16x8*)(Xs + qb * 32 * D + n_off[2 * kk2]);
          fr[set][1] = *(const bf16x8*)(Xs + qb * 32 * D + n_off[2 * kk2 + 1]);
        };
        // the dS wave's dP^T accumulator starts at -delta (each register's query row, the
        // same in every key lane), so that its MFMAs leave dP - delta
        f32x16 init = f32x16{};
        if (!pwave) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 d4 = *(const f32x4*)(ndel_s + qb * 32 + 8 * g + 4 * hl);
#pragma unroll
            for (int e = 0; e < 4; ++e) init[4 * g + e] = d4[e];
          }
        }
        rd(0, 0);
#pragma unroll
        for (int kk2 = 0; kk2 < KK / 2; ++kk2) {
          if (kk2 + 1 < KK / 2) rd(kk2 + 1, (kk2 + 1) & 1);
          // strict: each pair's reads stay ahead of the MFMAs (left to itself the scheduler
          // reuses one register quad and waits on every read); not where another block's
          // vector work is interleaved with these MFMAs
          if (strict) __builtin_amdgcn_sched_barrier(0);
          x[qb] = mfma32(fr[kk2 & 1][0], sf[2 * kk2], kk2 == 0 ? init : x[qb]);
          x[qb] = mfma32(fr[kk2 & 1][1], sf[2 * kk2 + 1], x[qb]);
          if (strict) __builtin_amdgcn_sched_barrier(0);
        }
      };
      // P = exp(S - LSE) of block qb (zero where masked), in bf16 to LDS for both
      // waves' second phase
      auto softmax = [&](int qb, bool need_mask) __attribute__((always_inline)) {
        bf16x8 pf[2];
        const int64_t qc0 = t.cpos0 + qb * 32;
        // allowed iff key_ok and (not causal or query coordinate >= key coordinate)
        int qmin = -1;  // smallest allowed query index inside the block, relative to qc0
        if (need_mask) {
          if (!key_ok) {
            qmin = 64;
          } else if (a.causal) {
            int64_t c = kcpos - qc0;
            c = c < -1 ? -1 : (c > 64 ? 64 : c);
            qmin = (int)c;
          }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *(const f32x4*)(lse_s + qb * 32 + 8 * g + 4 * hl);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float p = exp2_hw(__builtin_fmaf(x[qb][r], a.scale_log2, -l4[e]));
            if (need_mask) p = (8 * g + 4 * hl + e) >= qmin ? p : 0.f;
            pf[r >> 3][r & 7] = (bf16)p;
          }
        }
        pbuf[par][kblk][qb][0][lane] = pf[0];
        pbuf[par][kblk][qb][1][lane] = pf[1];
      };
      auto need_mask_of = [&](int qb) {
        return (t.rows < BM) || (it.krows < BN) || (a.causal && wave_kmax > t.cpos0 + qb * 32);
      };
      if (pwave && act[0] && act[1] && !need_mask_of(0)) {
        // common case, straight-line: block 1's score MFMAs interleaved with block 0's
        // softmax so that the wave's vector work runs under its own matrix work
        contract(0, true);
        __builtin_amdgcn_sched_barrier(0);
        contract(1, false);
        softmax(0, false);
        for (int j = 0; j < KK; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);  // five VALU / transcendental
        }
        __builtin_amdgcn_sched_barrier(0);
        softmax(1, false);
      } else {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          if (act[qb]) contract(qb, true);
        if (pwave) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            if (act[qb]) softmax(qb, need_mask_of(qb));
        }
      }
    };

    // ---- phase 2: dV^T += dO^T P (P wave) or dK^T += Q^T dS (dS wave); the
    // transposed operand is read from the [query][d] tile
    auto phase2 = [&](const bf16* QDs, int par) __attribute__((always_inline)) {
      const bf16* Ys = QDs + (pwave ? TILE : 0);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (!act[qb]) continue;
        // transposed fragments read two MFMAs ahead of their use; the first two are issued
        // with the P reads, before the dS wave's vector work
        bf16x8 tf[3];
        auto rdt = [&](int j) __attribute__((always_inline)) {
          const int db = j >> 1, c2 = j & 1;
          tf[j % 3] = tr_pair(Ys + (qb * 32 + 16 * c2) * D, t_off[db][0], t_off[db][1]);
        };
        bf16x8 yf[2];
        if (pwave) {
          // its own P, back from LDS: no registers held across the barrier
          yf[0] = pbuf[par][kblk][qb][0][lane];
          yf[1] = pbuf[par][kblk][qb][1][lane];
          rdt(0);
          rdt(1);
        } else {
          const bf16x8 p0 = pbuf[par][kblk][qb][0][lane];
          const bf16x8 p1 = pbuf[par][kblk][qb][1][lane];
          rdt(0);
          rdt(1);
          __builtin_amdgcn_sched_barrier(0);
          // dS = P (dP - delta); x already holds dP - delta
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = (float)(r < 8 ? p0[r & 7] : p1[r & 7]);
            yf[r >> 3][r & 7] = (bf16)(p * x[qb][r]);
          }
        }
#pragma unroll
        for (int j = 0; j < 2 * DB; ++j) {
          if (j + 2 < 2 * DB) rdt(j + 2);
          __builtin_amdgcn_sched_barrier(0);
          acc[j >> 1] = mfma32(tf[j % 3], yf[j & 1], acc[j >> 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // interval j (0 <= j <= n_iter): phase 2 of tile j - 1 (buffer Tp), the loads of
    // tile j + 1 into Tl (issued after phase 2, when the dS waves are deep in their
    // heavier phase 2), phase 1 of tile j (buffer Tc); buffer and statistics slots
    // rotate with j mod 3, P slots with j mod 2
    auto interval = [&](bf16* Tc, const bf16* Tp, bf16* Tl, int j, int rot) __attribute__((always_inline)) {
      const int par = (int)(j & 1);
      if (j >= 1) phase2(Tp, par ^ 1);
      if (j + 1 < n_iter) issue(Tl);
      // x and pf are rewritten by phase 1: keep the two phases apart
      __builtin_amdgcn_sched_barrier(0);
      if (j < n_iter) phase1(Tc, rot, par);
      if (j + 1 < n_iter) put_stats(rot == 2 ? 0 : rot + 1);
      wait_vmem();
      __syncthreads();
    };

    issue(sT0);
    put_stats(0);
    wait_vmem();
    __syncthreads();
    // unrolled by three so that every buffer sits at a fixed LDS address
    for (int j = 0;; j += 3) {
      interval(sT0, sT2, sT1, j, 0);
      if (j + 1 > n_iter) break;
      interval(sT1, sT0, sT2, j + 1, 1);
      if (j + 2 > n_iter) break;
      interval(sT2, sT1, sT0, j + 2, 2);
      if (j + 3 > n_iter) break;
    }
  }

  if (!key_ok) return;
  const int64_t obase = koff + 4 * hl;
  void* const dst = pwave ? a.dv : a.dk;
  const float mul = pwave ? 1.f : a.scale;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t off = obase + 32 * db + 8 * g;
      f32x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = mul * acc[db][4 * g + e];
      if (a.dkv_f32) {
        *(f32x4*)((float*)dst + off) = v4;
      } else {
        bf16x4 b4;
#pragma unroll
        for (int e = 0; e < 4; ++e) b4[e] = (bf16)v4[e];
        *(bf16x4*)((bf16*)dst + off) = b4;
      }
    }
  }
#endif
}

}  // namespace ba
