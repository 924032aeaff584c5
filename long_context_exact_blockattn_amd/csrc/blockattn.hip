// C ABI of the blockwise attention library: validation, dispatch, launches.
// Declarations and the contract of every entry point are in include/blockattn.h.
#include "../../include/blockattn.h"

#include <math.h>

#include <algorithm>
#include <cmath>

#include "ba_bwd.h"
#include "ba_common.h"
#include "ba_ffn.h"
#include "ba_fwd.h"
#include "ba_merge.h"
#include "ba_schedule.h"
#include "ba_ulysses.h"

namespace {

using namespace ba;

// the forward epilogue stages each wave's 32 fp32 rows in one of its eight tile-sized arrays
static_assert(kFwdWaves == 8 && kFwdBM == 32 * kFwdWaves && 32 * 4 <= kFwdBN * 2,
              "a wave's staged rows (32 x D fp32) must fit one tile buffer (BN x D bf16)");

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

int check_strides(const int64_t s[3]) {
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || s[i] % 8 != 0) return BA_ERR_STRIDE;
  // the kernels address a tile's rows with 32-bit byte offsets from its first row
  if (s[1] >= ((int64_t)1 << 24)) return BA_ERR_STRIDE;
  return BA_OK;
}

// Shape/stride checks common to every entry point.
int check_desc(const ba_desc* d) {
  if (!d) return BA_ERR_NULL;
  if (d->batch < 0 || d->heads_q < 1 || d->heads_kv < 1 || d->seqlen_q < 0 || d->seqlen_k < 0)
    return BA_ERR_SHAPE;
  if (d->heads_q % d->heads_kv != 0) return BA_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return BA_ERR_UNSUPPORTED;
  if (d->causal != 0 && d->causal != 1) return BA_ERR_SHAPE;
  int r = check_strides(d->q_stride);
  if (r) return r;
  if ((r = check_strides(d->kv_stride))) return r;
  return check_strides(d->o_stride);
}

int check_s2(const ba_desc* d, const ba_s2_desc* s2) {
  if (!s2) return BA_ERR_NULL;
  if (d->seqlen_q != d->seqlen_k || d->q_pos0 != 0 || d->k_pos0 != 0 || d->causal != 1)
    return BA_ERR_S2;
  if (s2->group <= 0 || s2->group % 2 != 0) return BA_ERR_S2;
  if (d->seqlen_q % s2->group != 0) return BA_ERR_S2;
  if ((s2->group / 2) % kFwdBM != 0) return BA_ERR_S2;
  const int grp = d->heads_q / d->heads_kv;
  if (s2->shift_head0 < 0 || s2->shift_head0 > d->heads_q || s2->shift_head0 % grp != 0)
    return BA_ERR_S2;
  return BA_OK;
}

float scale_of(const ba_desc* d) {
  return d->scale > 0.f ? d->scale : (float)(1.0 / sqrt((double)d->head_dim));
}

int launched() { return hipGetLastError() == hipSuccess ? BA_OK : BA_ERR_LAUNCH; }

Sched sched_of(const ba_desc* d, const ba_s2_desc* s2, int head) {
  Sched s;
  s.Sq = d->seqlen_q; s.Sk = d->seqlen_k; s.q_pos0 = d->q_pos0; s.k_pos0 = d->k_pos0;
  s.causal = s2 ? 1 : d->causal;
  s.s2_group = s2 ? s2->group : 0;
  s.s2_shift = (s2 && head >= s2->shift_head0) ? s2->group / 2 : 0;
  s.BM = kFwdBM; s.BN = kFwdBN;
  return s;
}

int fwd_impl(const ba_desc* d, const ba_s2_desc* s2, const void* q, const void* k, const void* v,
             void* o, int32_t o_dtype, float* lse, int32_t mode, void* o_final, hipStream_t stream) {
  int r = check_desc(d);
  if (r) return r;
  if (!std::isfinite(d->scale)) return BA_ERR_SHAPE;
  if (s2 && (r = check_s2(d, s2))) return r;
  const bool final_reached_only = (mode & BA_FINAL_REACHED_ONLY) != 0;
  mode &= ~(int32_t)BA_FINAL_REACHED_ONLY;
  if (mode != BA_OVERWRITE && mode != BA_ACCUMULATE) return BA_ERR_MODE;
  if (o_dtype != BA_F32 && o_dtype != BA_BF16) return BA_ERR_UNSUPPORTED;
  if (mode == BA_ACCUMULATE && o_dtype != BA_F32) return BA_ERR_MODE;
  if (d->batch == 0 || d->seqlen_q == 0) return BA_OK;
  if (!q || !o || !lse) return BA_ERR_NULL;
  if (d->seqlen_k > 0 && (!k || !v)) return BA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 4) || !aligned(o_final, 16) ||
      !aligned(k, 16) || !aligned(v, 16))
    return BA_ERR_ALIGN;

  FwdArgs a;
  a.q = (const bf16*)q; a.k = (const bf16*)k; a.v = (const bf16*)v;
  a.o = o; a.lse = lse; a.o_final = (bf16*)o_final;
  a.qs_b = d->q_stride[0]; a.qs_s = d->q_stride[1]; a.qs_h = d->q_stride[2];
  a.ks_b = d->kv_stride[0]; a.ks_s = d->kv_stride[1]; a.ks_h = d->kv_stride[2];
  a.os_b = d->o_stride[0]; a.os_s = d->o_stride[1]; a.os_h = d->o_stride[2];
  a.Sq = d->seqlen_q; a.Sk = d->seqlen_k; a.q_pos0 = d->q_pos0; a.k_pos0 = d->k_pos0;
  a.B = d->batch; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.grp = d->heads_q / d->heads_kv;
  a.causal = s2 ? 1 : d->causal;
  a.accumulate = mode == BA_ACCUMULATE;
  a.o_f32 = o_dtype == BA_F32;
  a.s2_group = s2 ? s2->group : 0;
  a.s2_shift_head0 = s2 ? s2->shift_head0 : 0;
  a.scale_log2 = scale_of(d) * kLog2e;
  a.n_qtiles = ceil_div(d->seqlen_q, kFwdBM);
  // ACCUMULATE leaves rows the chunk cannot reach untouched, so causal query
  // tiles wholly before the chunk are not launched (they are the last ranks of
  // the longest-first order); their final bf16 store, if asked for, is a plain
  // conversion of the running output
  int64_t skip_qt = 0;
  if (!s2 && d->causal && mode == BA_ACCUMULATE) {
    int64_t first_row = d->seqlen_k > 0 ? d->k_pos0 - d->q_pos0 : d->seqlen_q;
    first_row = first_row < 0 ? 0 : (first_row > d->seqlen_q ? d->seqlen_q : first_row);
    skip_qt = first_row / kFwdBM;
  }
  a.n_ranks = a.n_qtiles - skip_qt;
  a.n_items = (int64_t)d->batch * d->heads_q * a.n_ranks;
  // heads interleaved per XCD while a head has fewer than four rounds of the XCD's slots (the
  // ring's steps with few reached tiles per head: 32K ring +1.1 % against two rounds)
  a.hx = interleave_heads((int64_t)d->batch * d->heads_q, a.n_ranks, 2 * kFwdSlotsPerXcd);
  if (a.n_items > 0x7fffffffLL) return BA_ERR_SHAPE;
  if (o_final && skip_qt > 0 && !final_reached_only) {
    StoreArgs st;
    st.o_acc = (const float*)o;
    st.o_final = (bf16*)o_final;
    st.s_b = d->o_stride[0]; st.s_s = d->o_stride[1]; st.s_h = d->o_stride[2];
    st.rows = skip_qt * kFwdBM;
    st.Hq = d->heads_q; st.D = d->head_dim;
    st.n_threads = (int64_t)d->batch * st.rows * d->heads_q * (d->head_dim / 8);
    const int64_t blocks = ceil_div(st.n_threads, 256);
    if (blocks > 0x7fffffffLL) return BA_ERR_SHAPE;
    hipLaunchKernelGGL(store_final_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, st);
    if ((r = launched())) return r;
  }
  if (a.n_items == 0) return BA_OK;
  const dim3 grid((unsigned)a.n_items), block(kFwdThreads);
  if (d->head_dim == 128)
    hipLaunchKernelGGL(fwd_kernel<128>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_kernel<64>, grid, block, 0, stream, a);
  return launched();
}

int bwd_impl(const ba_desc* d, const ba_s2_desc* s2, const void* q, const void* k, const void* v,
             const void* o, const void* dout, const float* lse, float* delta, float* dq_acc, void* dk,
             void* dv, int32_t dkv_dtype, void* dq_final, int32_t flags, hipStream_t stream) {
  int r = check_desc(d);
  if (r) return r;
  if (!std::isfinite(d->scale)) return BA_ERR_SHAPE;
  if (s2 && (r = check_s2(d, s2))) return r;
  if (flags & ~(BA_BWD_COMPUTE_DELTA | BA_BWD_FINALIZE_DQ)) return BA_ERR_MODE;
  if (dkv_dtype != BA_F32 && dkv_dtype != BA_BF16) return BA_ERR_UNSUPPORTED;
  if (d->batch == 0 || (d->seqlen_q == 0 && d->seqlen_k == 0)) return BA_OK;
  const bool finalize = (flags & BA_BWD_FINALIZE_DQ) != 0;
  if (d->seqlen_q > 0 && (!q || !o || !dout || !lse || !delta || !dq_acc)) return BA_ERR_NULL;
  if (d->seqlen_q > 0 && finalize && !dq_final) return BA_ERR_NULL;
  if (d->seqlen_k > 0 && (!k || !v || !dk || !dv)) return BA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq_acc, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dq_final, 16) ||
      !aligned(lse, 4) || !aligned(delta, 4))
    return BA_ERR_ALIGN;

  BwdArgs a;
  a.q = (const bf16*)q; a.k = (const bf16*)k; a.v = (const bf16*)v;
  a.o = (const bf16*)o; a.dout = (const bf16*)dout;
  a.lse = lse; a.delta = delta; a.dq_acc = dq_acc; a.dk = dk; a.dv = dv;
  a.dq_final = (bf16*)dq_final;
  a.qs_b = d->q_stride[0]; a.qs_s = d->q_stride[1]; a.qs_h = d->q_stride[2];
  a.ks_b = d->kv_stride[0]; a.ks_s = d->kv_stride[1]; a.ks_h = d->kv_stride[2];
  a.os_b = d->o_stride[0]; a.os_s = d->o_stride[1]; a.os_h = d->o_stride[2];
  a.Sq = d->seqlen_q; a.Sk = d->seqlen_k; a.q_pos0 = d->q_pos0; a.k_pos0 = d->k_pos0;
  a.B = d->batch; a.Hq = d->heads_q; a.Hkv = d->heads_kv; a.grp = d->heads_q / d->heads_kv;
  a.causal = s2 ? 1 : d->causal;
  a.s2_group = s2 ? s2->group : 0;
  a.s2_shift_head0 = s2 ? s2->shift_head0 : 0;
  a.dkv_f32 = dkv_dtype == BA_F32;
  a.finalize = finalize;
  a.scale = scale_of(d);
  a.scale_log2 = a.scale * kLog2e;
  a.n_tiles = a.n_ranks = a.n_items = a.hx = 0;
  const bool d128 = d->head_dim == 128;

  if ((flags & BA_BWD_COMPUTE_DELTA) && d->seqlen_q > 0) {
    const int64_t n = (int64_t)d->batch * d->seqlen_q * d->heads_q * (d->head_dim / 8);
    const int64_t blocks = ceil_div(n, 256);
    if (blocks > 0x7fffffffLL) return BA_ERR_SHAPE;
    if (d128)
      hipLaunchKernelGGL(bwd_delta_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, a, n);
    else
      hipLaunchKernelGGL(bwd_delta_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, a, n);
    if ((r = launched())) return r;
  }
  if (d->seqlen_k > 0) {
    BwdArgs b = a;
    b.n_tiles = ceil_div(d->seqlen_k, kKvBN);
    b.n_items = (int64_t)d->batch * d->heads_kv * b.n_tiles;
    if (b.n_items > 0x7fffffffLL) return BA_ERR_SHAPE;
    if (d128)
      hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3((unsigned)b.n_items), dim3(kKvThreads), 0, stream, b);
    else
      hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3((unsigned)b.n_items), dim3(kKvThreads), 0, stream, b);
    if ((r = launched())) return r;
  }
  if (d->seqlen_q > 0) {
    BwdArgs b = a;
    b.n_tiles = ceil_div(d->seqlen_q, kDqBM);
    // causal query tiles wholly before the chunk have no allowed key (they are the last
    // ranks of the longest-first order) and are not launched; when finalizing, their bf16 dQ
    // is a plain conversion of the accumulator
    int64_t skip_qt = 0;
    if (!s2 && d->causal) {
      int64_t first_row = d->seqlen_k > 0 ? d->k_pos0 - d->q_pos0 : d->seqlen_q;
      first_row = first_row < 0 ? 0 : (first_row > d->seqlen_q ? d->seqlen_q : first_row);
      skip_qt = first_row / kDqBM;
    }
    b.n_ranks = b.n_tiles - skip_qt;
    b.n_items = (int64_t)d->batch * d->heads_q * b.n_ranks;
    b.hx = interleave_heads((int64_t)d->batch * d->heads_q, b.n_ranks, kDqSlotsPerXcd);
    if (b.n_items > 0x7fffffffLL) return BA_ERR_SHAPE;
    if (finalize && skip_qt > 0) {
      StoreArgs st;
      st.o_acc = dq_acc;
      st.o_final = (bf16*)dq_final;
      st.s_b = d->o_stride[0]; st.s_s = d->o_stride[1]; st.s_h = d->o_stride[2];
      st.rows = skip_qt * kDqBM;
      st.Hq = d->heads_q; st.D = d->head_dim;
      st.n_threads = (int64_t)d->batch * st.rows * d->heads_q * (d->head_dim / 8);
      const int64_t blocks = ceil_div(st.n_threads, 256);
      if (blocks > 0x7fffffffLL) return BA_ERR_SHAPE;
      hipLaunchKernelGGL(store_final_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, st);
      if ((r = launched())) return r;
    }
    if (b.n_items == 0) return BA_OK;
    if (d128)
      hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)b.n_items), dim3(kBwdThreads), 0, stream, b);
    else
      hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3((unsigned)b.n_items), dim3(kBwdThreads), 0, stream, b);
    if ((r = launched())) return r;
  }
  return BA_OK;
}

int ulysses_launch(bool pack, const void* src, void* dst, int64_t batch, int64_t seqlen_local,
                     int32_t heads, int32_t head_dim, int32_t n_devices, hipStream_t stream) {
  if (batch < 0 || seqlen_local < 0 || heads < 0 || head_dim < 0 || n_devices < 1) return BA_ERR_SHAPE;
  if (heads % n_devices != 0 || head_dim % 8 != 0) return BA_ERR_SHAPE;
  const int64_t n_chunks = batch * seqlen_local * heads * (head_dim / 8);
  if (n_chunks == 0) return BA_OK;
  if (!src || !dst) return BA_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return BA_ERR_ALIGN;
  UlyssesArgs a;
  a.src = (const u32x4*)src;
  a.dst = (u32x4*)dst;
  a.B = batch;
  a.Sl = seqlen_local;
  a.H = heads;
  a.CPD = head_dim / 8;
  a.N = n_devices;
  a.n_chunks = n_chunks;
  const int64_t blocks = (n_chunks + 255) / 256;
  if (blocks > 0x7fffffffLL) return BA_ERR_SHAPE;
  if (pack)
    hipLaunchKernelGGL(ulysses_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(ulysses_unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return launched();
}

int gemm_launch(int epi, const void* a, const void* b, const void* b3, void* c, int64_t m, int32_t k,
                int32_t n_out, hipStream_t stream) {
  GemmArgs g;
  g.a = (const bf16*)a;
  g.b = (const bf16*)b;
  g.b3 = (const bf16*)b3;
  g.c = (bf16*)c;
  g.M = m;
  g.K = k;
  g.n_out = n_out;
  g.tiles_m = (int32_t)((m + kGemmBM - 1) / kGemmBM);
  g.tiles_n = n_out / (epi == EPI_SWIGLU ? 128 : 256);
  g.n_items = (int64_t)g.tiles_m * g.tiles_n;
  if (g.n_items > 0x7fffffffLL) return BA_ERR_SHAPE;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(gemm_nt_kernel<EPI_SWIGLU>, dim3((unsigned)g.n_items), dim3(kGemmThreads), 0, stream, g);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<EPI_STORE>, dim3((unsigned)g.n_items), dim3(kGemmThreads), 0, stream, g);
  return launched();
}

}  // namespace

// Entry for the allocation-free variant (noalloc.hip), which brings its own delta buffer.
__attribute__((visibility("hidden"))) int ba_bwd_impl(const ba_desc* d, const void* q, const void* k,
                                                      const void* v, const void* o, const void* dout,
                                                      const float* lse, float* delta, float* dq_acc, void* dk,
                                                      void* dv, int32_t dkv_dtype, void* dq_final, int32_t flags,
                                                      hipStream_t stream) {
  return bwd_impl(d, nullptr, q, k, v, o, dout, lse, delta, dq_acc, dk, dv, dkv_dtype, dq_final, flags, stream);
}

extern "C" {

int blockattn_fwd(const ba_desc* desc, const void* q, const void* k, const void* v, void* o,
                  int32_t o_dtype, float* lse, int32_t mode, void* o_final, hipStream_t stream) {
  return fwd_impl(desc, nullptr, q, k, v, o, o_dtype, lse, mode, o_final, stream);
}

int s2attn_fwd(const ba_desc* desc, const ba_s2_desc* s2, const void* q, const void* k,
               const void* v, void* o, int32_t o_dtype, float* lse, hipStream_t stream) {
  if (!desc) return BA_ERR_NULL;
  if (!s2) return BA_ERR_NULL;
  return fwd_impl(desc, s2, q, k, v, o, o_dtype, lse, BA_OVERWRITE, nullptr, stream);
}

int lse_merge(const ba_desc* d, float* o_acc, float* lse_acc, const void* o_part,
              int32_t part_dtype, const float* lse_part, void* o_final, hipStream_t stream) {
  int r = check_desc(d);
  if (r) return r;
  if (part_dtype != BA_F32 && part_dtype != BA_BF16) return BA_ERR_UNSUPPORTED;
  if (d->batch == 0 || d->seqlen_q == 0) return BA_OK;
  if (!o_acc || !lse_acc || !o_part || !lse_part) return BA_ERR_NULL;
  if (!aligned(o_acc, 16) || !aligned(o_part, 16) || !aligned(o_final, 16) ||
      !aligned(lse_acc, 4) || !aligned(lse_part, 4))
    return BA_ERR_ALIGN;
  MergeArgs a;
  a.o_acc = o_acc; a.lse_acc = lse_acc; a.o_part = o_part; a.lse_part = lse_part;
  a.o_final = (bf16*)o_final;
  a.s_b = d->o_stride[0]; a.s_s = d->o_stride[1]; a.s_h = d->o_stride[2];
  a.Sq = d->seqlen_q; a.Hq = d->heads_q; a.D = d->head_dim; a.part_f32 = part_dtype == BA_F32;
  a.n_threads = (int64_t)d->batch * d->seqlen_q * d->heads_q * (d->head_dim / 8);
  const int64_t blocks = ceil_div(a.n_threads, 256);
  if (blocks > 0x7fffffffLL) return BA_ERR_SHAPE;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return launched();
}

int blockattn_bwd(const ba_desc* desc, const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, float* delta, float* dq_acc, void* dk,
                  void* dv, int32_t dkv_dtype, void* dq_final, int32_t flags, hipStream_t stream) {
  if (!desc) return BA_ERR_NULL;
  return bwd_impl(desc, nullptr, q, k, v, o, dout, lse, delta, dq_acc, dk, dv, dkv_dtype, dq_final,
                  flags, stream);
}

int s2attn_bwd(const ba_desc* desc, const ba_s2_desc* s2, const void* q, const void* k,
               const void* v, const void* o, const void* dout, const float* lse, float* delta,
               float* dq_acc, void* dk, void* dv, int32_t dkv_dtype, void* dq_final, int32_t flags,
               hipStream_t stream) {
  if (!desc || !s2) return BA_ERR_NULL;
  return bwd_impl(desc, s2, q, k, v, o, dout, lse, delta, dq_acc, dk, dv, dkv_dtype, dq_final,
                  flags, stream);
}

int ulysses_pack(const void* x, void* send, int64_t batch, int64_t seqlen_local, int32_t heads,
                 int32_t head_dim, int32_t n_devices, hipStream_t stream) {
  return ulysses_launch(true, x, send, batch, seqlen_local, heads, head_dim, n_devices, stream);
}

int ulysses_unpack(const void* recv, void* x, int64_t batch, int64_t seqlen_local, int32_t heads,
                   int32_t head_dim, int32_t n_devices, hipStream_t stream) {
  return ulysses_launch(false, recv, x, batch, seqlen_local, heads, head_dim, n_devices, stream);
}

int bpt_ffn(const void* x, const void* w1, const void* w3, const void* w2, void* out, void* hidden,
            int64_t rows, int32_t d_model, int32_t d_ff, int64_t block_rows, hipStream_t stream) {
  if (rows < 0 || d_model < 0 || d_ff < 0 || block_rows < 1) return BA_ERR_SHAPE;
  if (d_model % 256 != 0 || d_ff % 128 != 0) return BA_ERR_SHAPE;
  if (rows == 0 || d_model == 0 || d_ff == 0) return BA_OK;
  if (!x || !w1 || !w3 || !w2 || !out || !hidden) return BA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w3, 16) || !aligned(w2, 16) || !aligned(out, 16) ||
      !aligned(hidden, 16))
    return BA_ERR_ALIGN;
  // the kernels address operands with 32-bit element offsets
  const int64_t bm = std::min(block_rows, rows);
  const int64_t lim = (int64_t)1 << 31;
  if (rows * (int64_t)d_model >= lim || bm * (int64_t)d_ff >= lim || (int64_t)d_ff * d_model >= lim)
    return BA_ERR_SHAPE;
  for (int64_t r0 = 0; r0 < rows; r0 += block_rows) {
    const int64_t m = std::min(block_rows, rows - r0);
    int r = gemm_launch(EPI_SWIGLU, (const bf16*)x + r0 * d_model, w1, w3, hidden, m, d_model, d_ff, stream);
    if (r) return r;
    r = gemm_launch(EPI_STORE, hidden, w2, nullptr, (bf16*)out + r0 * d_model, m, d_ff, d_model, stream);
    if (r) return r;
  }
  return BA_OK;
}

const char* blockattn_status_string(int status) {
  switch (status) {
    case BA_OK: return "BA_OK";
    case BA_ERR_NULL: return "BA_ERR_NULL: a required pointer is NULL";
    case BA_ERR_SHAPE: return "BA_ERR_SHAPE: invalid sizes";
    case BA_ERR_STRIDE: return "BA_ERR_STRIDE: strides must be non-negative multiples of 8 elements";
    case BA_ERR_ALIGN: return "BA_ERR_ALIGN: tensors must be 16-byte aligned (lse/delta 4-byte)";
    case BA_ERR_UNSUPPORTED: return "BA_ERR_UNSUPPORTED: head_dim must be 64 or 128; dtype must be F32 or BF16";
    case BA_ERR_S2: return "BA_ERR_S2: invalid S2 layout";
    case BA_ERR_MODE: return "BA_ERR_MODE: invalid mode/flags (ACCUMULATE needs an fp32 o)";
    case BA_ERR_LAUNCH: return "BA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case BA_ERR_WORKSPACE:
      return "BA_ERR_WORKSPACE: the problem needs more than the library's static scratch buffer holds, "
             "or its address could not be obtained";
    default: return "unknown blockattn status";
  }
}

int64_t blockattn_debug_fwd_schedule(const ba_desc* desc, const ba_s2_desc* s2, int32_t head,
                                     int64_t* out, int64_t cap) {
  int r = check_desc(desc);
  if (r) return -r;
  if (s2 && (r = check_s2(desc, s2))) return -r;
  if (head < 0 || head >= desc->heads_q) return -BA_ERR_SHAPE;
  const Sched s = sched_of(desc, s2, head);
  const int64_t nq = num_qtiles(s);
  int64_t n = 0;
  for (int64_t w = 0; w < nq; ++w) {
    const QTile t = make_qtile(s, qtile_of_rank(s, nq, w));
    for (int64_t kt = t.kt_begin; kt < t.kt_end; ++kt) {
      const KTile kt_ = make_ktile(s, kt);
      if (out && n < cap) {
        out[4 * n + 0] = t.row0; out[4 * n + 1] = t.rows;
        out[4 * n + 2] = kt_.row0; out[4 * n + 3] = kt_.rows;
      }
      ++n;
    }
  }
  return n;
}

int blockattn_debug_tile_sizes(int32_t head_dim, int32_t* block_q, int32_t* block_k) {
  if (head_dim != 64 && head_dim != 128) return BA_ERR_UNSUPPORTED;
  if (!block_q || !block_k) return BA_ERR_NULL;
  *block_q = kFwdBM;
  *block_k = kFwdBN;
  return BA_OK;
}

}  // extern "C"
