// A caller of the C ABI with no Python and no PyTorch: device buffers from
// hipMalloc, inputs from a fixed integer generator, one stream.
//
// Checks, on one GPU:
//  1. the validation contract: bad arguments return their status and enqueue
//     nothing (the output buffer is untouched);
//  2. a 4-chunk ring in a shuffled order (OVERWRITE then ACCUMULATE, final bf16
//     store on the last step) equals one call over all keys within the parity
//     tolerances (the two round P to bf16 against different running maxima and
//     merge in fp32), and the bf16 output is the rounding of the fp32 one -- the
//     order independence of the blockwise method (Ring Attention summary,
//     Summary);
//  3. the backward over the same ring (delta on the first step, dQ accumulated
//     in fp32 and converted on the last, dK and dV written per chunk) equals one
//     backward call over all keys within a relative L2 of 1e-2 per gradient;
//  4. the same backward ring through blockattn_bwd_noalloc (delta in the
//     library's static buffer, recomputed on every call) gives the same bits.
// Prints one line "abi_example ok ..." and exits 0, or prints the failure and
// exits 1.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/blockattn.h"

namespace {

#define HIP_OK(x)                                                                   \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      fprintf(stderr, "abi_example: %s failed: %s\n", #x, hipGetErrorString(e_));   \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

// bf16 by round to nearest even from the fp32 bit pattern (finite inputs)
uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// values in [-2, 2) from a 64-bit linear congruential sequence (Knuth's MMIX constants)
struct Lcg {
  uint64_t s;
  float next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((s >> 40) & 0xffffff) / (float)(1 << 22) - 2.0f;
  }
};

int fail(const char* what) {
  fprintf(stderr, "abi_example FAILED: %s\n", what);
  return 1;
}

}  // namespace

int main() {
  const int B = 1, H = 2, D = 128;
  const int64_t S = 1000, n_chunks = 4, C = S / n_chunks;
  const int64_t n = (int64_t)B * S * H * D, n_rows = (int64_t)B * H * S;

  std::vector<uint16_t> hq(n), hk(n), hv(n);
  Lcg g{12345};
  for (int64_t i = 0; i < n; ++i) hq[i] = to_bf16(g.next());
  for (int64_t i = 0; i < n; ++i) hk[i] = to_bf16(g.next());
  for (int64_t i = 0; i < n; ++i) hv[i] = to_bf16(g.next());

  void *q, *k, *v, *o_ring, *o_one, *o_bf16;
  float *lse_ring, *lse_one;
  HIP_OK(hipMalloc(&q, n * 2));
  HIP_OK(hipMalloc(&k, n * 2));
  HIP_OK(hipMalloc(&v, n * 2));
  HIP_OK(hipMalloc(&o_ring, n * 4));
  HIP_OK(hipMalloc(&o_one, n * 4));
  HIP_OK(hipMalloc(&o_bf16, n * 2));
  HIP_OK(hipMalloc((void**)&lse_ring, n_rows * 4));
  HIP_OK(hipMalloc((void**)&lse_one, n_rows * 4));
  HIP_OK(hipMemcpy(q, hq.data(), n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk.data(), n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv.data(), n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(o_one, 0, n * 4));
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));

  ba_desc d;
  memset(&d, 0, sizeof d);
  d.batch = B;
  d.heads_q = H;
  d.heads_kv = H;
  d.head_dim = D;
  d.seqlen_q = S;
  d.seqlen_k = S;
  d.causal = 1;
  d.scale = 0.f;
  const int64_t strides[3] = {S * H * D, H * D, D};
  memcpy(d.q_stride, strides, sizeof strides);
  memcpy(d.kv_stride, strides, sizeof strides);
  memcpy(d.o_stride, strides, sizeof strides);

  // ---- 1. validation: nothing is enqueued on an error
  {
    ba_desc bad = d;
    bad.head_dim = 96;
    if (blockattn_fwd(&bad, q, k, v, o_one, BA_F32, lse_one, BA_OVERWRITE, nullptr, st) != BA_ERR_UNSUPPORTED)
      return fail("head_dim 96 not rejected");
    if (blockattn_fwd(&d, nullptr, k, v, o_one, BA_F32, lse_one, BA_OVERWRITE, nullptr, st) != BA_ERR_NULL)
      return fail("NULL q not rejected");
    if (blockattn_fwd(&d, (char*)q + 2, k, v, o_one, BA_F32, lse_one, BA_OVERWRITE, nullptr, st) != BA_ERR_ALIGN)
      return fail("misaligned q not rejected");
    if (blockattn_fwd(&d, q, k, v, o_one, BA_BF16, lse_one, BA_ACCUMULATE, nullptr, st) != BA_ERR_MODE)
      return fail("ACCUMULATE into bf16 not rejected");
    bad = d;
    bad.q_stride[1] = H * D + 4;
    if (blockattn_fwd(&bad, q, k, v, o_one, BA_F32, lse_one, BA_OVERWRITE, nullptr, st) != BA_ERR_STRIDE)
      return fail("stride not a multiple of 8 not rejected");
    bad = d;
    bad.o_stride[2] = -D;
    if (blockattn_fwd(&bad, q, k, v, o_one, BA_F32, lse_one, BA_OVERWRITE, nullptr, st) != BA_ERR_STRIDE)
      return fail("negative output stride not rejected");
    HIP_OK(hipStreamSynchronize(st));
    std::vector<float> zero(n);
    HIP_OK(hipMemcpy(zero.data(), o_one, n * 4, hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < n; ++i)
      if (zero[i] != 0.f) return fail("a rejected call wrote its output");
  }

  // ---- 2. one call over all keys, then the ring in a shuffled chunk order
  if (blockattn_fwd(&d, q, k, v, o_one, BA_F32, lse_one, BA_OVERWRITE, nullptr, st) != BA_OK)
    return fail("one-shot forward");
  const int order[4] = {2, 0, 3, 1};
  for (int t = 0; t < n_chunks; ++t) {
    ba_desc dc = d;
    dc.seqlen_k = C;
    dc.k_pos0 = order[t] * C;
    const char* kc = (const char*)k + dc.k_pos0 * strides[1] * 2;
    const char* vc = (const char*)v + dc.k_pos0 * strides[1] * 2;
    const int st_ = blockattn_fwd(&dc, q, kc, vc, o_ring, BA_F32, lse_ring, t == 0 ? BA_OVERWRITE : BA_ACCUMULATE,
                                  t == n_chunks - 1 ? o_bf16 : nullptr, st);
    if (st_ != BA_OK) {
      fprintf(stderr, "ring step %d: %s\n", t, blockattn_status_string(st_));
      return 1;
    }
  }
  HIP_OK(hipStreamSynchronize(st));

  std::vector<float> a(n), b(n), la(n_rows), lb(n_rows);
  std::vector<uint16_t> ob(n);
  HIP_OK(hipMemcpy(a.data(), o_ring, n * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(b.data(), o_one, n * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(ob.data(), o_bf16, n * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(la.data(), lse_ring, n_rows * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lb.data(), lse_one, n_rows * 4, hipMemcpyDeviceToHost));
  double max_o = 0, max_l = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (!isfinite(a[i]) || !isfinite(b[i])) return fail("non-finite output");
    max_o = fmax(max_o, fabs((double)a[i] - b[i]));
    if (ob[i] != to_bf16(a[i])) return fail("bf16 output is not the rounding of the fp32 one");
  }
  for (int64_t i = 0; i < n_rows; ++i) max_l = fmax(max_l, fabs((double)la[i] - lb[i]));
  if (max_o > 1e-2 || max_l > 1e-3) {
    fprintf(stderr, "ring vs one call: max|dO| %.3e max|dLSE| %.3e\n", max_o, max_l);
    return fail("ring result differs from the one-call result");
  }

  // ---- 3. backward: the ring of chunks against one call over all keys
  std::vector<uint16_t> hdo(n);
  for (int64_t i = 0; i < n; ++i) hdo[i] = to_bf16(g.next());
  void *dout, *dq1, *dk1, *dv1, *dq2, *dk2, *dv2;
  float *delta, *dqa1, *dqa2;
  HIP_OK(hipMalloc(&dout, n * 2));
  HIP_OK(hipMalloc(&dq1, n * 2));
  HIP_OK(hipMalloc(&dk1, n * 2));
  HIP_OK(hipMalloc(&dv1, n * 2));
  HIP_OK(hipMalloc(&dq2, n * 2));
  HIP_OK(hipMalloc(&dk2, n * 2));
  HIP_OK(hipMalloc(&dv2, n * 2));
  HIP_OK(hipMalloc((void**)&delta, n_rows * 4));
  HIP_OK(hipMalloc((void**)&dqa1, n * 4));
  HIP_OK(hipMalloc((void**)&dqa2, n * 4));
  HIP_OK(hipMemcpy(dout, hdo.data(), n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(dqa1, 0, n * 4));
  HIP_OK(hipMemset(dqa2, 0, n * 4));
  if (blockattn_bwd(&d, q, k, v, o_bf16, dout, lse_ring, delta, dqa1, dk1, dv1, BA_BF16, dq1,
                    BA_BWD_COMPUTE_DELTA | BA_BWD_FINALIZE_DQ, st) != BA_OK)
    return fail("one-shot backward");
  for (int t = 0; t < n_chunks; ++t) {
    ba_desc dc = d;
    dc.seqlen_k = C;
    dc.k_pos0 = order[t] * C;
    const int64_t koff = dc.k_pos0 * strides[1] * 2;
    const int flags = (t == 0 ? BA_BWD_COMPUTE_DELTA : 0) | (t == n_chunks - 1 ? BA_BWD_FINALIZE_DQ : 0);
    const int st_ = blockattn_bwd(&dc, q, (const char*)k + koff, (const char*)v + koff, o_bf16, dout, lse_ring,
                                  delta, dqa2, (char*)dk2 + koff, (char*)dv2 + koff, BA_BF16, dq2, flags, st);
    if (st_ != BA_OK) {
      fprintf(stderr, "backward ring step %d: %s\n", t, blockattn_status_string(st_));
      return 1;
    }
  }
  HIP_OK(hipStreamSynchronize(st));
  double rel[3];
  void* const pairs[3][2] = {{dq1, dq2}, {dk1, dk2}, {dv1, dv2}};
  std::vector<uint16_t> ga(n), gb(n);
  for (int j = 0; j < 3; ++j) {
    HIP_OK(hipMemcpy(ga.data(), pairs[j][0], n * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gb.data(), pairs[j][1], n * 2, hipMemcpyDeviceToHost));
    double num = 0, den = 0;
    for (int64_t i = 0; i < n; ++i) {
      const double x = from_bf16(ga[i]), y = from_bf16(gb[i]);
      if (!isfinite(x) || !isfinite(y)) return fail("non-finite gradient");
      num += (x - y) * (x - y);
      den += x * x;
    }
    rel[j] = sqrt(num / (den > 0 ? den : 1.0));
  }
  if (rel[0] > 1e-2 || rel[1] > 1e-2 || rel[2] > 1e-2) {
    fprintf(stderr, "backward ring vs one call: rel L2 dq %.3e dk %.3e dv %.3e\n", rel[0], rel[1], rel[2]);
    return fail("ring backward differs from the one-call backward");
  }
  // ---- 4. the allocation-free entry point over the same ring: the same bits
  void *dq3, *dk3, *dv3;
  float* dqa3;
  HIP_OK(hipMalloc(&dq3, n * 2));
  HIP_OK(hipMalloc(&dk3, n * 2));
  HIP_OK(hipMalloc(&dv3, n * 2));
  HIP_OK(hipMalloc((void**)&dqa3, n * 4));
  HIP_OK(hipMemset(dqa3, 0, n * 4));
  for (int t = 0; t < n_chunks; ++t) {
    ba_desc dc = d;
    dc.seqlen_k = C;
    dc.k_pos0 = order[t] * C;
    const int64_t koff = dc.k_pos0 * strides[1] * 2;
    const int flags = t == n_chunks - 1 ? BA_BWD_FINALIZE_DQ : 0;
    const int st_ = blockattn_bwd_noalloc(&dc, q, (const char*)k + koff, (const char*)v + koff, o_bf16, dout,
                                          lse_ring, dqa3, (char*)dk3 + koff, (char*)dv3 + koff, BA_BF16, dq3,
                                          flags, st);
    if (st_ != BA_OK) {
      fprintf(stderr, "allocation-free backward ring step %d: %s\n", t, blockattn_status_string(st_));
      return 1;
    }
  }
  HIP_OK(hipStreamSynchronize(st));
  void* const same[3][2] = {{dq2, dq3}, {dk2, dk3}, {dv2, dv3}};
  for (int j = 0; j < 3; ++j) {
    HIP_OK(hipMemcpy(ga.data(), same[j][0], n * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gb.data(), same[j][1], n * 2, hipMemcpyDeviceToHost));
    if (memcmp(ga.data(), gb.data(), n * 2) != 0) return fail("the allocation-free backward differs from the ring");
  }
  hipFree(dq3); hipFree(dk3); hipFree(dv3); hipFree(dqa3);

  printf("abi_example ok: ring of %d chunks vs one call over S=%lld keys: max|dO| %.3e, max|dLSE| %.3e; "
         "backward rel L2 dq %.3e dk %.3e dv %.3e; allocation-free backward bit-identical; first output %.6f\n",
         (int)n_chunks, (long long)S, max_o, max_l, rel[0], rel[1], rel[2], from_bf16(ob[0]));
  hipFree(q); hipFree(k); hipFree(v); hipFree(o_ring); hipFree(o_one); hipFree(o_bf16);
  hipFree(lse_ring); hipFree(lse_one);
  hipFree(dout); hipFree(dq1); hipFree(dk1); hipFree(dv1); hipFree(dq2); hipFree(dk2); hipFree(dv2);
  hipFree(delta); hipFree(dqa1); hipFree(dqa2);
  hipStreamDestroy(st);
  return 0;
}
