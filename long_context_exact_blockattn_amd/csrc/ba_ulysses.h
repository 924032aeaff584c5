// Layout permutes around the all-to-all of DeepSpeed Ulysses sequence
// parallelism, one device's share.  Ulysses is one of the sequence-parallel
// methods the long-context recipe supports beside Ring Attention (project page
// "How It Works"); it swaps a sequence sharding for a head sharding around
// attention.
//
// With the sequence split over N devices, device r holds x = [B, Sl, H, D]
// (Sl = S / N).  An all-to-all gives every device all S rows of H / N heads:
//   pack:    send[n][b][s][j][d] = x[b][s][n * (H/N) + j][d]   (n = destination)
//   unpack:  x[b][s][n * (H/N) + j][d] = recv[n][b][s][j][d]   (n = source)
// Pure copies of bf16 elements, HBM-bound (2 bytes read and 2 written per
// element).  One thread moves one 16-byte chunk (8 elements of D); a (b, s, n)
// group is a contiguous run of (H/N) * D elements on both sides, so reads and
// writes are coalesced.
#pragma once

#include "ba_common.h"

namespace ba {

struct UlyssesArgs {
  const u32x4* src;
  u32x4* dst;
  int64_t B, Sl;
  int32_t H, CPD, N;  // CPD = D / 8 chunks per head row
  int64_t n_chunks;
};

// pack: thread t = destination chunk (n, b, s, j, c)
__global__ __launch_bounds__(256) void ulysses_pack_kernel(UlyssesArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.n_chunks) return;
  const int hn = a.H / a.N;
  const int64_t run = (int64_t)hn * a.CPD;       // chunks per (n, b, s)
  const int64_t within = t % run;                // j * CPD + c
  const int64_t nbs = t / run;                   // (n * B + b) * Sl + s
  const int64_t bs = nbs % (a.B * a.Sl);         // b * Sl + s
  const int64_t n = nbs / (a.B * a.Sl);
  const int64_t src = bs * ((int64_t)a.H * a.CPD) + n * run + within;
  a.dst[t] = a.src[src];
#endif
}

// unpack: thread t = destination chunk (b, s, h, c) of x
__global__ __launch_bounds__(256) void ulysses_unpack_kernel(UlyssesArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.n_chunks) return;
  const int hn = a.H / a.N;
  const int64_t run = (int64_t)hn * a.CPD;
  const int64_t row = (int64_t)a.H * a.CPD;      // chunks per (b, s)
  const int64_t bs = t / row;
  const int64_t hc = t % row;                    // h * CPD + c
  const int64_t n = hc / run;
  const int64_t within = hc % run;
  const int64_t src = (n * (a.B * a.Sl) + bs) * run + within;
  a.dst[t] = a.src[src];
#endif
}

}  // namespace ba
