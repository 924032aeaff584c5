// Shared device types and small helpers for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define BA_HD __host__ __device__ __forceinline__

namespace ba {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

#if defined(__HIP_DEVICE_COMPILE__)

// v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] * B[16x32].
// Accumulator layout (measured on gfx950): lane l, register r holds
// C[8*(r/4) + 4*(l/32) + r%4][l%32].  The k index of an operand register is
// the same function of (l/32, item) for A and B, so any consistent k order of
// the two operands gives the product.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Hardware base-2 exponential / logarithm (v_exp_f32, v_log_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i receives
// item j = the (i%4)-th 16-bit value at the address supplied by lane (i/4)+4j.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ float wave_xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// max / sum of x over lanes l and l ^ 32 on the vector ALU: v_permlane32_swap
// exchanges one 32-lane half of its two operands, so with both operands = x the
// two results hold x of lane l and of lane l ^ 32 (in some order, which a
// symmetric reduction does not see).  No LDS round trip, unlike a shuffle.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over [base, base + bytes) (raw, stride 0; dword 3 = the gfx9
// data format used for untyped loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct buffer -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// the address is the resource base (scalar registers) plus a per-lane byte
// offset (plus a scalar offset), so a tile's loads need no per-lane address
// arithmetic; lane L of the wave writes lds_base + 16*L (lds_base the same for
// every lane), and a lane whose offset lies past the resource's size reads
// zeros.  Every tile load uses this form: with the FLAT form
// (global_load_lds) in flight the compiler can no longer count the wave's
// outstanding LDS reads and waits for all of them before each use.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds_base), 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(0): this wave's outstanding vector-memory loads (including
// direct-to-LDS ones) have landed.  expcnt and lgkmcnt are left unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
#endif

// ---- LDS tile layout shared by every kernel --------------------------------
// A tile is R rows x D bf16 with no padding; each row is D/8 chunks of 16
// bytes and chunk c of row r is stored in slot c ^ swz(r).  The swizzle makes
// both access patterns the kernels use conflict-free on the 64 LDS banks:
//  - 16-byte reads of one chunk from 16 consecutive rows (MFMA operands whose
//    contraction runs over D): swz is a bijection on r mod 16;
//  - transposing 8-byte reads of 4 consecutive rows (from a multiple of 4) x
//    4 aligned chunks (operands whose contraction runs over the rows): the
//    high chunk bits of swz differ across the 4 rows.
template <int D>
BA_HD int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  if (D == 32) return (r >> 2) & 3;  // 4 chunks, 16 banks per row: 16-byte reads only
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);  // D == 64: 8 chunks, 32 banks per row
}

// element offset of (row r, element e) inside a tile
template <int D>
BA_HD int tile_off(int r, int e) {
  return r * D + ((((e >> 3) ^ swz<D>(r)) << 3) | (e & 7));
}
}  // namespace ba
