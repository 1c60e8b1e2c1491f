// Device helpers shared by the gfx950 kernels of libmoss.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moss.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MOSS_LDS __attribute__((address_space(3)))

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// Eight bf16 in a uint4 <-> eight fp32.
__device__ __forceinline__ void unpack8(const u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}
__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return w;
}

// In the 32x32 MFMA result layout, lanes l and l ^ 32 hold columns 8q + 4hh
// + (0..3) of one row, packed as bf16 (`lo` for q = 2p, `hi` for q = 2p + 1).
// Trading halves across the two lanes (v_permlane32_swap) leaves lane hh
// with columns 8(2p + hh) + (0..7): one 16-byte store per lane instead of two
// 8-byte ones.
__device__ __forceinline__ u32x4 pair_cols(u32x2 lo, u32x2 hi) {
  u32x4 r;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const auto s = __builtin_amdgcn_permlane32_swap(lo[d], hi[d], false, false);
    r[d] = s[0];
    r[2 + d] = s[1];
  }
  return r;
}

// SiLU in fp32, z / (1 + e^-z), from the hardware base-2 exponential and
// reciprocal (v_exp_f32, v_rcp_f32, about 1 ulp each): five instructions in
// place of a range-reduced expf and an IEEE division (the up projection's
// epilogue evaluates 64 of them per lane per tile; 585 -> 572 us).  For z
// below about -87 the result is a denormal or zero rather than z e^z.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// Sum over the 64 lanes of a wavefront (every lane gets the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Sum over aligned groups of `G` lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// One 16-byte-per-lane load from global memory straight into LDS: lane l's
// bytes land at LDS address lds + 16 l (lds wave-uniform, set through M0).
// Issued from asm, the compiler's wait-count tracking does not see it, so
// its waits on LDS fragment reads stay exact (while a direct load it knows
// of is pending, it waits for every outstanding LDS operation).  Callers
// wait for these loads themselves (s_waitcnt vmcnt) before the barrier that
// publishes the data.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory");
}

// A raw buffer resource (V#) over `bytes` bytes from `base`: no stride, 32-bit data format
// (the raw-buffer setting on gfx9-family parts).  Buffer loads past `bytes` return zero.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

// As dma16, through a buffer load: 16 bytes per lane into LDS at lds + 16 lane
// (buffer_load_dwordx4 ... lds) from byte offset voff + soff of the buffer rsrc, the offset split
// into a per-lane part (voff) and a wave-uniform part (soff, the instruction's scalar offset: no
// per-lane add).  The resource's bounds check covers voff only, so the caller keeps voff + soff in
// bounds itself.
__device__ __forceinline__ void dma16_buf_so(uint32_t voff, u32x4 rsrc, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(rsrc),
               "s"(soff)
               : "memory");
}

// Per-launch batch metadata passed by value (txt_len lives on the host).
struct ItemLens {
  int32_t len[MOSS_MAX_BATCH];
};

// Per-item timesteps, passed to a kernel by value.
struct ItemTimes {
  float t[MOSS_MAX_BATCH];
};
