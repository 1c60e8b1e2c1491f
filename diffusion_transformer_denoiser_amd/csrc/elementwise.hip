// Bandwidth-bound kernels of the block: row join, adaLN GEMV, modulated
// RMSNorm, gated residual add, SiLU-gated product, rotary tables.
//
// The MOSS-Image transformer page (TensorFold PR #1528, "What it adds") names
// the modulated RMSNorm, SiLU and gated-add kernels and the precision policy
// (bf16 storage, fp32 sums and norms).  Every kernel here moves 16 bytes per
// lane per access (eight bf16) so that a wavefront touches 1 KiB contiguous.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace {

constexpr int kThreads = 256;

// ---- a0: h0 = [txt; x] into the fp32 residual stream, pad text rows zero ----
__global__ __launch_bounds__(kThreads) void join_rows_kernel(const u32x4* __restrict__ x,
                                                             const u32x4* __restrict__ txt, ItemLens lens,
                                                             f32x4* __restrict__ out, int n_txt, int n_img,
                                                             int chunks_per_row, long total) {
  const int rows = n_txt + n_img;
  for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < total; i += (long)gridDim.x * kThreads) {
    const long row = i / chunks_per_row;
    const int c = (int)(i - row * chunks_per_row);
    const int b = (int)(row / rows);
    const int r = (int)(row - (long)b * rows);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < n_txt) {
      if (r < lens.len[b]) v = txt[((long)b * n_txt + r) * chunks_per_row + c];
    } else {
      v = x[((long)b * n_img + (r - n_txt)) * chunks_per_row + c];
    }
    float f[8];
    unpack8(v, f);
    out[2 * i] = f32x4{f[0], f[1], f[2], f[3]};
    out[2 * i + 1] = f32x4{f[4], f[5], f[6], f[7]};
  }
}

// ---- a1: s = SiLU(cond) in fp32, then mod = W_mod s -------------------------
constexpr int kGemvSet = 32;  // weight matrices one modulation launch takes
struct GemvSet {
  const uint16_t* w[kGemvSet];  // [6 d, d] bf16 each
  unsigned skip[kGemvSet];      // items whose gates that matrix's output zeroes
};

__global__ __launch_bounds__(kThreads) void silu_cond_kernel(const uint16_t* __restrict__ cond,
                                                             float* __restrict__ s, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) s[i] = silu_f32(bf16_to_f32(cond[i]));
}

// One wavefront per output row; every item of the batch shares the weight read.
// Lane l takes the 16-byte chunks l, l + 64, ... of the row (CPL of them at
// most) and issues all its weight loads before any arithmetic, so a
// wavefront has its whole row in flight at once (the row is read once).
// blockIdx.y picks one of up to kGemvSet weight matrices (the modulations of
// a whole block stack depend only on cond, so one launch computes them all
// and streams every block's W_mod back to back).
// s is read by every row: with kGemvRows wavefronts per workgroup, one copy of it goes into LDS
// (when it fits) rather than each wavefront reading its own from L2.
constexpr int kGemvRows = 8;                  // wavefronts (rows) per workgroup
constexpr int kGemvLdsFloats = 8192;          // s staged in LDS up to 32 KiB (batch * d floats)
template <int CPL>
__global__ __launch_bounds__(64 * kGemvRows) void adaln_gemv_kernel(const float* __restrict__ s, GemvSet set,
                                                                    float* __restrict__ mod, int batch, int n_out,
                                                                    int d) {
  __shared__ __attribute__((aligned(16))) float s_lds[kGemvLdsFloats];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kGemvRows + (threadIdx.x >> 6);
  const bool live = row < n_out;
  const uint16_t* __restrict__ w = set.w[blockIdx.y];
  const unsigned skip_items = set.skip[blockIdx.y];
  mod += (size_t)blockIdx.y * batch * n_out;
  const u32x4* wr = reinterpret_cast<const u32x4*>(w + (size_t)min(row, n_out - 1) * d);
  const int nch = d >> 3;
  u32x4 wv[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    wv[i] = c < nch ? wr[c] : u32x4{0u, 0u, 0u, 0u};
  }
  const bool staged = batch * d <= kGemvLdsFloats;
  if (staged) {
    // the weight loads are in flight; copy s meanwhile
    for (int k = threadIdx.x; k < batch * d / 4; k += 64 * kGemvRows)
      reinterpret_cast<f32x4*>(s_lds)[k] = reinterpret_cast<const f32x4*>(s)[k];
    __syncthreads();
  }
  const float* sv = staged ? s_lds : s;
  if (!live) return;
  float acc[MOSS_MAX_BATCH];
#pragma unroll
  for (int b = 0; b < MOSS_MAX_BATCH; ++b) acc[b] = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float f[8];
      unpack8(wv[i], f);
#pragma unroll
      for (int b = 0; b < MOSS_MAX_BATCH; ++b) {
        if (b < batch) {
          const f32x4* sp = reinterpret_cast<const f32x4*>(sv + (size_t)b * d + 8 * c);
          const f32x4 s0 = sp[0], s1 = sp[1];
          acc[b] += f[0] * s0[0] + f[1] * s0[1] + f[2] * s0[2] + f[3] * s0[3] + f[4] * s1[0] +
                    f[5] * s1[1] + f[6] * s1[2] + f[7] * s1[3];
        }
      }
    }
  }
  // chunks 2 and 5 are gate1 and gate2: a block skipped for an item gets zero gates there, so both
  // gated adds leave that item's residual exactly as it was
  const int chunk = row / d;
  const bool gate = chunk == 2 || chunk == 5;
#pragma unroll
  for (int b = 0; b < MOSS_MAX_BATCH; ++b) {
    if (b < batch) {
      const float t = wave_sum(acc[b]);
      if (lane == 0) mod[(size_t)b * n_out + row] = (gate && ((skip_items >> b) & 1u)) ? 0.0f : t;
    }
  }
}

// Row layout for the norms below: lane l's chunk i holds values 4 (l + 64 i) .. +3, so each
// load or store instruction of a wavefront covers one contiguous stretch of the row (1 KiB of
// fp32, 512 B of bf16).  The shift and scale of a chunk are loaded where they are used, which
// keeps the register count (and so the wavefronts in flight per SIMD) up.
// Lanes l and l ^ 1 trade one 8-byte half (DPP quad_perm [1, 0, 3, 2]).
__device__ __forceinline__ u32x2 swap_neighbour(u32x2 x) {
  return u32x2{(uint32_t)__builtin_amdgcn_mov_dpp((int)x[0], 0xB1, 0xF, 0xF, false),
               (uint32_t)__builtin_amdgcn_mov_dpp((int)x[1], 0xB1, 0xF, 0xF, false)};
}

template <int C4>
__device__ __forceinline__ void modulate_store(const f32x4 (&v)[C4], float ss, const float* __restrict__ sh,
                                                const float* __restrict__ sc, uint16_t* __restrict__ dst, int lane,
                                                int nch4, int d, float eps) {
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  auto mod4 = [&](const f32x4& x, int c) {
    const f32x4 shv = reinterpret_cast<const f32x4*>(sh)[c];
    const f32x4 scv = reinterpret_cast<const f32x4*>(sc)[c];
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (x[j] * r) * (1.0f + scv[j]) + shv[j];
    return u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
  };
  if (C4 % 2 == 0 && nch4 == 64 * C4) {
    // whole chunk pairs: for chunks i and i + 1, an even lane stores its own and its odd
    // neighbour's values of chunk i, the odd lane both lanes' values of chunk i + 1 (8
    // consecutive values, 16 bytes each): half the store instructions
    const bool odd = lane & 1;
#pragma unroll
    for (int i = 0; i < C4; i += 2) {
      const u32x2 p0 = mod4(v[i], lane + 64 * i), p1 = mod4(v[i + 1], lane + 64 * (i + 1));
      const u32x2 got = swap_neighbour(odd ? p0 : p1);
      const u32x4 o = odd ? u32x4{got[0], got[1], p1[0], p1[1]} : u32x4{p0[0], p0[1], got[0], got[1]};
      const int e = 4 * ((lane & ~1) + 64 * (odd ? i + 1 : i));
      *reinterpret_cast<u32x4*>(dst + e) = o;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < C4; ++i) {
    const int c = lane + 64 * i;
    if (c < nch4) {
      const f32x4 shv = reinterpret_cast<const f32x4*>(sh)[c];
      const f32x4 scv = reinterpret_cast<const f32x4*>(sc)[c];
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (v[i][j] * r) * (1.0f + scv[j]) + shv[j];
      reinterpret_cast<u32x2*>(dst)[c] = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
  }
}

template <int C4>
__global__ __launch_bounds__(kThreads) void mod_rmsnorm_kernel(const float* __restrict__ h,
                                                                const float* __restrict__ shift,
                                                                const float* __restrict__ scale, int mod_stride,
                                                                uint16_t* __restrict__ out, int total_rows,
                                                                int rows_per_item, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= total_rows) return;
  const int b = row / rows_per_item;
  const int nch4 = d >> 2;
  const f32x4* src = reinterpret_cast<const f32x4*>(h + (size_t)row * d);
  f32x4 v[C4];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < C4; ++i) {
    const int c = lane + 64 * i;
    if (c < nch4) {
      v[i] = src[c];
#pragma unroll
      for (int j = 0; j < 4; ++j) ss += v[i][j] * v[i][j];
    }
  }
  modulate_store<C4>(v, ss, shift + (size_t)b * mod_stride, scale + (size_t)b * mod_stride, out + (size_t)row * d,
                      lane, nch4, d, eps);
}

template <int C4>
__global__ __launch_bounds__(kThreads) void join_mod_rmsnorm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ txt, ItemLens lens, const float* __restrict__ shift,
    const float* __restrict__ scale, int mod_stride, float* __restrict__ h, uint16_t* __restrict__ out,
    int n_txt, int n_img, int d, float eps, int total_rows) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= total_rows) return;
  const int rows = n_txt + n_img;
  const int b = row / rows, r = row - b * rows;
  const int nch4 = d >> 2;
  const u32x2* src = nullptr;
  if (r >= n_txt) src = reinterpret_cast<const u32x2*>(x + ((size_t)b * n_img + (r - n_txt)) * d);
  else if (r < lens.len[b]) src = reinterpret_cast<const u32x2*>(txt + ((size_t)b * n_txt + r) * d);
  f32x4 v[C4];
  float ss = 0.0f;
  f32x4* hrow = reinterpret_cast<f32x4*>(h + (size_t)row * d);
  auto widen = [](u32x2 w) { return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])}; };
  if (C4 % 2 == 0 && nch4 == 64 * C4) {
    // whole chunk pairs, loaded 16 bytes per lane as modulate_store stores them: an even lane
    // reads chunk i of itself and its odd neighbour, the odd lane chunk i + 1 of both, and the
    // two trade the halves that belong to the other
    const bool odd = lane & 1;
    const u32x4* src4 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
    for (int i = 0; i < C4; i += 2) {
      const u32x4 q = src ? src4[((lane & ~1) + 64 * (odd ? i + 1 : i)) >> 1] : u32x4{0u, 0u, 0u, 0u};
      const u32x2 lo = {q[0], q[1]}, hi = {q[2], q[3]};
      const u32x2 got = swap_neighbour(odd ? lo : hi);
      v[i] = widen(odd ? got : lo);
      v[i + 1] = widen(odd ? hi : got);
    }
#pragma unroll
    for (int i = 0; i < C4; ++i) {
      hrow[lane + 64 * i] = v[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) ss += v[i][j] * v[i][j];
    }
  } else {
#pragma unroll
    for (int i = 0; i < C4; ++i) {
      const int c = lane + 64 * i;
      if (c < nch4) {
        const u32x2 w = src ? src[c] : u32x2{0u, 0u};
        v[i] = widen(w);
        hrow[c] = v[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) ss += v[i][j] * v[i][j];
      }
    }
  }
  modulate_store<C4>(v, ss, shift + (size_t)b * mod_stride, scale + (size_t)b * mod_stride, out + (size_t)row * d,
                      lane, nch4, d, eps);
}


// ---- a7/a12: h + gate * y on the fp32 residual ------------------------------------
// In place (out16 == nullptr), or, for the last add of a call, into the bf16
// output instead.
__global__ __launch_bounds__(kThreads) void gated_add_kernel(f32x4* __restrict__ h, const float* __restrict__ gate,
                                                             int gate_stride, const u32x4* __restrict__ y,
                                                             u32x4* __restrict__ out16, int chunks_per_row,
                                                             int rows_per_item, long total) {
  for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < total; i += (long)gridDim.x * kThreads) {
    const long row = i / chunks_per_row;
    const int c = (int)(i - row * chunks_per_row);
    const int b = (int)(row / rows_per_item);
    const f32x4* g = reinterpret_cast<const f32x4*>(gate + (size_t)b * gate_stride + 8 * c);
    const f32x4 g0 = g[0], g1 = g[1];
    const f32x4 h0 = h[2 * i], h1 = h[2 * i + 1];
    float yv[8];
    unpack8(y[i], yv);
    f32x4 o0, o1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o0[j] = h0[j] + g0[j] * yv[j];
      o1[j] = h1[j] + g1[j] * yv[4 + j];
    }
    if (out16) {
      const float o[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
      out16[i] = pack8(o);
    } else {
      h[2 * i] = o0;
      h[2 * i + 1] = o1;
    }
  }
}

// ---- a0 + a2 for a call's first block: join the rows into the fp32 residual
// and apply the first modulated RMSNorm, one wavefront per row, so h is
// written once and not read back.  Text pad rows (r >= txt_len) are zero rows.

// ---- a10: z = SiLU(u_gate) * u_up -------------------------------------------
__global__ __launch_bounds__(kThreads) void silu_mul_kernel(const uint16_t* __restrict__ u, u32x4* __restrict__ z,
                                                            int f, long total) {
  const int cpr = f >> 3;
  for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < total; i += (long)gridDim.x * kThreads) {
    const long row = i / cpr;
    const int c = (int)(i - row * cpr);
    const u32x4* ur = reinterpret_cast<const u32x4*>(u + (size_t)row * 2 * f);
    float g[8], up[8], o[8];
    unpack8(ur[c], g);
    unpack8(ur[cpr + c], up);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = silu_f32(g[j]) * up[j];
    z[i] = pack8(o);
  }
}

// ---- the sampler step: classifier-free guidance, then one Euler step ----------------
// x_out = x_in + dsigma * (v_neg + g * (v_pos - v_neg)); without v_neg (guidance 1)
// x_out = x_in + dsigma * v_pos.  Eight elements per thread: one 16-byte load of
// each velocity, two of x.
__global__ __launch_bounds__(kThreads) void guidance_euler_kernel(const u32x4* __restrict__ v_pos,
                                                                  const u32x4* __restrict__ v_neg, float g,
                                                                  float dsigma, const f32x4* x_in, f32x4* x_out,
                                                                  long total) {
  for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < total; i += (long)gridDim.x * kThreads) {
    float p[8], v[8];
    unpack8(v_pos[i], p);
    if (v_neg) {
      float q[8];
      unpack8(v_neg[i], q);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = q[j] + g * (p[j] - q[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p[j];
    }
    const f32x4 x0 = x_in[2 * i], x1 = x_in[2 * i + 1];
    f32x4 y0, y1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y0[j] = x0[j] + dsigma * v[j];
      y1[j] = x1[j] + dsigma * v[4 + j];
    }
    x_out[2 * i] = y0;
    x_out[2 * i + 1] = y1;
  }
}

// ---- the denoiser's ends ------------------------------------------------------
// 256 timestep features per item: cos(t w_i) for i < 128, then sin(t w_i),
// w_i = 10000^(-i/128), with the angle and its cos/sin in fp64, stored fp32.
__global__ __launch_bounds__(kThreads) void timestep_features_kernel(ItemTimes ts, float* __restrict__ f,
                                                                     int batch) {
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= batch * 256) return;
  const int b = idx >> 8, i = idx & 255, j = i & 127;
  const double ang = (double)ts.t[b] * exp(-(double)j / 128.0 * log(10000.0));
  f[idx] = (float)(i < 128 ? cos(ang) : sin(ang));
}

// y = SiLU(x) in fp32 (in place allowed).
__global__ __launch_bounds__(kThreads) void silu_f32_kernel(const float* x, float* y, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) y[i] = silu_f32(x[i]);
}

// bf16 (round to nearest even) of fp32 values.
__global__ __launch_bounds__(kThreads) void round_bf16_kernel(const float* __restrict__ x, uint16_t* __restrict__ y,
                                                              int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) y[i] = __builtin_bit_cast(uint16_t, (__bf16)x[i]);
}

// ---- rotary tables ------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void rope_build_kernel(int n_txt, int grid_w, double theta, float* rope,
                                                              int rows) {
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= rows * 64) return;
  const int t = idx >> 6, p = idx & 63;
  double ang = 0.0;
  if (t >= n_txt) {
    const int g = t - n_txt;
    const int y = g / grid_w, x = g - y * grid_w;
    const double w = pow(theta, -(double)(p & 31) / 32.0);
    ang = (double)(p < 32 ? y : x) * w;
  }
  rope[idx] = (float)cos(ang);
  rope[(size_t)rows * 64 + idx] = (float)sin(ang);
}

int grid_for(long work, int per_block) {
  long g = (work + per_block - 1) / per_block;
  if (g > 65536L * 8) g = 65536L * 8;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_join_rows(const uint16_t* x, const uint16_t* txt, const ItemLens& lens, float* out, int batch,
                            int n_txt, int n_img, int d, hipStream_t st) {
  const long total = (long)batch * (n_txt + n_img) * (d / 8);
  hipLaunchKernelGGL(join_rows_kernel, dim3(grid_for(total, kThreads)), dim3(kThreads), 0, st,
                     reinterpret_cast<const u32x4*>(x), reinterpret_cast<const u32x4*>(txt), lens,
                     reinterpret_cast<f32x4*>(out), n_txt, n_img, d / 8, total);
  return hipGetLastError();
}

hipError_t launch_silu_cond(const uint16_t* cond, float* s, int batch, int d, hipStream_t st) {
  const int n = batch * d;
  hipLaunchKernelGGL(silu_cond_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, st, cond, s, n);
  return hipGetLastError();
}

// y[m][b][:n_out] = W_m x[b] for the set's matrices m < n_mats (each [n_out, d_in] bf16)
static hipError_t launch_gemv_set(const float* x, const GemvSet& set, int n_mats, float* y, int batch, int d_in,
                                  int n_out, hipStream_t st) {
  const int cpl = (d_in / 8 + 63) / 64;
  const dim3 grid((n_out + kGemvRows - 1) / kGemvRows, n_mats), block(64 * kGemvRows);
  if (cpl <= 2)
    hipLaunchKernelGGL(adaln_gemv_kernel<2>, grid, block, 0, st, x, set, y, batch, n_out, d_in);
  else if (cpl <= 4)
    hipLaunchKernelGGL(adaln_gemv_kernel<4>, grid, block, 0, st, x, set, y, batch, n_out, d_in);
  else if (cpl <= 6)
    hipLaunchKernelGGL(adaln_gemv_kernel<6>, grid, block, 0, st, x, set, y, batch, n_out, d_in);
  else if (cpl <= 8)
    hipLaunchKernelGGL(adaln_gemv_kernel<8>, grid, block, 0, st, x, set, y, batch, n_out, d_in);
  else
    hipLaunchKernelGGL(adaln_gemv_kernel<16>, grid, block, 0, st, x, set, y, batch, n_out, d_in);
  return hipGetLastError();
}

hipError_t launch_adaln_gemv(const float* s, const uint16_t* w_mod, float* mod, int batch, int d, unsigned skip_items,
                             hipStream_t st) {
  GemvSet set{};
  set.w[0] = w_mod;
  set.skip[0] = skip_items;
  return launch_gemv_set(s, set, 1, mod, batch, d, 6 * d, st);
}

hipError_t launch_adaln_gemv_many(const float* s, const uint16_t* const* w_mods, const unsigned* skip, int n,
                                  float* mod, int batch, int d, hipStream_t st) {
  for (int i0 = 0; i0 < n; i0 += kGemvSet) {
    GemvSet set{};
    const int k = std::min(kGemvSet, n - i0);
    for (int i = 0; i < k; ++i) {
      set.w[i] = w_mods[i0 + i];
      set.skip[i] = skip[i0 + i];
    }
    const hipError_t e = launch_gemv_set(s, set, k, mod + (size_t)i0 * batch * 6 * d, batch, d, 6 * d, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_mod_rmsnorm(const float* h, const float* shift, const float* scale, int mod_stride,
                              uint16_t* out, int batch, int rows, int d, float eps, hipStream_t st) {
  const int total = batch * rows;
  const int c4 = (d / 4 + 63) / 64;
  const dim3 grid((total + 3) / 4), block(kThreads);
#define MOSS_NORM_CASE(N)                                                                                        \
  if (c4 <= N) {                                                                                                 \
    hipLaunchKernelGGL(mod_rmsnorm_kernel<N>, grid, block, 0, st, h, shift, scale, mod_stride, out, total, rows, \
                       d, eps);                                                                                  \
    return hipGetLastError();                                                                                    \
  }
  MOSS_NORM_CASE(4) MOSS_NORM_CASE(8) MOSS_NORM_CASE(12) MOSS_NORM_CASE(16) MOSS_NORM_CASE(32)
#undef MOSS_NORM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gated_add(float* h, const float* gate, int gate_stride, const uint16_t* y, uint16_t* out16,
                            int batch, int rows, int d, hipStream_t st) {
  const long total = (long)batch * rows * (d / 8);
  hipLaunchKernelGGL(gated_add_kernel, dim3(grid_for(total, kThreads)), dim3(kThreads), 0, st,
                     reinterpret_cast<f32x4*>(h), gate, gate_stride, reinterpret_cast<const u32x4*>(y),
                     reinterpret_cast<u32x4*>(out16), d / 8, rows, total);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t* u, uint16_t* z, int rows, int f, hipStream_t st) {
  const long total = (long)rows * (f / 8);
  hipLaunchKernelGGL(silu_mul_kernel, dim3(grid_for(total, kThreads)), dim3(kThreads), 0, st, u,
                     reinterpret_cast<u32x4*>(z), f, total);
  return hipGetLastError();
}

hipError_t launch_rope_build(int n_txt, int grid_h, int grid_w, float theta, float* rope, hipStream_t st) {
  const int rows = n_txt + grid_h * grid_w;
  hipLaunchKernelGGL(rope_build_kernel, dim3((rows * 64 + kThreads - 1) / kThreads), dim3(kThreads), 0, st, n_txt,
                     grid_w, (double)theta, rope, rows);
  return hipGetLastError();
}

hipError_t launch_guidance_euler(int rows, int width, const uint16_t* v_pos, const uint16_t* v_neg, float g,
                                 float dsigma, const float* x_in, float* x_out, hipStream_t st) {
  const long total = (long)rows * (width / 8);
  hipLaunchKernelGGL(guidance_euler_kernel, dim3(grid_for(total, kThreads)), dim3(kThreads), 0, st,
                     reinterpret_cast<const u32x4*>(v_pos), reinterpret_cast<const u32x4*>(v_neg), g, dsigma,
                     reinterpret_cast<const f32x4*>(x_in), reinterpret_cast<f32x4*>(x_out), total);
  return hipGetLastError();
}

hipError_t launch_join_mod_rmsnorm(const uint16_t* x, const uint16_t* txt, const ItemLens& lens, const float* shift,
                                   const float* scale, int mod_stride, float* h, uint16_t* out, int batch, int n_txt,
                                   int n_img, int d, float eps, hipStream_t st) {
  const int total = batch * (n_txt + n_img);
  const int c4 = (d / 4 + 63) / 64;
  const dim3 grid((total + 3) / 4), block(kThreads);
#define MOSS_NORM_CASE(N)                                                                                           \
  if (c4 <= N) {                                                                                                    \
    hipLaunchKernelGGL(join_mod_rmsnorm_kernel<N>, grid, block, 0, st, x, txt, lens, shift, scale, mod_stride, h,  \
                       out, n_txt, n_img, d, eps, total);                                                           \
    return hipGetLastError();                                                                                       \
  }
  MOSS_NORM_CASE(4) MOSS_NORM_CASE(8) MOSS_NORM_CASE(12) MOSS_NORM_CASE(16) MOSS_NORM_CASE(32)
#undef MOSS_NORM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(const float* x, const uint16_t* w, float* y, int batch, int d_in, int n_out, hipStream_t st) {
  GemvSet set{};
  set.w[0] = w;
  return launch_gemv_set(x, set, 1, y, batch, d_in, n_out, st);
}

hipError_t launch_timestep_features(const ItemTimes& ts, float* f, int batch, hipStream_t st) {
  hipLaunchKernelGGL(timestep_features_kernel, dim3((batch * 256 + kThreads - 1) / kThreads), dim3(kThreads), 0, st,
                     ts, f, batch);
  return hipGetLastError();
}

hipError_t launch_silu_f32(const float* x, float* y, int n, hipStream_t st) {
  hipLaunchKernelGGL(silu_f32_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, st, x, y, n);
  return hipGetLastError();
}

hipError_t launch_round_bf16(const float* x, uint16_t* y, int n, hipStream_t st) {
  hipLaunchKernelGGL(round_bf16_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, st, x, y, n);
  return hipGetLastError();
}
