// a4: per (row, head) RMSNorm of q and k over the 128 head dims, times the
// q/k gain, then the rotary rotation of interleaved pairs; v copied.  The
// results are written in the packed layouts the attention kernel reads
// (see moss.h): Q and K row-major per (item, head), V transposed per 64-key
// tile (dim-major, keys in order), so that a 16-byte read of a V^T row gives
// eight consecutive keys of one dim.
//
// The MOSS-Image transformer page (TensorFold PR #1528, "What it adds") names
// this kernel "q/k norm and rotary into packed rows".
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace {

constexpr int kTok = 64;      // tokens per workgroup
constexpr int kThreads = 256; // 16 groups of 16 lanes; a group owns one 128-dim row
constexpr int kVPitch = 136;  // LDS row pitch (bf16) of the V staging tile

__global__ __launch_bounds__(kThreads) void qk_norm_rope_pack_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ q_gain, const uint16_t* __restrict__ k_gain,
    const float* __restrict__ rope, uint16_t* __restrict__ qo, uint16_t* __restrict__ ko, uint16_t* __restrict__ vo,
    int rows, int rows_pad, int n_heads, float eps) {
  __shared__ uint16_t vs[kTok * kVPitch];
  const int tile = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int t0 = tile * kTok;
  const int d = n_heads * 128;
  const int tid = threadIdx.x;
  const int grp = tid >> 4, j = tid & 15;
  const size_t bh = (size_t)b * n_heads + head;

  float gq[8], gk[8];
  unpack8(reinterpret_cast<const u32x4*>(q_gain)[j], gq);
  unpack8(reinterpret_cast<const u32x4*>(k_gain)[j], gk);

  // q and k: 128 rows (64 tokens x {q, k}), 16 per pass
#pragma unroll 1
  for (int it = 0; it < 8; ++it) {
    const int rr = it * 16 + grp;
    const int which = rr >> 6;  // 0 = q, 1 = k
    const int t = t0 + (rr & 63);
    float f[8];
    float ss = 0.0f;
    if (t < rows) {
      const uint16_t* src = qkv + ((size_t)b * rows + t) * 3 * d + which * d + head * 128;
      unpack8(reinterpret_cast<const u32x4*>(src)[j], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = 0.0f;
    }
    ss = group_sum<16>(ss);
    u32x4 res = {0u, 0u, 0u, 0u};
    if (t < rows) {
      const float r = 1.0f / sqrtf(ss / 128.0f + eps);
      const float* g = which ? gk : gq;
      const f32x4 c4 = reinterpret_cast<const f32x4*>(rope + (size_t)t * 64)[j];
      const f32x4 s4 = reinterpret_cast<const f32x4*>(rope + (size_t)rows * 64 + (size_t)t * 64)[j];
      float o[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = (f[2 * p] * r) * g[2 * p];
        const float x1 = (f[2 * p + 1] * r) * g[2 * p + 1];
        o[2 * p] = x0 * c4[p] - x1 * s4[p];
        o[2 * p + 1] = x0 * s4[p] + x1 * c4[p];
      }
      res = pack8(o);
    }
    uint16_t* dst = (which ? ko : qo) + (bh * rows_pad + t) * 128;
    reinterpret_cast<u32x4*>(dst)[j] = res;
  }

  // v: stage the 64 x 128 tile in LDS, then write it transposed
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + kThreads * i;  // 1024 chunks: token = id / 16, chunk = id % 16
    const int tk = id >> 4, c = id & 15;
    const int t = t0 + tk;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t < rows) v = reinterpret_cast<const u32x4*>(qkv + ((size_t)b * rows + t) * 3 * d + 2 * d + head * 128)[c];
    *reinterpret_cast<u32x4*>(&vs[tk * kVPitch + c * 8]) = v;
  }
  __syncthreads();
  uint16_t* vt = vo + (bh * (rows_pad / kTok) + tile) * (kTok * 128);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + kThreads * i;  // 1024 chunks: dim = id / 8, keys t0 + 8*(id % 8) .. +7
    const int dim = id >> 3, pc = id & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)vs[(pc * 8 + 2 * e) * kVPitch + dim] | ((uint32_t)vs[(pc * 8 + 2 * e + 1) * kVPitch + dim] << 16);
    u32x4 out = {w[0], w[1], w[2], w[3]};
    reinterpret_cast<u32x4*>(vt)[id] = out;
  }
}

// Pad rows of the packed layouts: Q and K rows T..T_pad-1 (contiguous per
// (item, head)) and V^T keys T..T_pad-1 of every dim row of the last tiles.
__global__ __launch_bounds__(256) void zero_packed_pads_kernel(uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                                               uint16_t* __restrict__ v, int rows, int rows_pad,
                                                               int n_bh) {
  const int npad = rows_pad - rows;
  const long long per = (long long)npad * 128, total = per * n_bh;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long long)gridDim.x * blockDim.x) {
    const long long bh = i / per, r = i - bh * per;
    q[(bh * rows_pad + rows) * 128 + r] = 0;
    k[(bh * rows_pad + rows) * 128 + r] = 0;
    const long long dim = r / npad, key = rows + (r - dim * npad);
    v[((bh * (rows_pad / 64) + key / 64) * 128 + dim) * 64 + (key & 63)] = 0;
  }
}

// rope [2][rows][64] -> rope_pp[pp][t][4] = cos, cos, sin, sin of pairs 2 pp and 2 pp + 1 (row stride
// rows_pad); one thread per (pp, t)
__device__ __forceinline__ void rope_pair_entry(const float* __restrict__ rope, int rows, int rows_pad, long long i,
                                                float* __restrict__ out) {
  const long long t = i % rows, pp = i / rows;
  const float2 c = *reinterpret_cast<const float2*>(rope + t * 64 + 2 * pp);
  const float2 s = *reinterpret_cast<const float2*>(rope + ((long long)rows + t) * 64 + 2 * pp);
  *reinterpret_cast<f32x4*>(out + (pp * rows_pad + t) * 4) = f32x4{c.x, c.y, s.x, s.y};
}

__global__ __launch_bounds__(256) void rope_pairs_kernel(const float* __restrict__ rope, int rows, int rows_pad,
                                                         float* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // pp * rows + t
  if (i >= 32 * rows) return;
  rope_pair_entry(rope, rows, rows_pad, i, out);
}

// The once-per-call preparation of a block stack in one launch: SiLU(cond)
// for the modulation GEMVs, the rotary table as pairs of pairs for the QKV
// epilogue, and zeros in the pad rows of packed Q, K and V^T.  One flat
// index runs over the three jobs in turn.
__global__ __launch_bounds__(256) void call_prologue_kernel(const uint16_t* __restrict__ cond, float* __restrict__ s,
                                                            int n_cond, const float* __restrict__ rope, int rows,
                                                            int rows_pad, float* __restrict__ rope_pp,
                                                            uint16_t* __restrict__ q, uint16_t* __restrict__ k,
                                                            uint16_t* __restrict__ v, int n_bh) {
  const long long n1 = n_cond, n2 = 32LL * rows, npad = rows_pad - rows, n3 = npad * 128 * n_bh;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n1 + n2 + n3;
       i += (long long)gridDim.x * blockDim.x) {
    if (i < n1) {
      s[i] = silu_f32(bf16_to_f32(cond[i]));
    } else if (i < n1 + n2) {
      rope_pair_entry(rope, rows, rows_pad, i - n1, rope_pp);  // pp * rows + t
    } else {
      const long long j = i - n1 - n2, per = npad * 128;
      const long long bh = j / per, r = j - bh * per;
      q[(bh * rows_pad + rows) * 128 + r] = 0;
      k[(bh * rows_pad + rows) * 128 + r] = 0;
      const long long dim = r / npad, key = rows + (r - dim * npad);
      v[((bh * (rows_pad / 64) + key / 64) * 128 + dim) * 64 + (key & 63)] = 0;
    }
  }
}

}  // namespace

hipError_t launch_call_prologue(const uint16_t* cond, float* s, int n_cond, const float* rope, int batch, int rows,
                                int n_heads, float* rope_pp, uint16_t* q, uint16_t* k, uint16_t* v, hipStream_t st) {
  const int rp = packed_rows(rows);
  const long long total = (long long)n_cond + 32LL * rows + (long long)(rp - rows) * 128 * batch * n_heads;
  const int blocks = (int)std::min<long long>((total + 255) / 256, 2048);
  hipLaunchKernelGGL(call_prologue_kernel, dim3(blocks), dim3(256), 0, st, cond, s, n_cond, rope, rows, rp, rope_pp,
                     q, k, v, batch * n_heads);
  return hipGetLastError();
}

hipError_t launch_rope_pairs(const float* rope, int rows, float* rope_pp, hipStream_t st) {
  hipLaunchKernelGGL(rope_pairs_kernel, dim3((32 * rows + 255) / 256), dim3(256), 0, st, rope, rows,
                     packed_rows(rows), rope_pp);
  return hipGetLastError();
}

hipError_t launch_zero_packed_pads(int batch, int rows, int n_heads, uint16_t* q, uint16_t* k, uint16_t* v,
                                   hipStream_t st) {
  const int rp = packed_rows(rows);
  if (rp == rows) return hipSuccess;
  const long long total = (long long)(rp - rows) * 128 * batch * n_heads;
  const int blocks = (int)std::min<long long>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_packed_pads_kernel, dim3(blocks), dim3(256), 0, st, q, k, v, rows, rp, batch * n_heads);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope_pack(int batch, int rows, int n_heads, float eps, const uint16_t* qkv,
                                    const uint16_t* q_gain, const uint16_t* k_gain, const float* rope,
                                    uint16_t* q, uint16_t* k, uint16_t* v, hipStream_t st) {
  const int rp = packed_rows(rows);
  hipLaunchKernelGGL(qk_norm_rope_pack_kernel, dim3(rp / kTok, n_heads, batch), dim3(kThreads), 0, st, qkv, q_gain,
                     k_gain, rope, q, k, v, rows, rp, n_heads, eps);
  return hipGetLastError();
}
