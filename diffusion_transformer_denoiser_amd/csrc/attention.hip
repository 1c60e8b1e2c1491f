// a5: full (non-causal) attention at head dim 128 with an online fp32
// softmax (the MOSS-Image transformer page, TensorFold PR #1528, "What it
// adds" and "Shared code": the head-128 instance of the full vision attention,
// softmax in fp32).
//
// gfx950 design.  A workgroup owns 128 queries of one (item, head); each of
// its four wavefronts owns 32 queries and keeps them in registers as MFMA
// operands for the whole key loop.  Keys advance 64 at a time through two LDS
// stages (K rows, and V transposed as packed by the q/k kernel).
//
// Per key tile a wavefront computes S^T = K Q^T (keys x queries) with
// v_mfma_f32_32x32x16_bf16, so a lane holds 32 of the 64 scores of ONE query
// (lane l and lane l ^ 32 share a query and split its keys).  The running
// max and sum need one exchange between the two half-waves.  The
// probabilities, rounded to bf16, are already laid out as the second operand
// of O^T += V^T P^T: the key order inside each 16-key group of the packed V
// matches the order in which a lane holds its scores.  O^T stays in 64
// accumulators per lane; no probability goes through LDS.
//
// Keys that are text padding (txt_len <= key < n_txt) or past the last row
// get -inf before the max; a tile with no valid key leaves the state as is.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace {

constexpr int BQ = 128;  // queries per workgroup
constexpr int BKV = 64;  // keys per tile
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(const uint16_t* __restrict__ qp,
                                                            const uint16_t* __restrict__ kp,
                                                            const uint16_t* __restrict__ vp,
                                                            uint16_t* __restrict__ o, int rows, int rows_pad,
                                                            int n_heads, int n_txt, ItemLens lens,
                                                            float scale_log2) {
  __shared__ u32x4 sk[2][BKV * 16];  // 64 keys x 16 chunks (256 B per key)
  __shared__ u32x4 sv[2][128 * 8];   // 128 dims x 8 chunks (64 keys per dim)

  const int qt = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const size_t bh = (size_t)b * n_heads + head;
  const uint16_t* qb = qp + bh * rows_pad * 128;
  const uint16_t* kb = kp + bh * rows_pad * 128;
  const uint16_t* vb = vp + bh * rows_pad * 128;
  const int valid_txt = lens.len[b];

  // this lane's query and its 128 dims as eight k16 operand fragments
  const int qrow = qt * BQ + wave * 32 + l32;
  bf16x8 qf[8];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(qb + (size_t)qrow * 128);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = __builtin_bit_cast(bf16x8, src[2 * s + hh]);
  }

  f32x16 acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc_o[i][e] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  const int n_tiles = (rows + BKV - 1) / BKV;
  u32x4 rk[4], rv[4];
  auto gload = [&](int kt) {
    const u32x4* ks = reinterpret_cast<const u32x4*>(kb + (size_t)kt * BKV * 128);
    const u32x4* vs = reinterpret_cast<const u32x4*>(vb + (size_t)kt * BKV * 128);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rk[i] = ks[tid + kThreads * i];
      rv[i] = vs[tid + kThreads * i];
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      const int key = id >> 4, ck = id & 15;
      sk[buf][key * 16 + (ck ^ (key & 7))] = rk[i];
      const int dim = id >> 3, cv = id & 7;
      sv[buf][dim * 8 + (cv ^ (dim & 7))] = rv[i];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_tiles) gload(kt + 1);

    // S^T for two 32-key halves of the tile
    f32x16 sacc[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[h2][e] = 0.0f;
      const int key = h2 * 32 + l32;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, sk[buf][key * 16 + ((2 * s + hh) ^ (key & 7))]);
        sacc[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[h2], 0, 0, 0);
      }
    }

    // scores in log2 units; lane holds keys 32*h2 + 8*q + 4*hh + e at sacc[h2][4q + e]
    const int key0 = kt * BKV;
    const bool need_mask = (key0 + BKV > rows) || (key0 < n_txt && key0 + BKV > valid_txt);
    float mloc = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float sv2 = sacc[h2][e] * scale_log2;
        if (need_mask) {
          const int key = key0 + h2 * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          const bool bad = (key >= rows) || (key >= valid_txt && key < n_txt);
          sv2 = bad ? -INFINITY : sv2;
        }
        sacc[h2][e] = sv2;
        mloc = fmaxf(mloc, sv2);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float corr = exp2f(m_run - m_use);
    float lsum = 0.0f;
    bf16x8 pf[4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float p[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          p[t] = exp2f(sacc[h2][8 * half + t] - m_use);
          lsum += p[t];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) pf[2 * h2 + half][t] = (__bf16)p[t];
      }
    }
    lsum += __shfl_xor(lsum, 32, 64);
    l_run = l_run * corr + lsum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[i][e] *= corr;

    // O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dim = i * 32 + l32;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 vf = __builtin_bit_cast(bf16x8, sv[buf][dim * 8 + ((2 * s + hh) ^ (dim & 7))]);
        acc_o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s], acc_o[i], 0, 0, 0);
      }
    }

    if (kt + 1 < n_tiles) sstore(buf ^ 1);
    __syncthreads();
  }

  // acc_o[i][4q + e] = O^T[dim = 32 i + 8 q + 4 hh + e][query l32]
  if (qrow < rows) {
    const float inv = 1.0f / l_run;
    uint16_t* orow = o + ((size_t)b * rows + qrow) * (n_heads * 128) + head * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dim = 32 * i + 8 * q + 4 * hh;
        u32x2 v = {pack_bf16x2(acc_o[i][4 * q] * inv, acc_o[i][4 * q + 1] * inv),
                   pack_bf16x2(acc_o[i][4 * q + 2] * inv, acc_o[i][4 * q + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + dim) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_attention(int batch, int n_heads, int rows, int n_txt, const ItemLens& lens, const uint16_t* q,
                            const uint16_t* k, const uint16_t* v, uint16_t* o, hipStream_t st) {
  const int rp = packed_rows(rows);
  const float scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(rp / BQ, n_heads, batch), dim3(kThreads), 0, st, q, k, v, o, rows, rp,
                     n_heads, n_txt, lens, scale_log2);
  return hipGetLastError();
}
