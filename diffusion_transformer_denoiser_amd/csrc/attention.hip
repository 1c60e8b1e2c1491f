// a5: full (non-causal) attention at head dim 128 with an online fp32
// softmax (the MOSS-Image transformer page, TensorFold PR #1528, "What it
// adds" and "Shared code": the head-128 instance of the full vision attention,
// softmax in fp32).
//
// gfx950 design.  A workgroup owns 256 queries of one (item, head); each of
// its eight wavefronts owns 32 queries and keeps them in registers as MFMA
// operands for the whole key loop.  One workgroup fills a CU (2 wavefronts
// per SIMD), and each K/V tile is loaded into LDS once for 256 queries (a
// 128-query workgroup, two per CU, loaded every tile twice per CU and ran 1%
// slower overall).
//
//  * The two wavefronts of a SIMD work a phase apart (wavefronts 0-3 and 4-7
//    form two groups, one of each per SIMD).  A wavefront alternates a
//    matrix step (O^T += V^T P^T for the previous tile, then S^T = K Q^T for
//    this one) with a softmax step, so one group's softmax can issue while
//    the other group's MFMAs occupy the SIMD's matrix pipe.  With one phase
//    for both (the earlier form), both wavefronts of a SIMD ran their MFMAs,
//    then both their softmax, and the two pipes seldom overlapped.
//  * Keys advance 64 at a time through three LDS stages (K rows, and the 64-key
//    V^T tile: 128 dim rows of 64 keys), each filled straight from
//    global memory with global_load_lds_dwordx4 (issued from asm, so the
//    compiler's waits on the fragment reads stay exact).  The K chunk
//    c of key row r is stored at c ^ (r & 15) (256-byte rows) and the V
//    chunk c of dim row d at c ^ ((d >> 1) & 7) (128-byte rows), so the 16
//    rows a 16-lane group reads fall in distinct 16-byte bank slots.
//  * Per key tile a wavefront computes S^T = K Q^T (keys x queries) with
//    v_mfma_f32_32x32x16_bf16, so lane l holds 32 of the 64 scores of ONE
//    query and lane l ^ 32 the other 32; the max and the sum need one
//    v_permlane32_swap each.  The two 32-key accumulators (and the four PV
//    accumulators) alternate, so no MFMA waits for the result of the one
//    before it, and fragment reads run four MFMAs ahead of their use.
//  * The query fragments are loaded once, before the key loop, and marked
//    ready at the first barrier, so the loop never waits on the vector memory
//    counter (which the in-flight tile loads share) for them.
//  * Scores are scaled into log2 units inside the exp2 argument (one FMA per
//    score) and exponentiated with v_exp_f32 directly (results below 2^-126
//    of the row max flush to zero, which no bf16 probability could hold).
//    The running max used for the exponentials only moves when a row's max
//    grows by more than 8 (in log2 units) anywhere in the wavefront; until
//    then probabilities may reach 2^8, which fp32 sums and bf16 products hold
//    exactly as well, and O and the sum need no rescale.
//  * The probabilities, rounded to bf16, are already laid out as the second
//    operand of O^T += V^T P^T: the K fragments read their key rows with
//    quads 1 and 2 of each 16-key group swapped, so each lane holds the
//    scores of 8 consecutive keys per group, the keys one 16-byte read of a
//    V^T row gives.  O^T stays in 64 accumulators per lane; no probability
//    goes through LDS.
// Keys that are text padding (txt_len <= key < n_txt) or past the last row
// get -inf; a tile with no valid key leaves the state as it is.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace {

// fragment reads issued ahead of the MFMAs of a matrix step (deeper lookahead, 6 or 8, changed nothing)
constexpr int kReadsAhead = 4;

constexpr int NWV = 8;           // wavefronts per workgroup, 32 queries each: two groups of four
constexpr int BQ = 32 * NWV;     // queries per workgroup
constexpr int LPW = 16 / NWV;    // 1 KiB direct loads per wavefront per K (and per V) tile
constexpr int BKV = 64;          // keys per tile
constexpr int kThreads = 64 * NWV;
constexpr int kStage = 32768;    // K tile (16 KiB) then V^T tile (16 KiB)
constexpr int kStages = 3;       // K/V tiles in LDS
constexpr float kLazy = 8.0f;  // log2-unit growth of a row max that forces a rescale

// Row r of a 32-key block of S^T holds key quad_swap(r): quads 1 and 2 of
// each 16-key group trade places (the K fragment's lane l32 reads key row
// quad_swap(l32)).  A lane then holds, for each 16-key group, the scores of
// 8 consecutive keys (4hh..4hh+3 and 8+4hh..11+4hh of S^T's rows are keys
// 8hh..8hh+7), which is what the V^T fragment of the PV product pairs with:
// 8 consecutive keys of one dim, one 16-byte read from a plain V^T tile.
__device__ __forceinline__ int quad_swap(int r) {
  const int q = (r >> 2) & 3;
  return (r & ~15) | ((q == 1 ? 2 : (q == 2 ? 1 : q)) << 2) | (r & 3);
}

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(const uint16_t* __restrict__ qp,
                                                               const uint16_t* __restrict__ kp,
                                                               const uint16_t* __restrict__ vp,
                                                               uint16_t* __restrict__ o, int rows, int rows_pad,
                                                               int n_heads, int n_txt, ItemLens lens,
                                                               float scale_log2) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStage];

  // Workgroup ids are dealt round-robin over the 8 XCDs; remap them so each XCD runs a contiguous
  // stretch of the (item, head, query tile) order: the query tiles of a head then share their
  // XCD's L2, and its K/V tiles are fetched into one L2 rather than all eight.
  const int nqt = gridDim.x, nblk = nqt * gridDim.y * gridDim.z;
  const int id = blockIdx.x + nqt * (blockIdx.y + gridDim.y * blockIdx.z);
  const int per = nblk / 8, rem = nblk % 8, x = id % 8, l = id / 8;
  const int logical = (x < rem) ? x * (per + 1) + l : rem * (per + 1) + (x - rem) * per + l;
  const int qt = logical % nqt, head = (logical / nqt) % n_heads, b = logical / (nqt * n_heads);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const size_t bh = (size_t)b * n_heads + head;
  const uint16_t* qb = qp + bh * rows_pad * 128;
  const uint16_t* kb = kp + bh * rows_pad * 128;
  const uint16_t* vb = vp + bh * rows_pad * 128;
  const int valid_txt = lens.len[b];

  // this lane's query and its 128 dims as eight k16 operand fragments
  const int qrow = qt * BQ + wave * 32 + l32;
  bf16x8 qf[8];
  {
    // a workgroup may extend past the packed rows when BQ > 128: those lanes re-read the last packed
    // row and store nothing
    const u32x4* src = reinterpret_cast<const u32x4*>(qb + (size_t)min(qrow, rows_pad - 1) * 128);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = __builtin_bit_cast(bf16x8, src[2 * s + hh]);
  }

  // direct-to-LDS load sources: instruction i of this wavefront fills 1 KiB block (wave + 4i)
  // of the K tile (4 key rows of 256 B) and of the V^T tile (8 dim rows of 128 B)
  int koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int blk = wave + NWV * i;
    const int key = blk * 4 + (lane >> 4);
    koff[i] = key * 128 + (((lane & 15) ^ (key & 15)) * 8);
    const int dim = blk * 8 + (lane >> 3);
    voff[i] = dim * 64 + (((lane & 7) ^ ((dim >> 1) & 7)) * 8);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MOSS_LDS char*)smem + 1024u * __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int kt) {
    const uint16_t* ks = kb + (size_t)kt * BKV * 128;
    const uint16_t* vs = vb + (size_t)kt * BKV * 128;
    const uint32_t base = lds0 + (uint32_t)((kt % kStages) * kStage);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      dma16(ks + koff[i], base + 1024u * NWV * i);
      dma16(vs + voff[i], base + 16384u + 1024u * NWV * i);
    }
  };
  // this lane's fragment offsets within a stage
  int kfo[2][8], vfo[4][4];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int key = h2 * 32 + quad_swap(l32);
#pragma unroll
    for (int s = 0; s < 8; ++s) kfo[h2][s] = key * 256 + (((2 * s + hh) ^ (key & 15)) * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int dim = i * 32 + l32;
#pragma unroll
    for (int s = 0; s < 4; ++s) vfo[i][s] = 16384 + dim * 128 + (((2 * s + hh) ^ ((dim >> 1) & 7)) * 16);
  }

  f32x16 acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc_o[i][e] = 0.0f;
  float m_use = -INFINITY;  // max (log2 units, scaled) the exponentials are taken against
  float l_run = 0.0f;

  const int n_tiles = (rows + BKV - 1) / BKV;
  // Phase 2t is group 0's matrix step t and phase 2t+1 its softmax of tile
  // t; group 1 runs one phase behind.  Tile t's K is read in phases 2t and
  // 2t+1 and its V^T in 2t+2 and 2t+3, so three stages rotate: tile t+2 is
  // loaded after the barrier that ends phase 2t+1 (into the stage of tile
  // t-1, whose last reads were in that phase) and waited for at the barrier
  // that ends phase 2t+3.  Only those barriers are workgroup barriers; the
  // offset between the groups comes from the program order alone (a second
  // barrier per tile, to pin it, cost 1% per block).
  const int grp = wave >> 2;
  f32x16 sacc[2];
  bf16x8 pf[4];
  issue(0);
  if (n_tiles > 1) issue(1);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier"
               : "+v"(qf[0]), "+v"(qf[1]), "+v"(qf[2]), "+v"(qf[3]), "+v"(qf[4]), "+v"(qf[5]), "+v"(qf[6]),
                 "+v"(qf[7])
               :
               : "memory");
  auto qk = [&](int t) {
    const char* st = smem + (t % kStages) * kStage;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[h2][e] = 0.0f;
    bf16x8 kf[8][2];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) kf[s][h2] = *reinterpret_cast<const bf16x8*>(st + kfo[h2][s]);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) sacc[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s][h2], qf[s], sacc[h2], 0, 0, 0);
  };
  auto pv = [&](int t) {
    const char* st = smem + (t % kStages) * kStage;
    bf16x8 vf[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) vf[s][i] = *reinterpret_cast<const bf16x8*>(st + vfo[i][s]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s][i], pf[s], acc_o[i], 0, 0, 0);
    }
  };
  auto softmax = [&](int t) {
    const int key0 = t * BKV;
    if ((key0 + BKV > rows) || (key0 < n_txt && key0 + BKV > valid_txt)) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + h2 * 32 + quad_swap(8 * (e >> 2) + 4 * hh + (e & 3));
          const bool bad = (key >= rows) || (key >= valid_txt && key < n_txt);
          sacc[h2][e] = bad ? -INFINITY : sacc[h2][e];
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, sacc[h2][e]);
    mloc = pair_max(mloc) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mloc > m_use + kLazy) != 0ull) {
      const float m_new = fmaxf(m_use, mloc);
      const float corr = __builtin_amdgcn_exp2f(m_use - m_new);
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc_o[i][e] *= corr;
      m_use = m_new;
    }
    const float moff = (m_use == -INFINITY) ? 0.0f : m_use;
    float lsum = 0.0f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[h2][8 * half + tt], scale_log2, -moff));
          lsum += p;
          pf[2 * h2 + half][tt] = (__bf16)p;
        }
    l_run += pair_sum(lsum);
  };
  // ends of the even phases: nothing is scheduled across them
  auto bar = [&]() { __builtin_amdgcn_sched_barrier(0); };
  // end of phase 2t+1: tile t+1 (loaded after the previous such barrier) must be resident; then
  // tile t+2 goes into the stage of tile t-1
  auto bar_load = [&](int t) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (t + 2 < n_tiles) issue(t + 2);
    __builtin_amdgcn_sched_barrier(0);
  };
  // a matrix step: O^T += V^T P^T for tile t-1, then S^T = K Q^T for tile t
  // The matrix step runs at raised wavefront priority, so the SIMD issues its MFMAs as soon as the
  // pipe takes them and the other group's softmax fills the remaining slots (-5 us per block).
  auto pv_qk = [&](int t) {
    __builtin_amdgcn_s_setprio(1);
    pv(t - 1);
    qk(t);
    __builtin_amdgcn_sched_group_barrier(0x100, kReadsAhead, 0);
#pragma unroll
    for (int q = 0; q < 32 - kReadsAhead; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kReadsAhead, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  // Both groups pass the same n_tiles + 1 workgroup barriers (the first one above).
  if (__builtin_amdgcn_readfirstlane(grp) == 0) {
    qk(0);
    bar();
    for (int t = 0; t + 1 < n_tiles; ++t) {
      softmax(t);
      bar_load(t);
      pv_qk(t + 1);
      bar();
    }
    softmax(n_tiles - 1);
    bar_load(n_tiles - 1);
    pv(n_tiles - 1);
    bar();
  } else {
    bar();
    qk(0);
    bar_load(0);
    softmax(0);
    bar();
    for (int t = 1; t < n_tiles; ++t) {
      pv_qk(t);
      bar_load(t);
      softmax(t);
      bar();
    }
    pv(n_tiles - 1);
  }

  // acc_o[i][4q + e] = O^T[dim = 32 i + 8 q + 4 hh + e][query l32]
  if (qrow < rows) {
    const float inv = 1.0f / l_run;
    uint16_t* orow = o + ((size_t)b * rows + qrow) * (n_heads * 128) + head * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        u32x2 v[2];
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const int q = 2 * p + qq;
          v[qq] = u32x2{pack_bf16x2(acc_o[i][4 * q] * inv, acc_o[i][4 * q + 1] * inv),
                        pack_bf16x2(acc_o[i][4 * q + 2] * inv, acc_o[i][4 * q + 3] * inv)};
        }
        // dims 32 i + 8 (2p + hh) + (0..7)
        *reinterpret_cast<u32x4*>(orow + 32 * i + 8 * (2 * p + hh)) = pair_cols(v[0], v[1]);
      }
    }
  }
}

}  // namespace

hipError_t launch_attention(int batch, int n_heads, int rows, int n_txt, const ItemLens& lens, const uint16_t* q,
                            const uint16_t* k, const uint16_t* v, uint16_t* o, hipStream_t st) {
  const int rp = packed_rows(rows);
  const float scale_log2 = (float)(1.4426950408889634 / sqrt(128.0));
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((rp + BQ - 1) / BQ, n_heads, batch), dim3(kThreads), 0, st, q, k, v, o, rows, rp,
                     n_heads, n_txt, lens, scale_log2);
  return hipGetLastError();
}
