// a3/a6/a9/a11: the block's projections, c = a w^T with bf16 operands, fp32
// sums and a bf16 result (the MOSS-Image transformer page, TensorFold PR #1528,
// "What it adds": bf16 GEMMs with fp32 sums).
//
// gfx950 design: a workgroup computes a BM x BN tile of c with
// v_mfma_f32_32x32x16_bf16.  K advances 64 at a time through two LDS stages:
// while the MFMAs consume one stage, the next k-slab is loaded from global
// memory into registers and stored into the other stage after the MFMAs, one
// barrier per slab.  Rows of an LDS slab are 128 bytes (64 bf16 of k); the
// 16-byte chunk c of row r is stored at chunk c ^ (r & 7), so the 32 rows a
// wavefront reads for one MFMA operand fall on distinct banks.
//
// The MFMA's first operand is the weight tile and its second the activation
// tile, so each lane's 16 accumulators hold four runs of four consecutive
// output columns of one output row: the result leaves in 8-byte stores.
// There is no split-K and no atomic, so results are identical call to call.
#include "common.h"
#include "launch.h"

namespace {

constexpr int BK = 64;

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_kernel(const uint16_t* __restrict__ a, int lda,
                                                             const uint16_t* __restrict__ w, int ldw,
                                                             uint16_t* __restrict__ c, int ldc, int m, int k) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;  // wavefront tile (rows of c, columns of c)
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int ACH = BM * BK / 8, BCH = BN * BK / 8;  // 16-byte chunks per slab
  constexpr int LA = ACH / NT, LB = BCH / NT;
  static_assert(LA * NT == ACH && LB * NT == BCH, "tile / thread mismatch");

  __shared__ u32x4 sa[2][ACH];
  __shared__ u32x4 sb[2][BCH];

  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;

  // global -> register loads of one k-slab (rows past m are clamped; their results are never stored)
  const uint16_t* pa[LA];
  const uint16_t* pb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int id = tid + NT * i, r = id >> 3, ch = id & 7;
    const int row = min(m0 + r, m - 1);
    pa[i] = a + (size_t)row * lda + ch * 8;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int id = tid + NT * i, r = id >> 3, ch = id & 7;
    pb[i] = w + (size_t)(n0 + r) * ldw + ch * 8;
  }
  u32x4 ra[LA], rb[LB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + k0);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(pb[i] + k0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int id = tid + NT * i, r = id >> 3, ch = id & 7;
      sa[buf][r * 8 + (ch ^ (r & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int id = tid + NT * i, r = id >> 3, ch = id & 7;
      sb[buf][r * 8 + (ch ^ (r & 7))] = rb[i];
    }
  };

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = k / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 fw[FN], fa[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int r = wn * TN + i * 32 + l32;
        fw[i] = __builtin_bit_cast(bf16x8, sb[buf][r * 8 + ((2 * s + hh) ^ (r & 7))]);
      }
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int r = wm * TM + j * 32 + l32;
        fa[j] = __builtin_bit_cast(bf16x8, sa[buf][r * 8 + ((2 * s + hh) ^ (r & 7))]);
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fa[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // acc[i][j] is a 32 x 32 tile of c^T: lane holds row m = l32 of c and
  // columns n = 8q + 4hh + e (e = 0..3) in acc[4q + e].
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int row = m0 + wm * TM + j * 32 + l32;
    if (row < m) {
      uint16_t* crow = c + (size_t)row * ldc;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + wn * TN + i * 32 + 8 * q + 4 * hh;
          u32x2 v = {pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                     pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
          *reinterpret_cast<u32x2*>(crow + col) = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_nt(int m, int n, int k, const uint16_t* a, int lda, const uint16_t* w, int ldw,
                          uint16_t* c, int ldc, hipStream_t st) {
  if (n % 256 == 0) {
    constexpr int BM = 256, BN = 256;
    hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, 2, 4>), dim3(n / BN, (m + BM - 1) / BM), dim3(512), 0, st, a, lda,
                       w, ldw, c, ldc, m, k);
  } else {
    constexpr int BM = 256, BN = 128;
    hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, 4, 2>), dim3(n / BN, (m + BM - 1) / BM), dim3(512), 0, st, a, lda,
                       w, ldw, c, ldc, m, k);
  }
  return hipGetLastError();
}
