// a3/a6/a9/a11: the block's projections, c = a w^T with bf16 operands, fp32
// sums and a bf16 result (the MOSS-Image transformer page, TensorFold PR #1528,
// "What it adds": bf16 GEMMs with fp32 sums).
//
// gfx950 design.  A workgroup of 8 wavefronts computes a BM x BN tile of c
// (256 x 256 mostly) with v_mfma_f32_32x32x16_bf16; each wavefront owns a
// (BM/WM) x (BN/WN) sub-tile whose fp32 accumulators stay in registers for
// the whole K loop.
//
//  * K advances 64 at a time through two LDS stages (128 KiB for the 256 x 256
//    tiles; launches of one tile per workgroup whose tiles leave room use
//    three or four).  In the 256 x 256 and 224 x 256 launches (but QKV's,
//    whose epilogue borrows a whole stage) the weight tiles have a ring of
//    their own, one stage deeper, in the LDS the two A stages leave (160 and
//    152 KiB in all), and are loaded two slabs ahead: with one slab of
//    lead the waves waited on them (the down projection 296 -> 280 us, out
//    89 -> 83 us, same-box A/B).  Each slab is fetched straight into LDS with
//    buffer_load_dwordx4 ... lds (issued from asm, see dma16_buf_so), the
//    next slab's loads spread evenly over the MFMAs of the current slab's
//    first two k16 steps, so they have the last two steps to land before the
//    slab's one barrier.  A slab row is 128 bytes: every load covers whole
//    cache lines (32-k slabs read half lines, twice as many L2 requests;
//    4096 x 24576 x 3072 went from 519 to 483 us standalone with this scheme).
//  * The MFMA operands of the next k16 step are read from LDS into registers
//    during the current one, one read after each of its first MFMAs; nothing
//    is reordered across those points (sched_barrier), so the reads, loads
//    and MFMAs issue interleaved in the order written.
//  * Few instructions between two MFMAs (a wavefront issues at most one
//    every few cycles, an MFMA runs 32): a load is four instructions (no
//    branch; the k offset in the scalar offset), a lane's fragment reads
//    share one base per k16 step, the next slab's first read addresses are
//    ready before the barrier, and a tile's first k-step adds to zero rather
//    than to cleared registers.
//  * The 16-byte chunk c of row r is stored at c ^ ((r >> 1) & 7), so the 16
//    rows a 16-lane group reads for one operand fragment land in 16 distinct
//    16-byte slots of the LDS banks.
//  * Tiles are numbered in groups of six column tiles, row-major within a
//    group, and workgroup ids (dealt round-robin over the 8 XCDs) are
//    remapped so each XCD runs a contiguous stretch of that order: with groups of six, the ~32 tiles an XCD holds at
//    once span about 5 row and 6 column panels, which its L2 shares (fetch
//    from beyond L2 down ~40% from an M-fastest order).
//  * The weight tile is the MFMA's first operand and the activation tile the
//    second, so a lane's accumulators hold runs of four consecutive output
//    columns of one row; lane pairs trade halves (pair_cols) so that bf16
//    results leave in 16-byte stores (half the store instructions of 8-byte
//    ones: QKV 271 -> 257 us, up 589 -> 583 us on one box).
//  * Launches with more tiles than CUs run one workgroup per CU, each taking
//    every G-th tile in turn; its loads run on across its tiles, so a tile's
//    first slab is in LDS when the previous tile's epilogue starts.
//  * The QKV epilogue's q and k rows pass through LDS so that each store
//    instruction writes whole 128-byte half-head rows.
// There is no split-K and no atomic: results are identical call to call.
//
// Epilogues (the MOSS-Image transformer page's SiLU and gated-add kernels,
// "What it adds", applied to the fp32 sums before any rounding):
//  * kStore: c = bf16(acc).
//  * kSiluGate (the up projection, w = [gate rows; up rows], n = 2F): the
//    weight tile of column tile t holds gate rows and up rows of the same
//    128 outputs, interleaved per 32 so that one lane owns both sums of an
//    output; c[:, F-wide] = bf16(SiLU(gate) * up).  u is never stored.
//  * kGatedAdd (the out and down projections): h[r, :] += gate[b, :] * acc on
//    the fp32 residual, or, for the last add of a call, out = bf16(h + gate *
//    acc) with h unchanged.  The projection output is never stored.
#include <algorithm>
#include <type_traits>
#include <cmath>

#include "common.h"
#include "launch.h"

namespace {

constexpr int KB = 64;      // k per slab (a 128-byte row segment: whole cache lines)

enum Epi { kStore = 0, kSiluGate = 1, kGatedAdd = 2, kQkvPack = 3 };

struct EpiArgs {
  float* h;           // kGatedAdd: fp32 residual [m, n], row stride n
  const float* gate;  // kGatedAdd: gate of item b at gate + b * gate_stride
  int gate_stride;
  int rows_per_item;  // kGatedAdd, kQkvPack: rows of one item
  uint16_t* out16;    // kGatedAdd: when set, bf16 result here instead of updating h
  // kQkvPack: q/k gains [128], the rotary table re-laid as pairs of pairs (launch_rope_pairs:
  // rope_pp[pp][t] = {cos, cos, sin, sin} of pairs 2 pp and 2 pp + 1, row stride rows_pad), packed outputs
  const uint16_t* q_gain;
  const uint16_t* k_gain;
  const float* rope_pp;
  uint16_t* qo;
  uint16_t* ko;
  uint16_t* vo;
  int rows_pad, n_heads;
  float eps;
  int col0;           // kQkvPack: absolute column of this launch's column 0
};

// Column tiles per group of the tile order.  For the up projection's whole tiles (96 column
// tiles) groups of 3 to 6 run level and 16 lose 0.9% per block (two interleaved same-box runs
// each; 16 had won 4 us over 6 before the weight tiles' ring of their own, which made the loads
// the waves wait on fewer); QKV's and the out and down projections' sweeps (3, 4, 10, 12, 15)
// stayed within the runs' 1% spread.
constexpr int kGroupN = 6;
constexpr int kGroupNQkv = 6;
constexpr int kGroupNGated = 6;

// Workgroup id -> (tile_m, tile_n).  Logical order: column tiles in groups of
// GRP, each group row-major (N fastest); workgroup ids are dealt round-robin
// over the 8 XCDs, so they are remapped to give each XCD a contiguous run of
// that order.
template <int GRP>
__device__ __forceinline__ void tile_of(int id, int mt, int nt, int& tm, int& tn) {
  const int nblk = mt * nt;
  const int per = nblk / 8, rem = nblk % 8;
  const int x = id % 8, l = id / 8;
  const int logical = (x < rem) ? x * (per + 1) + l : rem * (per + 1) + (x - rem) * per + l;
  const int g = logical / (GRP * mt), r = logical % (GRP * mt);
  const int cols = min(GRP, nt - g * GRP);
  tm = r / cols;
  tn = g * GRP + r % cols;
}

// acc[i][j] is a 32 x 32 tile of c^T: lane holds row m = l32 of c and
// columns n = 8q + 4hh + e (e = 0..3) in acc[4q + e].
template <int BM, int BN, int WM, int WN, int EPI>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[BN / WN / 32][BM / WM / 32], int m0, int n0, int tn,
                                         int wm, int wn, int l32, int hh, int m, int n, uint16_t* __restrict__ c,
                                         int ldc, const EpiArgs& ep) {
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int row = m0 + wm * TM + j * 32 + l32;
    if (row >= m) continue;
    if (EPI == kSiluGate) {
      uint16_t* crow = c + (size_t)row * ldc;
#pragma unroll
      for (int pr = 0; pr < FN / 2; ++pr)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          u32x2 v[2];
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const int q = 2 * p + qq;
            float z[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] = silu_f32(acc[2 * pr][j][4 * q + e]) * acc[2 * pr + 1][j][4 * q + e];
            v[qq] = u32x2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
          }
          const int col = tn * (BN / 2) + wn * (TN / 2) + pr * 32 + 8 * (2 * p + hh);
          *reinterpret_cast<u32x4*>(crow + col) = pair_cols(v[0], v[1]);
        }
    } else if (EPI == kGatedAdd) {
      const int b = row / ep.rows_per_item;
      const float* g = ep.gate + (size_t)b * ep.gate_stride;
      float* hrow = ep.h + (size_t)row * n;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          u32x2 v[2];
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const int q = 2 * p + qq;
            const int col = n0 + wn * TN + i * 32 + 8 * q + 4 * hh;
            const f32x4 g4 = *reinterpret_cast<const f32x4*>(g + col);
            const f32x4 h4 = *reinterpret_cast<const f32x4*>(hrow + col);
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = h4[e] + g4[e] * acc[i][j][4 * q + e];
            if (ep.out16)
              v[qq] = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            else
              *reinterpret_cast<f32x4*>(hrow + col) = o;
          }
          if (ep.out16)
            *reinterpret_cast<u32x4*>(ep.out16 + (size_t)row * n + n0 + wn * TN + i * 32 + 8 * (2 * p + hh)) =
                pair_cols(v[0], v[1]);
        }
      }
    } else {
      uint16_t* crow = c + (size_t)row * ldc;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          u32x2 v[2];
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const int q = 2 * p + qq;
            v[qq] = u32x2{pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                          pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
          }
          const int col = n0 + wn * TN + i * 32 + 8 * (2 * p + hh);
          *reinterpret_cast<u32x4*>(crow + col) = pair_cols(v[0], v[1]);
        }
      }
    }
  }
}

// kGatedAdd for the one-wavefront-row layout (BM x 256 tiles, 8 wavefronts
// of BM x 32) on a workgroup's last tile, when the ring is idle: the sums go
// through LDS so that the fp32 residual is read and written in whole
// 512-byte row segments (two rows per instruction) rather than as 32-byte
// pieces of 32 rows.  The 256 columns go in two halves of 128 (BM x 132
// floats, rows padded by 16 bytes against bank conflicts).
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void epilogue_gated_lds(const f32x16 (&acc)[BN / WN / 32][BM / WM / 32], char* smem,
                                                   int m0, int n0, int wave, int l32, int hh, int m, int n,
                                                   const EpiArgs& ep) {
  constexpr int FM = BM / 32;
  constexpr int LDR = 132;  // floats per staged row
  static_assert(WM == 1 && WN == 8 && BN == 256, "one wavefront row of 32-column strips");
  static_assert(BM * LDR * 4 <= 2 * (BM + BN) * KB * 2, "half a tile fits the two stages");
  float* st = reinterpret_cast<float*>(smem);
  const int lane = threadIdx.x & 63;
  const int c4 = 4 * (lane & 31);  // this lane's 4 columns of the half
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((wave >> 2) == half) {
      // acc[0][j][4q + e] = sum at row j*32 + l32, column (wave % 4)*32 + 8q + 4hh + e of the half
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {acc[0][j][4 * q], acc[0][j][4 * q + 1], acc[0][j][4 * q + 2], acc[0][j][4 * q + 3]};
          *reinterpret_cast<f32x4*>(st + (j * 32 + l32) * LDR + (wave & 3) * 32 + 8 * q + 4 * hh) = v;
        }
    }
    __syncthreads();
    // each wavefront takes rows wave, wave + 8, ...: lanes 0-31 one row, 32-63 the next
    constexpr int IT = BM / 16;              // row pairs per wavefront
    constexpr int NB = IT % 2 == 0 ? IT / 2 : IT;  // residual loads in flight at once
    const int col = n0 + half * 128 + c4;
    // the gate row of the tile's item, when all its rows belong to one item
    const int b0 = m0 / ep.rows_per_item;
    const bool one_item = b0 == (min(m0 + BM, m) - 1) / ep.rows_per_item;
    f32x4 g1 = {0.f, 0.f, 0.f, 0.f};
    if (one_item) g1 = *reinterpret_cast<const f32x4*>(ep.gate + (size_t)b0 * ep.gate_stride + col);
#pragma unroll
    for (int i0 = 0; i0 < IT; i0 += NB) {
      f32x4 h4[NB];
#pragma unroll
      for (int it = 0; it < NB; ++it) {
        const int row = m0 + ((i0 + it) * 8 + wave) * 2 + hh;
        if (row < m) h4[it] = *reinterpret_cast<const f32x4*>(ep.h + (size_t)row * n + col);
      }
#pragma unroll
      for (int it = 0; it < NB; ++it) {
        const int lr = ((i0 + it) * 8 + wave) * 2 + hh, row = m0 + lr;
        if (row >= m) continue;
        const f32x4 g4 =
            one_item ? g1 : *reinterpret_cast<const f32x4*>(ep.gate + (size_t)(row / ep.rows_per_item) * ep.gate_stride + col);
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(st + lr * LDR + c4);
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = h4[it][e] + g4[e] * a4[e];
        if (ep.out16) {
          const u32x2 v = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          *reinterpret_cast<u32x2*>(ep.out16 + (size_t)row * n + col) = v;
        } else {
          *reinterpret_cast<f32x4*>(ep.h + (size_t)row * n + col) = o;
        }
      }
    }
    __syncthreads();
  }
}

// kQkvPack: the QKV projection with a4 in its epilogue.  Each value is first
// rounded to bf16, as the projection output would store it.  A wavefront owns
// 64 columns, half of one head of q, k or v; for q and k the per-(row, head)
// sum of squares (of the fp32 sums) adds the partner wavefront's half through
// LDS, then each value is scaled by 1/sqrt(mean + eps) and the gain and its
// pair rotated,
// and the row goes to the packed Q or K layout [B, H, T_pad, 128].  v values
// go to V^T [B, H, T_pad/64, 128, 64] one bf16 at a time (the 32 lanes of a
// half wavefront write 32 consecutive keys of one dim: one 64-byte segment).
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void epilogue_qkv(const f32x16 (&acc)[BN / WN / 32][BM / WM / 32], char* smem, int m0,
                                             int n0, int wave, int wm, int wn, int l32, int hh, int m,
                                             const EpiArgs& ep) {
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  static_assert(TN == 64 && FN == 2 && WN % 2 == 0, "a head's 128 columns are one pair of wavefronts");
  const int T = ep.rows_per_item, H = ep.n_heads, D = H * 128;
  const int col = ep.col0 + n0 + wn * TN;  // this wavefront's first column of [q | k | v]
  const int which = col / D, head = (col - which * D) >> 7, half = ((col - which * D) >> 6) & 1;

  // the value as the projection output would store it (rounded where used, not kept in registers)
  auto xr = [&](int i, int j, int e) { return (float)(__bf16)acc[i][j][e]; };
  // per-row sums of squares over the fp32 sums (before the bf16 rounding; the scale differs from
  // the rounded values' by about 1e-5 relative, far inside a bf16 ulp, and costs no rounding here)
  float ss[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    float sj = 0.0f;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) sj += acc[i][j][e] * acc[i][j][e];
    ss[j] = sj + __shfl_xor(sj, 32, 64);  // the wavefront's 64 columns of row j*32 + l32
  }
  // [wavefront][TM] in a ring stage no load writes before the next tile's first k-step.  The
  // barriers wait for LDS only: the next tile's slab loads stay in flight.
  float* ss_lds = reinterpret_cast<float*>(smem);
  if (hh == 0)
#pragma unroll
    for (int j = 0; j < FM; ++j) ss_lds[wave * TM + j * 32 + l32] = ss[j];
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int j = 0; j < FM; ++j) ss[j] += ss_lds[(wave ^ 1) * TM + j * 32 + l32];
  // every partner read done before that stage is loaded again
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  if (which < 2) {
    // gains of this lane's dims half*64 + 32 i + 8 q + 4 hh + e
    float g[FN][4][4];
    const uint16_t* gsrc = (which ? ep.k_gain : ep.q_gain) + half * 64 + 4 * hh;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 w2 = *reinterpret_cast<const u32x2*>(gsrc + i * 32 + 8 * q);
        g[i][q][0] = bf16_lo(w2[0]);
        g[i][q][1] = bf16_hi(w2[0]);
        g[i][q][2] = bf16_lo(w2[1]);
        g[i][q][3] = bf16_hi(w2[1]);
      }
    uint16_t* dbase = which ? ep.ko : ep.qo;
    // Each 32-row block's results go through this wavefront's 4 KiB of LDS (its own: no barrier)
    // and leave as whole 128-byte half-head rows, eight rows per store instruction: stored straight
    // from the MFMA layout, each instruction wrote 16 bytes into each of 64 rows, and the q/k
    // stores cost about 15 us of the QKV projection.  Chunk c of row r sits at c ^ (r & 7).
    static_assert(WM * WN * 4096 <= (BM + BN) * KB * 2, "the transposes fit one ring stage");
    char* tr = smem + wave * 4096;
    const int lane = l32 + 32 * hh;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int row = m0 + wm * TM + j * 32 + l32;
      if (row < m) {
      const int b = row / T, t = row - b * T;
      const float r = 1.0f / sqrtf(ss[j] / 128.0f + ep.eps);
      // pairs p0 = half*32 + 16 i + 4 q + 2 hh and p0 + 1: one 16-byte entry of the pair-of-pairs table
      // per (i, q); the 32 lanes of a half wavefront read 32 consecutive rows of it, 512 contiguous bytes
      const float* cr = ep.rope_pp + ((size_t)(half * 16 + hh) * ep.rows_pad + t) * 4;
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          u32x2 v[2];
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const int q = 2 * p + qq;
            const size_t po = (size_t)(8 * i + 2 * q) * ep.rows_pad * 4;  // pair-of-pairs p0 / 2 - (half*16 + hh)
            const f32x4 cs4 = *reinterpret_cast<const f32x4*>(cr + po);
            const float cs[2] = {cs4[0], cs4[1]}, sn[2] = {cs4[2], cs4[3]};
            float o[4];
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
              const float x0 = (xr(i, j, 4 * q + 2 * pr) * r) * g[i][q][2 * pr];
              const float x1 = (xr(i, j, 4 * q + 2 * pr + 1) * r) * g[i][q][2 * pr + 1];
              o[2 * pr] = x0 * cs[pr] - x1 * sn[pr];
              o[2 * pr + 1] = x0 * sn[pr] + x1 * cs[pr];
            }
            v[qq] = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          }
          // dims 32 i + 8 (2p + hh) + (0..7) of this half head: chunk 4 i + 2 p + hh of the row
          const int c = 4 * i + 2 * p + hh;
          *reinterpret_cast<u32x4*>(tr + l32 * 128 + ((c ^ (l32 & 7)) * 16)) = pair_cols(v[0], v[1]);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // lane: chunk lane & 7 of rows k*8 + lane/8 of the block
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rr = 8 * k + (lane >> 3), cc = lane & 7;
        const int row2 = m0 + wm * TM + j * 32 + rr;
        const u32x4 val = *reinterpret_cast<const u32x4*>(tr + rr * 128 + ((cc ^ (rr & 7)) * 16));
        if (row2 < m) {
          const int b2 = row2 / T, t2 = row2 - b2 * T;
          *reinterpret_cast<u32x4*>(dbase + (((size_t)b2 * H + head) * ep.rows_pad + t2) * 128 + half * 64 + cc * 8) =
              val;
        }
      }
    }
    // every wavefront done with its transposes before any of them starts the next tile, whose slab
    // loads go into this stage (all wavefronts of a tile take this branch: a tile lies in q, k or v)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int row = m0 + wm * TM + j * 32 + l32;
      if (row >= m) continue;
      const int b = row / T, t = row - b * T;
      uint16_t* dst = ep.vo + ((((size_t)b * H + head) * (ep.rows_pad / 64) + t / 64) * 128 + half * 64 + 4 * hh) * 64 +
                      (t & 63);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            dst[(i * 32 + 8 * q + e) * 64] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][4 * q + e]);
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI, int NST = 2, int GRP = kGroupN, int NSW = NST>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_kernel(const uint16_t* __restrict__ a, int lda,
                                                             const uint16_t* __restrict__ w, int ldw,
                                                             uint16_t* __restrict__ c, int ldc, int m_begin,
                                                             int m, int n, int k, EpiArgs ep) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int NR = FM + FN, NMF = FM * FN;             // fragment reads and MFMAs per k-step
  constexpr int AB = BM * KB * 2, BB = BN * KB * 2, SB = AB + BB;  // bytes per slab (one stage)
  // 1 KiB load instructions per wavefront; when the A chunks do not divide among the wavefronts
  // (224-row tiles: 28 chunks), the last wavefronts load the last chunk again (same bytes, same place)
  constexpr int CA = AB / 1024, CB = BB / 1024;
  constexpr int LA = (CA + NW - 1) / NW, LB = CB / NW;
  constexpr int PER = LA + LB;
  static_assert(CA * 1024 == AB && LB * NW * 1024 == BB, "slab / wavefront mismatch");
  static_assert(EPI != kSiluGate || FN % 2 == 0, "the SiLU epilogue pairs gate and up fragments per wavefront");
  // NSW == NST: stage s holds slab s's A tile then its weight tile.  NSW == NST + 1: the weight
  // tiles get a ring of their own, one stage deeper, after the NST A stages, and are loaded one
  // slab further ahead than the A tiles.
  static_assert(NSW == NST || NSW == NST + 1, "weight stages: as many as the A stages, or one more");
  constexpr bool SPLIT = NSW != NST;
  constexpr int INFL = (NST - 2) * PER + (SPLIT ? LB : 0);  // loads a slab wait leaves in flight
  static_assert(NST >= 2 && INFL <= 63, "stages, and the loads a slab wait leaves in flight");
  __shared__ __attribute__((aligned(1024))) char smem[NST * AB + NSW * BB];
  constexpr auto a_base = [](int st) { return (uint32_t)(SPLIT ? st * AB : st * SB); };
  constexpr auto w_base = [](int st) { return (uint32_t)(SPLIT ? NST * AB + st * BB : st * SB + AB); };

  // This launch covers rows [m_begin, m).  Workgroup b computes tiles b, b + G, b + 2G, ... of the
  // launch (G workgroups); the loads run on from one of its tiles into the next, so a tile's first
  // slab is in LDS when the previous tile's epilogue starts.
  const int mt = (m - m_begin + BM - 1) / BM, ntn = n / BN, ntiles = mt * ntn;
  const int G = gridDim.x;
  const int mine = (ntiles - (int)blockIdx.x + G - 1) / G;
  const int nk = k / KB, total = mine * nk;  // slabs this workgroup loads and consumes
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // the operands as buffers (the launcher checks that both fit 32-bit byte offsets)
  const u32x4 ra = buffer_rsrc(a, (uint32_t)((size_t)m * lda * 2));
  const u32x4 rw = buffer_rsrc(w, (uint32_t)((size_t)n * ldw * 2));

  // Load instruction i of wavefront `wave` fills the 1 KiB at (wave + NW*i) of a slab: rows
  // 8*(wave + NW*i) + lane/8, stored slot lane%8, which holds chunk (lane%8) ^ ((row >> 1) & 7).
  // Rows past m are clamped to m - 1; their results are never stored.
  uint32_t ca[LA];  // LDS byte offset of A chunk i of this wavefront
#pragma unroll
  for (int i = 0; i < LA; ++i) ca[i] = 1024u * min(wv + NW * i, CA - 1);
  uint32_t va[LA], vb[LB];  // byte offsets of this lane's 16 bytes of slab 0 of the current tile
  auto aim = [&](int r, bool do_a, bool do_w) {  // point the A (weight) loads at this workgroup's tile r
    int tm, tn;
    tile_of<GRP>(blockIdx.x + r * G, mt, ntn, tm, tn);
    const int m0 = m_begin + tm * BM, n0 = tn * BN;
#pragma unroll
    for (int i = 0; i < LA && do_a; ++i) {
      const int rr = min(wv + NW * i, CA - 1) * 8 + (lane >> 3);
      va[i] = (uint32_t)(((size_t)min(m0 + rr, m - 1) * lda + ((lane & 7) ^ ((rr >> 1) & 7)) * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < LB && do_w; ++i) {
      const int rr = (wave + NW * i) * 8 + (lane >> 3);
      int wrow = n0 + rr;
      if (EPI == kSiluGate) {
        // tile row rr -> wavefront rr / TN, fragment f = (rr % TN) / 32: even f = gate rows, odd f =
        // the up rows of the same outputs
        const int f = (rr % TN) / 32;
        const int zc = tn * (BN / 2) + (rr / TN) * (TN / 2) + (f / 2) * 32 + (rr & 31);
        wrow = ((f & 1) ? n / 2 : 0) + zc;
      }
      vb[i] = (uint32_t)(((size_t)wrow * ldw + ((lane & 7) ^ ((rr >> 1) & 7)) * 8) * 2);
    }
  };
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MOSS_LDS char*)smem;
  int lt = 0, lk = 0, lst = 0;     // the next slab to load: tile, slab within it, stage
  int ltw = 0, lkw = 0, lstw = 0;  // with a weight ring of its own: the next weight slab
  auto issue_one = [&](int q) {  // load instruction q of that slab; the last one moves on
    if constexpr (!SPLIT) {
      const uint32_t base = lds0 + (uint32_t)(lst * SB), koff = (uint32_t)(lk * (KB * 2));
      if (q < LA)
        dma16_buf_so(va[q], ra, koff, base + ca[q]);
      else
        dma16_buf_so(vb[q - LA], rw, koff, base + AB + 1024u * (wv + NW * (q - LA)));
      if (q == PER - 1) {
        lst = lst + 1 == NST ? 0 : lst + 1;
        if (++lk == nk) {
          lk = 0;
          if (++lt < mine) aim(lt, true, true);
        }
      }
    } else {
      if (q < LA) {
        dma16_buf_so(va[q], ra, (uint32_t)(lk * (KB * 2)), lds0 + a_base(lst) + ca[q]);
        if (q == LA - 1) {
          lst = lst + 1 == NST ? 0 : lst + 1;
          if (++lk == nk) {
            lk = 0;
            if (++lt < mine) aim(lt, true, false);
          }
        }
      } else {
        dma16_buf_so(vb[q - LA], rw, (uint32_t)(lkw * (KB * 2)), lds0 + w_base(lstw) + 1024u * (wv + NW * (q - LA)));
        if (q == PER - 1) {
          lstw = lstw + 1 == NSW ? 0 : lstw + 1;
          if (++lkw == nk) {
            lkw = 0;
            if (++ltw < mine) aim(ltw, false, true);
          }
        }
      }
    }
  };
  // Byte offsets of this lane's fragments within a stage.  Fragment j of the A tile (i of the
  // weight tile) covers rows wm*TM + 32j + l32 (wn*TN + 32i + l32); TM and TN are multiples of 16,
  // so a row's chunk swizzle (row >> 1) & 7 is the lane's own, and fragment j sits 32 rows (4 KiB)
  // past fragment 0: one base per k16 step, the 4 KiB steps folded into the reads' offset field.
  static_assert(TM % 16 == 0 && TN % 16 == 0, "fragment blocks share the lane's swizzle");
  constexpr uint32_t FRAG = 32 * KB * 2;  // bytes between consecutive 32-row fragment blocks
  const int swz = (l32 >> 1) & 7;
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    oa[s] = (uint32_t)((wm * TM + l32) * (KB * 2) + ((2 * s + hh) ^ swz) * 16);
    ob[s] = (uint32_t)((wn * TN + l32) * (KB * 2) + ((2 * s + hh) ^ swz) * 16);
  }
  // fragment read x of a k-step, in the order the step's MFMAs first use them (w0 a0 w1 .. a1 ..;
  // the MFMAs run over the weight fragments in the inner loop)
  auto rd_at = [&](const char* sa, const char* sw, uint32_t a_off, uint32_t b_off, int x, bf16x8* fa, bf16x8* fw) {
    if (x == 0)
      fw[0] = *reinterpret_cast<const bf16x8*>(sw + b_off);
    else if (x == 1)
      fa[0] = *reinterpret_cast<const bf16x8*>(sa + a_off);
    else if (x < FN + 1)
      fw[x - 1] = *reinterpret_cast<const bf16x8*>(sw + b_off + (x - 1) * FRAG);
    else
      fa[x - FN] = *reinterpret_cast<const bf16x8*>(sa + a_off + (x - FN) * FRAG);
  };
  auto rd = [&](const char* sa, const char* sw, int s, int x, bf16x8* fa, bf16x8* fw) {
    rd_at(sa, sw, oa[s], ob[s], x, fa, fw);
  };
  // The LDS addresses of k-step 0's fragment 0 reads of the next slab (A and weight), worked out
  // during the current slab's last k-step so that the reads issue straight after the slab barrier.
  int stage = 0;  // g % NST
  int stw = 0;    // g % NSW (the weight stage, with a weight ring of its own)
  auto wstage = [&]() { return SPLIT ? stw : stage; };
  uint32_t nxa = 0, nxb = 0;
  auto set_next = [&](int sa, int sw) {
    nxa = lds0 + a_base(sa) + oa[0];
    nxb = lds0 + w_base(sw) + ob[0];
  };
  auto rd0 = [&](int x, bf16x8* fa, bf16x8* fw) {
    const uint32_t addr = x == 0 ? nxb : x == 1 ? nxa : x < FN + 1 ? nxb + (x - 1) * FRAG : nxa + (x - FN) * FRAG;
    const bf16x8 v = *reinterpret_cast<MOSS_LDS const bf16x8*>((size_t)addr);
    if (x == 0)
      fw[0] = v;
    else if (x == 1)
      fa[0] = v;
    else if (x < FN + 1)
      fw[x - 1] = v;
    else
      fa[x - FN] = v;
  };
  set_next(0, 0);

  // the first NST - 1 slabs (and, with a weight ring of its own, the weight tile of one more);
  // then wait for slab 0 alone
  aim(0, true, true);
#pragma unroll
  for (int sl = 0; sl < NST - 1; ++sl)
    if (sl < total)
#pragma unroll
      for (int q = 0; q < PER; ++q) issue_one(q);
  if constexpr (SPLIT) {
#pragma unroll
    for (int q = LA; q < PER; ++q) issue_one(q);
  }
  if (INFL > 0 && total >= NSW - 1)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(INFL) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

  int g = 0;  // the slab being consumed, counted over this workgroup's tiles
  for (int r = 0; r < mine; ++r) {
    int tm, tn;
    tile_of<GRP>(blockIdx.x + r * G, mt, ntn, tm, tn);
    const int m0 = m_begin + tm * BM, n0 = tn * BN;

    // the tile's first k-step starts its sums from zero (the MFMAs take 0 as the accumulator input,
    // so no registers are cleared per tile): the first slab is a separate copy of the slab body
    f32x16 acc[FN][FM];

    // Scalar loads (kernel arguments the epilogue uses) complete out of order, so while the
    // compiler counts one as possibly in flight it makes every LDS wait a full lgkmcnt(0); waiting
    // for them here, visibly, lets the k-loop's first MFMA wait for its own two fragments only.
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt and expcnt unconstrained
    auto slab = [&](auto first_slab) {
      constexpr bool FIRST = decltype(first_slab)::value;
      // the A tile of slab g + NST - 1 and the weight tile of slab g + NSW - 1 are loaded during
      // steps 0-1, the A loads first.  Past a workgroup's last slab the loads go on without a test
      // (no branch among the MFMAs): they read rows of its last tile again, in bounds, into the
      // stage of a slab already consumed, and the last slabs wait for them.
      const char* cur = smem + a_base(stage);
      const char* curw = smem + w_base(wstage());
      bf16x8 fa[2][FM], fw[2][FN];
#pragma unroll
      for (int x = 0; x < NR; ++x) {
        // in use order, so the first MFMA waits for its own two fragments only
        rd0(x, fa[0], fw[0]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma clang loop unroll(full)
      for (int s = 0; s < 4; ++s) {
#pragma clang loop unroll(full)
        for (int t = 0; t < NMF; ++t) {
          const int j = t / FN, i = t % FN;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[s & 1][i], fa[s & 1][j],
                                                              FIRST && s == 0 ? f32x16{} : acc[i][j], 0, 0, 0);
          // one fragment read of the next k-step after each of the first MFMAs (the rest after the
          // last one when there are more reads than MFMAs), and the next slab's loads spread evenly
          // over the MFMAs of k-steps 0 and 1; nothing moves across these points
          __builtin_amdgcn_sched_barrier(0);
          if (s < 3) {
#pragma unroll
            for (int x = t; x < (t + 1 == NMF ? NR : t + 1); ++x)
              if (x < NR) rd(cur, curw, s + 1, x, fa[(s + 1) & 1], fw[(s + 1) & 1]);
          }
          if (s == 3 && t == 0)
            set_next(stage + 1 == NST ? 0 : stage + 1, SPLIT ? (stw + 1 == NSW ? 0 : stw + 1) : (stage + 1 == NST ? 0 : stage + 1));
          if (s < 2) {
            const int u = s * NMF + t;
#pragma unroll
            for (int q = u * PER / (2 * NMF); q < (u + 1) * PER / (2 * NMF); ++q) issue_one(q);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // slab g + 1 resident and every read of slab g done before the next slab's loads overwrite it.
      // Loads complete in order, so leaving the newest INFL in flight is exact: the (NST - 2) * PER
      // of the slabs after g + 1 and, with a weight ring of its own, the weight loads issued after
      // slab g + 1's A loads; epilogue stores issued in between only make the wait longer.
      if (INFL > 0 && g + NSW - 1 < total)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(INFL) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      stage = stage + 1 == NST ? 0 : stage + 1;
      if constexpr (SPLIT) stw = stw + 1 == NSW ? 0 : stw + 1;
      ++g;
    };
    slab(std::true_type{});  // nk >= 1: the launcher refuses k < 64
    for (int kt = 1; kt < nk; ++kt) slab(std::false_type{});

    if constexpr (EPI == kQkvPack) {
      // the stage of the tile's last slab stays free until the next tile's slab NST - 1 is loaded
      static_assert(!SPLIT, "the q/k epilogue takes a whole stage as its spare");
      char* spare = smem + ((g + NST - 1) % NST) * SB;
      epilogue_qkv<BM, BN, WM, WN>(acc, spare, m0, n0, wave, wm, wn, l32, hh, m, ep);
    } else if constexpr (EPI == kGatedAdd && WM == 1 && WN == 8 && BN == 256 && NST == 2) {
      if (r + 1 == mine)
        epilogue_gated_lds<BM, BN, WM, WN>(acc, smem, m0, n0, wave, l32, hh, m, n, ep);
      else
        epilogue<BM, BN, WM, WN, EPI>(acc, m0, n0, tn, wm, wn, l32, hh, m, n, c, ldc, ep);
    } else {
      epilogue<BM, BN, WM, WN, EPI>(acc, m0, n0, tn, wm, wn, l32, hh, m, n, c, ldc, ep);
    }
  }
}

int cu_count() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

// Tile rounds over the CUs.  Rows past the last whole 256-row tile: when
// that tile is mostly empty and its column tiles would start one more round
// of 256-row tiles, the whole tiles run first and the leftover rows follow as
// 64- or 128-row by 128-column tiles (4 wavefronts each).  Otherwise, for a
// plain store, a last round less than half full is avoided by giving the
// whole rounds the first column tiles and running the rest as 128-row tiles.
template <int EPI>
hipError_t launch(int m, int n, int k, const uint16_t* a, int lda, const uint16_t* w, int ldw, uint16_t* c, int ldc,
                  const EpiArgs& ep, hipStream_t st) {
  // the kernels address both operands through 32-bit buffer byte offsets
  if ((size_t)m * lda * 2 > 0xffffffffu || (size_t)n * ldw * 2 > 0xffffffffu || k <= 0 || k % KB != 0)
    return hipErrorInvalidValue;
  if (n % 256 == 0) {
    const int nt = n / 256, full = m / 256, rem = m % 256, cus = cu_count();
    bool split = false;
    if (full > 0 && rem > 0 && rem <= 128) {
      // a round of tail tiles costs about half a round of whole tiles (64 rows, measured at 4130 rows;
      // 128 rows taken as 0.7): they are few, so each runs at its load latency
      const double tail = rem <= 64 ? 0.55 : 0.7;
      const double whole = std::ceil((double)full * nt / cus), all = std::ceil((double)(full + 1) * nt / cus);
      split = whole + tail * std::ceil((double)nt / cus) < all;
    }
    if (!split && (EPI == kStore || EPI == kQkvPack)) {
      // When the 256 x 256 tiles leave a last round less than half full, the
      // whole rounds take the first column tiles and the remaining columns
      // run as 128-row tiles: one round again, but about half as deep.
      const int mt = (m + 255) / 256, rounds = mt * nt / cus, left = mt * nt % cus;
      const int nt1 = rounds * cus / mt, nt2 = nt - nt1, mt2 = (m + 127) / 128;
      if (rounds >= 1 && left > 0 && 2 * left <= cus && nt1 > 0 && nt2 > 0 && mt2 * nt2 <= cus) {
        hipLaunchKernelGGL((gemm_nt_kernel<256, 256, 2, 4, EPI, 2, kGroupNQkv>), dim3(std::min(mt * nt1, cus)), dim3(512), 0, st, a,
                           lda, w, ldw, c, ldc, 0, m, nt1 * 256, k, ep);
        EpiArgs ep2 = ep;
        ep2.col0 = ep.col0 + nt1 * 256;
        // three stages (144 KiB): one workgroup per tile, each waiting on its loads; a third stage
        // keeps two slabs in flight (QKV's six column tiles at 4130 rows: 55 -> 47 us, same box)
        hipLaunchKernelGGL((gemm_nt_kernel<128, 256, 2, 4, EPI, 3>), dim3(mt2 * nt2), dim3(512), 0, st, a, lda,
                           w + (size_t)nt1 * 256 * ldw, ldw, c ? c + (size_t)nt1 * 256 : c, ldc, 0, m, nt2 * 256, k,
                           ep2);
        return hipGetLastError();
      }
    }
    const int m_main = split ? full * 256 : m;
    if constexpr (EPI == kGatedAdd) {
      // 224-row tiles when they take no more rounds over the CUs than 256-row ones: each CU then
      // does 7/8 of the work (the out and down projections' one part-full round at 4096+34 rows:
      // 204 tiles of 256 rows or 228 of 224 on 256 CUs).  Eight wavefronts of 224 x 32 (8 fragment
      // reads per 7 MFMAs against 6 per 8) keep most of the saving: down 331 -> 318 us; four of
      // 224 x 64 (1 per SIMD) kept less.
      const int t256 = ((m + 255) / 256) * nt, t224 = ((m + 223) / 224) * nt;
      if (!split && (t224 + cus - 1) / cus == (t256 + cus - 1) / cus) {
        hipLaunchKernelGGL((gemm_nt_kernel<224, 256, 1, 8, EPI, 2, kGroupNGated, 3>), dim3(t224), dim3(512), 0, st, a, lda, w, ldw, c,
                           ldc, 0, m, n, k, ep);
        return hipGetLastError();
      }
    }
    // one workgroup per CU, each taking every cus-th tile
    hipLaunchKernelGGL((gemm_nt_kernel<256, 256, 2, 4, EPI, 2, kGroupN, EPI == kQkvPack ? 2 : 3>), dim3(std::min(((m_main + 255) / 256) * nt, cus)),
                       dim3(512), 0, st, a, lda, w, ldw, c, ldc, 0, m_main, n, k, ep);
    if (split) {
      // The tail is bound by reading all of w once: more workgroups, and more slabs in flight per
      // workgroup, stream it faster.  At the 4096+34-row up projection: 64 x 128 tiles (twice the
      // workgroups of 64 x 256) 50 -> 36 us; 64 x 64 tiles of two wavefronts (four times) 39-43 ->
      // 37 us; their ring at four stages instead of two 37 -> 27 us (same box).  The QKV epilogue
      // needs a head's 128 columns in one pair of wavefronts, so it keeps 64 x 128.
      if (rem <= 64) {
        if constexpr (EPI != kQkvPack)
          hipLaunchKernelGGL((gemm_nt_kernel<64, 64, 2, 1, EPI, 4>), dim3(4 * nt), dim3(128), 0, st, a, lda, w, ldw,
                             c, ldc, m_main, m, n, k, ep);
        else
          hipLaunchKernelGGL((gemm_nt_kernel<64, 128, 2, 2, EPI, 4>), dim3(2 * nt), dim3(256), 0, st, a, lda, w, ldw,
                             c, ldc, m_main, m, n, k, ep);
      } else
        hipLaunchKernelGGL((gemm_nt_kernel<128, 128, 2, 2, EPI, 3>), dim3(2 * nt), dim3(256), 0, st, a, lda, w, ldw,
                           c, ldc, m_main, m, n, k, ep);
    }
  } else {
    hipLaunchKernelGGL((gemm_nt_kernel<256, 128, 4, 2, EPI>), dim3(((m + 255) / 256) * (n / 128)), dim3(512), 0, st,
                       a, lda, w, ldw, c, ldc, 0, m, n, k, ep);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nt(int m, int n, int k, const uint16_t* a, int lda, const uint16_t* w, int ldw,
                          uint16_t* c, int ldc, hipStream_t st) {
  return launch<kStore>(m, n, k, a, lda, w, ldw, c, ldc, EpiArgs{}, st);
}

hipError_t launch_gemm_qkv_pack(int batch, int rows, int n_heads, float eps, const uint16_t* a, const uint16_t* w_qkv,
                                const uint16_t* q_gain, const uint16_t* k_gain, const float* rope_pp, uint16_t* q,
                                uint16_t* k, uint16_t* v, hipStream_t st) {
  const int d = n_heads * 128;
  EpiArgs ep{};
  ep.rows_per_item = rows;
  ep.q_gain = q_gain;
  ep.k_gain = k_gain;
  ep.rope_pp = rope_pp;
  ep.qo = q;
  ep.ko = k;
  ep.vo = v;
  ep.rows_pad = packed_rows(rows);
  ep.n_heads = n_heads;
  ep.eps = eps;
  ep.col0 = 0;
  return launch<kQkvPack>(batch * rows, 3 * d, d, a, d, w_qkv, d, nullptr, 3 * d, ep, st);
}

hipError_t launch_gemm_silu(int m, int f, int k, const uint16_t* a, int lda, const uint16_t* w_up, int ldw,
                            uint16_t* z, int ldz, hipStream_t st) {
  return launch<kSiluGate>(m, 2 * f, k, a, lda, w_up, ldw, z, ldz, EpiArgs{}, st);
}

hipError_t launch_gemm_gated_add(int m, int n, int k, const uint16_t* a, int lda, const uint16_t* w, int ldw,
                                 float* h, const float* gate, int gate_stride, int rows_per_item, uint16_t* out16,
                                 hipStream_t st) {
  const EpiArgs ep{h, gate, gate_stride, rows_per_item, out16};
  return launch<kGatedAdd>(m, n, k, a, lda, w, ldw, nullptr, n, ep, st);
}
