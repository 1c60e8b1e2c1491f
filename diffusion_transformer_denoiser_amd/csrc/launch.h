// Host-side launchers of the gfx950 kernels (one per step of the block).
// Shapes are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct ItemLens;
struct ItemTimes;

hipError_t launch_join_rows(const uint16_t* x, const uint16_t* txt, const ItemLens& lens, float* out, int batch,
                            int n_txt, int n_img, int d, hipStream_t st);
hipError_t launch_silu_cond(const uint16_t* cond, float* s, int batch, int d, hipStream_t st);
// mod = W_mod s per item; items whose bit is set in skip_items get zero gate1 and gate2.
hipError_t launch_adaln_gemv(const float* s, const uint16_t* w_mod, float* mod, int batch, int d, unsigned skip_items,
                             hipStream_t st);
// The modulations of n blocks in as few launches as possible: mod [n][batch][6 d] fp32, block i from
// w_mods[i] with the gates of the items in skip[i] zeroed.
hipError_t launch_adaln_gemv_many(const float* s, const uint16_t* const* w_mods, const unsigned* skip, int n,
                                  float* mod, int batch, int d, hipStream_t st);
// join_rows into h (fp32) and the first modulated RMSNorm into out (bf16) in one pass.
hipError_t launch_join_mod_rmsnorm(const uint16_t* x, const uint16_t* txt, const ItemLens& lens, const float* shift,
                                   const float* scale, int mod_stride, float* h, uint16_t* out, int batch, int n_txt,
                                   int n_img, int d, float eps, hipStream_t st);
hipError_t launch_mod_rmsnorm(const float* h, const float* shift, const float* scale, int mod_stride,
                              uint16_t* out, int batch, int rows, int d, float eps, hipStream_t st);
// h (fp32) + gate * y: in place when out16 is null, else into out16 (bf16) with h unchanged.
hipError_t launch_gated_add(float* h, const float* gate, int gate_stride, const uint16_t* y, uint16_t* out16,
                            int batch, int rows, int d, hipStream_t st);
hipError_t launch_silu_mul(const uint16_t* u, uint16_t* z, int rows, int f, hipStream_t st);
hipError_t launch_rope_build(int n_txt, int grid_h, int grid_w, float theta, float* rope, hipStream_t st);
// x_out = x_in + dsigma * (v_neg + g (v_pos - v_neg)), or x_in + dsigma * v_pos without v_neg; width % 8 == 0.
hipError_t launch_guidance_euler(int rows, int width, const uint16_t* v_pos, const uint16_t* v_neg, float g,
                                 float dsigma, const float* x_in, float* x_out, hipStream_t st);

// c[m, n] = sum_k a[m, k] w[n, k]; n % 128 == 0, k % 64 == 0, strides % 8 == 0.
hipError_t launch_gemm_nt(int m, int n, int k, const uint16_t* a, int lda, const uint16_t* w, int ldw,
                          uint16_t* c, int ldc, hipStream_t st);

// z[m, f] = SiLU(a w_up[j]^T) * (a w_up[f + j]^T) for w_up = [gate rows; up rows] [2f, k].
// f % 128 == 0 (and 2f % 256 == 0 for the 256-wide tiles the pairing needs).
hipError_t launch_gemm_silu(int m, int f, int k, const uint16_t* a, int lda, const uint16_t* w_up, int ldw,
                            uint16_t* z, int ldz, hipStream_t st);
// h[r, :] += gate[r / rows_per_item, :] * (a w^T)[r, :] on the fp32 residual h [m, n];
// with out16 set, out16 = bf16(h + gate * a w^T) and h is left unchanged.
hipError_t launch_gemm_gated_add(int m, int n, int k, const uint16_t* a, int lda, const uint16_t* w, int ldw,
                                 float* h, const float* gate, int gate_stride, int rows_per_item, uint16_t* out16,
                                 hipStream_t st);

// Rows of the packed attention layouts: rows rounded up to a multiple of 128.
inline int packed_rows(int rows) { return (rows + 127) / 128 * 128; }

// The rotary table [2][rows][64] re-laid as pairs of pairs: rope_pp[pp][t][4] = {rope[0][t][2 pp],
// rope[0][t][2 pp + 1], rope[1][t][2 pp], rope[1][t][2 pp + 1]} (cos, cos, sin, sin; 32 pp, t < rows,
// row stride packed_rows(rows)); 512 packed_rows(rows) bytes.
hipError_t launch_rope_pairs(const float* rope, int rows, float* rope_pp, hipStream_t st);
// The QKV projection of a [batch * rows, 128 n_heads] with a4 in its epilogue: packed Q and K
// [B, H, T_pad, 128] (normed, gained, rotated with rope_pp from launch_rope_pairs) and V^T
// [B, H, T_pad/64, 128, 64]; pad rows untouched.
hipError_t launch_gemm_qkv_pack(int batch, int rows, int n_heads, float eps, const uint16_t* a, const uint16_t* w_qkv,
                                const uint16_t* q_gain, const uint16_t* k_gain, const float* rope_pp, uint16_t* q,
                                uint16_t* k, uint16_t* v, hipStream_t st);
// Once per call, one launch: s = SiLU(cond) (n_cond values), rope_pp as launch_rope_pairs, and
// the pad rows zeroed as launch_zero_packed_pads.
hipError_t launch_call_prologue(const uint16_t* cond, float* s, int n_cond, const float* rope, int batch, int rows,
                                int n_heads, float* rope_pp, uint16_t* q, uint16_t* k, uint16_t* v, hipStream_t st);
// Zero the pad rows T..T_pad-1 of packed Q and K and the pad keys of V^T.
hipError_t launch_zero_packed_pads(int batch, int rows, int n_heads, uint16_t* q, uint16_t* k, uint16_t* v,
                                   hipStream_t st);
hipError_t launch_qk_norm_rope_pack(int batch, int rows, int n_heads, float eps, const uint16_t* qkv,
                                    const uint16_t* q_gain, const uint16_t* k_gain, const float* rope,
                                    uint16_t* q, uint16_t* k, uint16_t* v, hipStream_t st);
hipError_t launch_attention(int batch, int n_heads, int rows, int n_txt, const ItemLens& lens, const uint16_t* q,
                            const uint16_t* k, const uint16_t* v, uint16_t* o, hipStream_t st);

// The denoiser's ends: y[b, :n_out] = W x[b] (W [n_out, d_in] bf16, x fp32, d_in % 8 == 0);
// 256 sinusoidal timestep features per item; SiLU in fp32 (in place allowed); fp32 -> bf16.
hipError_t launch_gemv(const float* x, const uint16_t* w, float* y, int batch, int d_in, int n_out, hipStream_t st);
hipError_t launch_timestep_features(const ItemTimes& ts, float* f, int batch, hipStream_t st);
hipError_t launch_silu_f32(const float* x, float* y, int n, hipStream_t st);
hipError_t launch_round_bf16(const float* x, uint16_t* y, int n, hipStream_t st);
