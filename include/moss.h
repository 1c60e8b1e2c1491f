/*
 * moss.h - C ABI of libmoss.so: the forward of a MOSS-Image-style diffusion
 * transformer (DiT) denoiser block, and of a stack of such blocks, on AMD
 * Instinct MI355X (gfx950).
 *
 * The block is the one listed under "What it adds" on the MOSS-Image
 * transformer page (TensorFold PR #1528, "MOSS-Image's transformer on the CUDA
 * runtime"): an adaLN-modulated RMSNorm, a QKV projection, per-head q/k
 * RMSNorm with rotary embedding into packed rows, full (non-causal) attention
 * at head dim 128 over text + image rows, an output projection, a gated
 * residual add, a second modulated RMSNorm, a SiLU-gated MLP, and a second
 * gated add.  Weights and activations are bf16; sums, norms and the softmax
 * are fp32 (same section, precision bullet).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 *  - Every tensor pointer is a device pointer owned by the caller, unless the
 *    comment says "host".  The library never allocates device memory, never
 *    copies weights and keeps no state between calls apart from a per-device
 *    capability cache and the optional timing probe.
 *  - Every tensor pointer must be 16-byte aligned; row-major, dense.
 *  - Calls are asynchronous: they validate, enqueue kernels on `stream` and
 *    return.  The caller synchronises.  Calls on different streams are safe
 *    when each has its own workspace and outputs.
 *  - All arguments are validated before any HIP call.  No exception crosses
 *    the ABI and no environment variable is read.  On error nothing is
 *    enqueued (for MOSS_EHIP, the kernels enqueued before the failing
 *    launch stay enqueued).
 *  - Results are deterministic: the same inputs give the same bytes on every
 *    call (no atomics, no split reductions whose order varies).
 */
#ifndef MOSS_H
#define MOSS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
#define MOSS_OK 0
#define MOSS_EINVAL 1     /* a bad argument: null pointer, bad shape, misalignment, bad txt_len, eps <= 0 */
#define MOSS_EALIAS 2     /* an output overlaps an input or the workspace, or an input lies in the workspace */
#define MOSS_EWORKSPACE 3 /* workspace null or smaller than moss_workspace_bytes() */
#define MOSS_EDEVICE 4    /* no HIP device, or the device is not gfx950 */
#define MOSS_EHIP 5       /* a HIP launch failed; moss_status_string() holds the text */

/* Limits checked by validation. */
#define MOSS_HEAD_DIM 128
#define MOSS_MAX_BATCH 16
#define MOSS_MAX_DMODEL 8192
#define MOSS_MAX_ROWS 65536 /* n_txt + n_img per item */

/* Geometry of one call.  Rows of an item are its n_txt text rows followed by
 * its n_img image rows (T = n_txt + n_img).  head_dim must be 128,
 * d_model = n_heads * 128 (<= MOSS_MAX_DMODEL), mlp_inner a positive multiple
 * of 128, eps > 0 (added to the mean square inside the square root). */
typedef struct {
  int32_t batch, n_img, n_txt, d_model, n_heads, head_dim, mlp_inner;
  float eps;
} moss_dims;

/* One block's weights (device, bf16 bits).  Projections are row-major
 * [out, in], i.e. y = x W^T:
 *   w_mod  [6D, D]  adaLN: rows give shift1, scale1, gate1, shift2, scale2, gate2
 *   w_qkv  [3D, D]  q rows, then k rows, then v rows; head h owns 128 rows of each
 *   q_gain [128], k_gain [128]  RMSNorm gains of q and k, shared by the heads
 *   w_out  [D, D]
 *   w_up   [2F, D]  gate half (rows 0..F-1) then up half
 *   w_down [D, F]                                                            */
typedef struct {
  const uint16_t *w_mod, *w_qkv, *q_gain, *k_gain, *w_out, *w_up, *w_down;
} moss_block_weights;

/* Text for a status code (for MOSS_EHIP, the failing HIP call's message from
 * this thread's last failure).  Never NULL. */
const char* moss_status_string(int status);

/* MOSS_OK if `hip_device` exists and is gfx950 (MI355X class), else
 * MOSS_EDEVICE.  The MOSS-Image transformer page's model load likewise
 * refuses GPUs it was not checked on ("What it adds"). Makes HIP calls. */
int moss_device_check(int hip_device);

/* Bytes of device workspace one moss_block_forward / moss_stack_forward call
 * with these dims needs (n_blocks >= 1; 1 for moss_block_forward; every
 * block's modulation is computed up front, so it grows by 24 B D per block).
 * Returns 0 when the dims are invalid.  One plan serves every call whose dims
 * and block count are no larger, as the CUDA port page's `fit` plans one
 * scratch for every geometry (TensorFold PR #2281, "What this changes"). */
size_t moss_workspace_bytes(const moss_dims* dims, int32_t n_blocks);

/* Fill the 2D axial rotary tables rope[2][T][64] (fp32, device): cos, then
 * sin, one entry per row, in row order (n_txt text rows, then the image rows
 * y-major: row n_txt + y*grid_w + x).  Text rows get angle 0.  Image row
 * (y, x) gets angle y*w_p on pairs p < 32 and x*w_(p-32) on pairs p >= 32,
 * w_i = theta^(-i/32).  Angles and cos/sin are evaluated in fp64 and rounded
 * to fp32.  The rotary tables are shared config code on the MOSS-Image
 * transformer page ("What it adds").  MOSS_EINVAL on non-positive grid sides,
 * negative n_txt, more than MOSS_MAX_ROWS rows, theta <= 1, or a bad pointer. */
int moss_rope_build(int32_t n_txt, int32_t grid_h, int32_t grid_w, float theta, float* rope,
                    hipStream_t stream);

/* One block forward.
 *   x       [B, n_img, D]  image rows (bf16)
 *   txt     [B, n_txt, D]  text rows (bf16); rows at or past txt_len[b] are never read
 *   txt_len host [B] valid text rows per item, 0 <= txt_len[b] <= n_txt and
 *           txt_len[b] + n_img >= 1; NULL means all n_txt valid.  Text rows
 *           past txt_len are padding: they enter the block as zero rows, are
 *           computed as queries like any row, and are masked as keys.
 *   cond    [B, D]  conditioning vector (bf16), e.g. the timestep embedding
 *   w       host struct of device weight pointers (see moss_block_weights)
 *   rope    [2][T][64] fp32 tables as moss_rope_build writes them
 *   out     [B, T, D] block output (bf16), text rows first; must not overlap
 *           any input or the workspace
 *   workspace, ws_bytes: device scratch of at least moss_workspace_bytes(dims, 1);
 *           no input or weight may lie in it (the call overwrites it while the
 *           inputs are still needed): MOSS_EALIAS
 * Computes, per item, h0 = [txt; x], mod = W_mod SiLU(cond), a = RMSNorm(h0)
 * (1 + scale1) + shift1, qkv = a W_qkv^T, per head q/k RMSNorm x gain and
 * rotary, O = softmax(q k^T / sqrt(128) + mask) v, h1 = h0 + gate1 (O W_out^T),
 * m = RMSNorm(h1) (1 + scale2) + shift2, u = m W_up^T, z = SiLU(u_gate) u_up,
 * out = h1 + gate2 (z W_down^T).  Each stored intermediate (a, qkv, q/k/v,
 * O, m, z) is rounded to bf16; the modulation vector is fp32; the projection
 * outputs feeding the gated adds and the SiLU gate stay fp32 (they are
 * consumed in the GEMM epilogues); the residual stream h0 -> h1 -> out is a
 * running sum kept in fp32 and rounded once, into out. */
int moss_block_forward(const moss_dims* dims, const uint16_t* x, const uint16_t* txt,
                       const int32_t* txt_len, const uint16_t* cond, const moss_block_weights* w,
                       const float* rope, uint16_t* out, void* workspace, size_t ws_bytes,
                       hipStream_t stream);

/* moss_block_forward for callers that cannot allocate or be handed device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and results (byte for byte) as
 * moss_block_forward, without the workspace: the call uses a scratch array of
 * MOSS_NOALLOC_SCRATCH_BYTES (256 MiB) that the library holds in each GPU's
 * memory from its load to the end of the process, and calls no hipMalloc or
 * hipFree.  A geometry whose workspace (moss_workspace_bytes(dims, 1)) exceeds
 * that returns MOSS_EWORKSPACE: one block at up to 4096 + 34 rows at batch 1
 * (4188 rows: 248 MiB) or about 2 x 2100 rows at D = 3072 fits.  Every call on
 * one GPU shares that GPU's array, which keeps the last call's contents: calls
 * that overlap on one GPU (other streams, other threads) race and must not be
 * issued.  The call writes every scratch byte it reads first, so nothing needs
 * clearing between calls.  Other codes as moss_block_forward. */
#define MOSS_NOALLOC_SCRATCH_BYTES (256u << 20)
int moss_block_forward_noalloc(const moss_dims* dims, const uint16_t* x, const uint16_t* txt,
                               const int32_t* txt_len, const uint16_t* cond, const moss_block_weights* w,
                               const float* rope, uint16_t* out, hipStream_t stream);
/* The scratch limit above, in bytes. */
size_t moss_noalloc_scratch_bytes(void);

/* n_blocks block forwards in sequence (blocks: host array of n_blocks weight
 * structs), each on the previous block's output, with the same cond, rope and
 * txt_len.  Arguments otherwise as moss_block_forward; `out` holds the
 * final output; the residual stream between blocks stays in fp32 in the
 * workspace. */
int moss_stack_forward(const moss_dims* dims, int32_t n_blocks, const uint16_t* x, const uint16_t* txt,
                       const int32_t* txt_len, const uint16_t* cond, const moss_block_weights* blocks,
                       const float* rope, uint16_t* out, void* workspace, size_t ws_bytes,
                       hipStream_t stream);

/* moss_stack_forward with some blocks not applied to some items: skip is a
 * host array [n_blocks][batch] (row i for block i); a nonzero skip[i][b]
 * leaves item b's residual unchanged through block i while the other items
 * run it (the CUDA port page's guidance pass skips one block on one branch,
 * TensorFold PR #2281, "What this changes").  When the items that run a
 * block are a contiguous run (in a guidance pair, always), the block runs on
 * their rows alone and costs nothing for the others; a block no item runs
 * launches nothing; other patterns run every item with the skipping items'
 * two gates zeroed, so their residual still passes through exactly.  An item
 * that skips the last block gets its residual, rounded to bf16, in `out`.
 * skip == NULL is moss_stack_forward.  Other arguments, ownership and errors
 * as moss_stack_forward. */
int moss_stack_forward_skip(const moss_dims* dims, int32_t n_blocks, const uint16_t* x, const uint16_t* txt,
                            const int32_t* txt_len, const uint16_t* cond, const moss_block_weights* blocks,
                            const uint8_t* skip, const float* rope, uint16_t* out, void* workspace,
                            size_t ws_bytes, hipStream_t stream);

/* One sampler step on a latent (the CUDA port page, TensorFold PR #2281,
 * "What this changes": classifier-free guidance with an empty negative, and
 * guidance 1 skipping the negative pass; the transformer page, "Measured":
 * Euler steps at guidance 3):
 *   x_out = x_in + dsigma * (v_neg + guidance * (v_pos - v_neg)),
 * or x_out = x_in + dsigma * v_pos when v_neg is NULL (guidance must then be
 * 1).  v_pos, v_neg: [rows, width] bf16 velocities (device); x_in, x_out:
 * [rows, width] fp32 latents (device; x_out == x_in updates in place, any
 * other overlap is refused).  dsigma = sigma_next - sigma_now.  Arithmetic in
 * fp32.  width % 8 == 0, pointers 16-byte aligned.  MOSS_EINVAL on bad sizes,
 * pointers or non-finite guidance/dsigma, or a NULL v_neg with guidance != 1;
 * MOSS_EALIAS when x_out overlaps a velocity or partly overlaps x_in.
 * rows == 0 is a no-op. */
int moss_guidance_euler(int32_t rows, int32_t width, const uint16_t* v_pos, const uint16_t* v_neg, float guidance,
                        float dsigma, const float* x_in, float* x_out, hipStream_t stream);

/* ---- the whole denoiser forward (the ends around the stack) ------------- */

/* Weights of the denoiser's ends, bf16 bits, row-major [out, in] (device;
 * caller-owned).  The pages name these parts and sizes, not their formulas
 * (the MOSS-Image transformer page, TensorFold PR #1528, "What it adds": the
 * timestep's modulation; the encoder page, PR #1512: hidden size 4096; the
 * CUDA port page, PR #2281: latents of 128 values per row); each takes the
 * standard DiT form without biases. */
typedef struct {
  const uint16_t* w_t1;    /* [D, 256]: timestep features -> hidden */
  const uint16_t* w_t2;    /* [D, D]: SiLU(hidden) -> cond */
  const uint16_t* w_txt;   /* [D, enc_dim]: prompt rows -> model width */
  const uint16_t* w_in;    /* [D, 128]: latent rows -> model width */
  const uint16_t* w_fmod;  /* [2D, D]: SiLU(cond) -> final (shift, scale) */
  const uint16_t* w_final; /* [128, D]: normed image rows -> velocity */
  int32_t enc_dim;         /* prompt row width (4096 for the released encoder); % 64 == 0, <= 16384 */
} moss_denoiser_weights;

/* Workspace bytes for moss_denoiser_forward with these dims (the stack's plan
 * plus the ends' scratch); 0 when the dims are invalid or n_img < 1. */
size_t moss_denoiser_workspace_bytes(const moss_dims* dims, int32_t n_blocks);

/* One denoiser forward: velocity = f(latent, prompt rows, t).
 *   features = cos(t w_i), i < 128, then sin(t w_i), w_i = 10000^(-i/128);
 *   cond = bf16(W_t2 SiLU(W_t1 features));
 *   txt = bf16(enc W_txt^T), x = bf16(latent W_in^T);
 *   h = the block stack on (x, txt, cond), kept in fp32 (skip as in
 *       moss_stack_forward_skip, may be NULL);
 *   velocity = bf16(bf16(modRMSNorm(h_image_rows; shift, scale)) W_final^T),
 *       (shift, scale) = W_fmod SiLU(cond).
 * latent [B, n_img, 128] bf16, enc [B, n_txt, enc_dim] bf16 (rows at or past
 * txt_len[b] are never read; NULL when n_txt == 0), t host [B] (finite; the
 * pipeline's timestep scale, e.g. 1000 sigma), velocity [B, n_img, 128] bf16,
 * all device pointers 16-byte aligned.  rope, txt_len, blocks and the error
 * codes as moss_stack_forward; velocity must not overlap any input, weight
 * or the workspace, and no input or weight may lie in the workspace
 * (MOSS_EALIAS); n_img >= 1. */
int moss_denoiser_forward(const moss_dims* dims, int32_t n_blocks, const uint16_t* latent, const uint16_t* enc,
                          const int32_t* txt_len, const float* t, const moss_denoiser_weights* ends,
                          const moss_block_weights* blocks, const uint8_t* skip, const float* rope,
                          uint16_t* velocity, void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- single-step entry points (same conventions; used by the tests) ----- */

/* Packed attention layouts written by moss_k_qk_norm_rope_pack and
 * moss_k_gemm_qkv_pack and read by
 * moss_k_attention, with T_pad = moss_packed_rows(T) (T rounded up to 128):
 *   Q, K: [B, H, T_pad, 128] bf16; rows T..T_pad-1 are zero.
 *   V:    [B, H, T_pad/64, 128, 64] bf16: per 64-key tile, V transposed
 *         (dim-major) with the keys in order; keys T..T_pad-1 are zero. */
int32_t moss_packed_rows(int32_t rows);

/* a0: out[b, r] = r < n_txt ? (r < txt_len[b] ? txt[b, r] : 0) : x[b, r - n_txt];
 * x and txt bf16, out [B, T, D] fp32 (the residual stream the block keeps in
 * fp32 between its gated adds).  txt_len host or NULL. */
int moss_k_join_rows(int32_t batch, int32_t n_txt, int32_t n_img, int32_t d_model, const uint16_t* x,
                     const uint16_t* txt, const int32_t* txt_len, float* out, hipStream_t stream);

/* a1: mod[b, :] = W_mod SiLU(cond[b, :]) in fp32; cond [B, D], w_mod [6D, D],
 * mod [B, 6D] fp32.  Needs 4*B*D bytes of workspace for SiLU(cond). */
int moss_k_adaln_gemv(int32_t batch, int32_t d_model, const uint16_t* cond, const uint16_t* w_mod,
                      float* mod, void* workspace, size_t ws_bytes, hipStream_t stream);

/* a2/a8: out[b, r, :] = h[b, r, :] / sqrt(mean(h^2) + eps) * (1 + scale[b, :]) + shift[b, :];
 * h [B, rows, D] fp32 residual, out [B, rows, D] bf16; shift and scale fp32
 * with item stride mod_stride floats (shift[b] at shift + b * mod_stride).
 * The modulated RMSNorm kernel of the MOSS-Image transformer page ("What it
 * adds"). */
int moss_k_mod_rmsnorm(int32_t batch, int32_t rows, int32_t d_model, float eps, const float* h,
                       const float* shift, const float* scale, int32_t mod_stride, uint16_t* out,
                       hipStream_t stream);

/* a3/a6/a9/a11: c[m, n] = sum_k a[m, k] w[n, k] (fp32 sums, bf16 result).
 * a [M, K] with row stride lda, w [N, K] with row stride ldw, c [M, N] with
 * row stride ldc (elements).  N and K multiples of 128; strides multiples of
 * 8.  The bf16 GEMM projections of the MOSS-Image transformer page ("What it
 * adds"). */
int moss_k_gemm_nt(int32_t m, int32_t n, int32_t k, const uint16_t* a, int32_t lda, const uint16_t* w,
                   int32_t ldw, uint16_t* c, int32_t ldc, hipStream_t stream);

/* a3 + a4 as the block runs them: the QKV projection of a [B*T, D] (bf16,
 * row stride D) by w_qkv [3D, D] with a4 applied to its fp32 sums after one
 * bf16 rounding (the value the projection would store): q and k per row and
 * head RMS-normed over the 128 dims, times q_gain / k_gain, rotated by rope;
 * written packed as described above into q, k and v, pad rows zeroed.  D =
 * 128 n_heads.  The bf16 GEMM and the "q/k norm and rotary into packed rows"
 * kernel of the MOSS-Image transformer page ("What it adds"), fused so the
 * qkv rows never reach memory.  Needs 512 * moss_packed_rows(rows) bytes of
 * workspace (the rotary table re-laid for the epilogue's loads), else
 * MOSS_EWORKSPACE; MOSS_EINVAL / MOSS_EALIAS as moss_k_qk_norm_rope_pack,
 * the workspace included. */
int moss_k_gemm_qkv_pack(int32_t batch, int32_t rows, int32_t n_heads, float eps, const uint16_t* a,
                         const uint16_t* w_qkv, const uint16_t* q_gain, const uint16_t* k_gain, const float* rope,
                         uint16_t* q, uint16_t* k, uint16_t* v, void* workspace, size_t ws_bytes,
                         hipStream_t stream);

/* a4: from qkv [B, T, 3D] (bf16), per row and head: q_hat = rotary(RMSNorm(q) * q_gain),
 * k_hat likewise with k_gain, v unchanged; written packed as described above
 * into q, k, v.  rope as moss_rope_build writes it.  The "q/k norm and rotary
 * into packed rows" kernel of the MOSS-Image transformer page ("What it adds"). */
int moss_k_qk_norm_rope_pack(int32_t batch, int32_t rows, int32_t n_heads, float eps, const uint16_t* qkv,
                             const uint16_t* q_gain, const uint16_t* k_gain, const float* rope,
                             uint16_t* q, uint16_t* k, uint16_t* v, hipStream_t stream);

/* a5: o[b, t, h*128 + d] = sum_j softmax_j(q_t . k_j / sqrt(128)) v_j[d] over the
 * valid keys j of item b (all rows except text rows txt_len[b] <= j < n_txt),
 * non-causal; q, k, v packed as above; o [B, T, H*128] bf16.  Softmax in
 * fp32, probabilities rounded to bf16 for the product with v.  The head-128
 * full attention of the MOSS-Image transformer page ("What it adds", "Shared
 * code").  txt_len host or NULL. */
int moss_k_attention(int32_t batch, int32_t n_heads, int32_t rows, int32_t n_txt, const int32_t* txt_len,
                     const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                     hipStream_t stream);

/* a9 + a10 as the block runs them: z[r, j] = SiLU((a w_up^T)[r, j]) * (a w_up^T)[r, F + j],
 * a [m, k] (row stride lda), w_up [2F, k] gate rows then up rows (row stride
 * ldw), z [m, F] bf16 (row stride ldz); fp32 sums and SiLU, one bf16
 * rounding.  mlp_inner and k multiples of 128.  The bf16 GEMM and SiLU
 * kernels of the MOSS-Image transformer page ("What it adds"), fused so the
 * 2F-wide product never reaches memory. */
int moss_k_gemm_silu(int32_t m, int32_t mlp_inner, int32_t k, const uint16_t* a, int32_t lda, const uint16_t* w_up,
                     int32_t ldw, uint16_t* z, int32_t ldz, hipStream_t stream);

/* a6 + a7 and a11 + a12 as the block runs them: h[r, :] += gate[b, :] * (a w^T)[r, :]
 * with b = r / rows_per_item, on the fp32 residual h [m, n] (row stride n);
 * a [m, k] (row stride lda), w [n, k] (row stride ldw), gate fp32 with item
 * stride gate_stride floats.  With out not NULL the sum is rounded to bf16
 * into out [m, n] and h is left unchanged.  n and k multiples of 128; m a
 * multiple of rows_per_item, with at most MOSS_MAX_BATCH items.  The GEMM and
 * gated-add kernels of the MOSS-Image transformer page ("What it adds"),
 * fused so the projection output never reaches memory. */
int moss_k_gemm_gated_add(int32_t m, int32_t n, int32_t k, const uint16_t* a, int32_t lda, const uint16_t* w,
                          int32_t ldw, float* h, const float* gate, int32_t gate_stride, int32_t rows_per_item,
                          uint16_t* out, hipStream_t stream);

/* a10: z[r, c] = SiLU(u[r, c]) * u[r, F + c] for u [R, 2F], z [R, F] (bf16,
 * fp32 arithmetic).  The SiLU kernel of the MOSS-Image transformer page
 * ("What it adds"). */
int moss_k_silu_mul(int32_t rows, int32_t mlp_inner, const uint16_t* u, uint16_t* z, hipStream_t stream);

/* a7/a12: h[b, r, :] + gate[b, :] * y[b, r, :] on the fp32 residual h, with
 * y bf16 and gate fp32 (item stride gate_stride floats).  With out NULL the
 * sum replaces h in place; otherwise it is rounded to bf16 into out [B, rows,
 * D] and h is left unchanged (the last add of a call).  The gated add kernel
 * of the MOSS-Image transformer page ("What it adds"); the residual is a
 * running sum, kept in fp32 under the page's fp32-sums policy. */
int moss_k_gated_add(int32_t batch, int32_t rows, int32_t d_model, float* h, const float* gate,
                     int32_t gate_stride, const uint16_t* y, uint16_t* out, hipStream_t stream);

/* ---- timing probe -------------------------------------------------------- */
/* Step identifiers for the probe (the launches of moss_block_forward /
 * moss_stack_forward, in order).  The gated adds and the SiLU gate run in the
 * epilogues of the out, down and up projections: MOSS_STEP_OUT, _UP and _DOWN
 * time the fused launches, and MOSS_STEP_GATE1, _SILU and _GATE2 record
 * nothing.  The q/k norm, rotary and packing run in the QKV projection's
 * epilogue: MOSS_STEP_QKV times the fused launch and MOSS_STEP_QKNORM records
 * nothing.  The row join runs in one pass with the first block's first norm:
 * MOSS_STEP_JOIN times that pass, and MOSS_STEP_NORM1 the first norms of the
 * later blocks of a stack. */
#define MOSS_STEP_JOIN 0
#define MOSS_STEP_ADALN 1
#define MOSS_STEP_NORM1 2
#define MOSS_STEP_QKV 3
#define MOSS_STEP_QKNORM 4
#define MOSS_STEP_ATTN 5
#define MOSS_STEP_OUT 6
#define MOSS_STEP_GATE1 7
#define MOSS_STEP_NORM2 8
#define MOSS_STEP_UP 9
#define MOSS_STEP_SILU 10
#define MOSS_STEP_DOWN 11
#define MOSS_STEP_GATE2 12
#define MOSS_NUM_STEPS 13

/* Arm the probe: from the next launch of step `step` by moss_block_forward /
 * moss_stack_forward (and, for MOSS_STEP_ADALN, the GEMV launch of
 * moss_k_adaln_gemv; any stream, this process) on, launches 0, every,
 * 2 every, ... of that step, up to `max_launches` of them, are bracketed by
 * HIP events recorded on the launch stream (timing-only events: no
 * system-scope fence; each record still takes a few microseconds of stream
 * time, which `every` spreads out).  Replaces any earlier arming.
 * MOSS_EINVAL for a bad step, max_launches outside [1, 4096] or every < 1;
 * MOSS_EHIP if events cannot be created. */
int moss_probe_arm(int32_t step, int32_t max_launches, int32_t every);

/* Disarm, wait for the recorded events and write the duration in ms of each
 * bracketed launch (up to max_out) into ms (host).  Returns the number of
 * launches recorded (>= 0), or -MOSS_EHIP / -MOSS_EINVAL. */
int32_t moss_probe_collect(float* ms, int32_t max_out);

#ifdef __cplusplus
}
#endif

#endif /* MOSS_H */
