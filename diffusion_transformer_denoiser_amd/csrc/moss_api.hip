// The C ABI of libmoss.so (declared in include/moss.h): argument validation,
// workspace planning, the launch sequence of one block and of a stack, status
// strings and the timing probe.  No function here allocates device memory.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "launch.h"
#include "moss.h"

namespace {

thread_local std::string g_hip_error;

int hip_fail(hipError_t e, const char* what) {
  char buf[256];
  snprintf(buf, sizeof(buf), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  g_hip_error = buf;
  return MOSS_EHIP;
}

#define MOSS_TRY(expr, what)                  \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ---- geometry ----------------------------------------------------------------
bool dims_ok(const moss_dims* d) {
  if (!d) return false;
  if (d->batch < 1 || d->batch > MOSS_MAX_BATCH) return false;
  if (d->n_img < 0 || d->n_txt < 0) return false;
  const long t = (long)d->n_txt + d->n_img;
  if (t < 1 || t > MOSS_MAX_ROWS) return false;
  if (d->head_dim != MOSS_HEAD_DIM || d->n_heads < 1) return false;
  if ((long)d->d_model != (long)d->n_heads * MOSS_HEAD_DIM || d->d_model > MOSS_MAX_DMODEL) return false;
  if (d->mlp_inner < 128 || d->mlp_inner % 128 != 0 || d->mlp_inner > 8 * MOSS_MAX_DMODEL) return false;
  if (!(d->eps > 0.0f) || !isfinite(d->eps)) return false;
  return true;
}

bool lens_ok(const moss_dims* d, const int32_t* txt_len, ItemLens* out) {
  for (int b = 0; b < MOSS_MAX_BATCH; ++b) out->len[b] = 0;
  for (int b = 0; b < d->batch; ++b) {
    const int32_t n = txt_len ? txt_len[b] : d->n_txt;
    if (n < 0 || n > d->n_txt || (long)n + d->n_img < 1) return false;
    out->len[b] = n;
  }
  return true;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t s_cond, mod, h, a, rope_pp, qp, kp, vp, z, total;
};

// Offsets (bytes) into the workspace.  h is the fp32 residual stream (the
// running sum of the gated adds, rounded to bf16 only when `out` is written).
// a holds the first norm's output, then the attention output, then the second
// norm's output.  rope_pp is the rotary table re-laid for the QKV epilogue
// (once per call).  qp, kp and vp are the packed Q, K and V^T the QKV
// projection writes from its epilogue (their pad rows are zeroed once per
// call and never written again); z is the MLP activation.  No projection
// output reaches memory as such: QKV is normed, rotated and packed in its
// epilogue, the out and down projections add into h in theirs, and the up
// projection applies the SiLU gate in its own.
Layout plan(const moss_dims* d, int n_blocks) {
  Layout L;
  const size_t B = d->batch, T = (size_t)d->n_txt + d->n_img, D = d->d_model, F = d->mlp_inner;
  const size_t R = B * T, Tp = packed_rows((int)T), H = d->n_heads;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round256(bytes);
    return o;
  };
  L.s_cond = take(4 * B * D);
  L.mod = take(4 * B * 6 * D * (size_t)n_blocks);  // every block's modulation, computed up front
  L.h = take(4 * R * D);
  L.a = take(2 * R * D);
  const size_t packed = 2 * B * H * Tp * 128;
  L.rope_pp = take(512 * Tp);
  L.qp = take(packed);
  L.kp = take(packed);
  L.vp = take(packed);
  L.z = take(2 * R * F);
  L.total = off;
  return L;
}

// byte range [p, p + n) overlaps [q, q + m)
bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + m && b < a + n;
}

// ---- device capability cache ---------------------------------------------------
std::mutex g_dev_mu;
std::vector<int> g_dev_state;  // 0 unknown, 1 gfx950, 2 other

int check_device(int dev) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0 || dev < 0 || dev >= count) return MOSS_EDEVICE;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if ((int)g_dev_state.size() < count) g_dev_state.resize(count, 0);
    if (g_dev_state[dev] == 1) return MOSS_OK;
    if (g_dev_state[dev] == 2) return MOSS_EDEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOSS_EDEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  g_dev_state[dev] = ok ? 1 : 2;
  return ok ? MOSS_OK : MOSS_EDEVICE;
}

int check_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOSS_EDEVICE;
  return check_device(dev);
}

// ---- timing probe -------------------------------------------------------------------
struct Probe {
  std::mutex mu;
  int step = -1;
  int max = 0;
  int used = 0;
  int every = 1;
  int seen = 0;                // launches of the armed step since arming
  std::vector<hipEvent_t> ev;  // 2 per launch
};
Probe g_probe;

// Records the start event of a probed launch; returns its slot or -1.
int probe_begin(int step, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_probe.mu);
  if (g_probe.step != step || g_probe.used >= g_probe.max) return -1;
  if (g_probe.seen++ % g_probe.every != 0) return -1;
  const int slot = g_probe.used;
  if (hipEventRecord(g_probe.ev[2 * slot], st) != hipSuccess) return -1;
  g_probe.used = slot + 1;
  return slot;
}
void probe_end(int slot, hipStream_t st) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_probe.mu);
  (void)hipEventRecord(g_probe.ev[2 * slot + 1], st);
}

struct StepTimer {
  int slot;
  hipStream_t st;
  StepTimer(int step, hipStream_t s) : slot(probe_begin(step, s)), st(s) {}
  ~StepTimer() { probe_end(slot, st); }
};

// ---- the block ----------------------------------------------------------------------
struct Ctx {
  const moss_dims* d;
  ItemLens lens;
  Layout L;
  char* ws;
  hipStream_t st;
};

// One block on the fp32 residual h; when out16 is not null the block's last
// gated add writes the bf16 result there instead of updating h.
// The call's inputs, for its first block: the rows are joined into h in the same pass as the first norm.
struct FirstRows {
  const uint16_t* x;
  const uint16_t* txt;
};

// mod: this block's modulation [B][6 D] (computed for the whole stack up front; items a block skips
// have zero gates there, so a block run on them leaves their residual unchanged).
int run_block(const Ctx& c, const moss_block_weights* w, const float* rope, float* h, uint16_t* out16,
              const float* mod, const FirstRows* first) {
  const moss_dims* d = c.d;
  const int B = d->batch, T = d->n_txt + d->n_img, D = d->d_model, F = d->mlp_inner, H = d->n_heads;
  const int R = B * T;
  uint16_t* a = reinterpret_cast<uint16_t*>(c.ws + c.L.a);
  uint16_t* qp = reinterpret_cast<uint16_t*>(c.ws + c.L.qp);
  uint16_t* kp = reinterpret_cast<uint16_t*>(c.ws + c.L.kp);
  uint16_t* vp = reinterpret_cast<uint16_t*>(c.ws + c.L.vp);
  uint16_t* z = reinterpret_cast<uint16_t*>(c.ws + c.L.z);
  const int ms = 6 * D;  // item stride of the modulation vector
  hipStream_t st = c.st;
  if (first) {
    StepTimer t(MOSS_STEP_JOIN, st);  // row join + the first norm, one pass
    MOSS_TRY(launch_join_mod_rmsnorm(first->x, first->txt, c.lens, mod + 0 * D, mod + 1 * D, ms, h, a, B, d->n_txt,
                                     d->n_img, D, d->eps, st),
             "join_mod_rmsnorm");
  } else {
    StepTimer t(MOSS_STEP_NORM1, st);
    MOSS_TRY(launch_mod_rmsnorm(h, mod + 0 * D, mod + 1 * D, ms, a, B, T, D, d->eps, st), "mod_rmsnorm");
  }
  {
    StepTimer t(MOSS_STEP_QKV, st);  // QKV projection + q/k norm, rotary and packing
    MOSS_TRY(launch_gemm_qkv_pack(B, T, H, d->eps, a, w->w_qkv, w->q_gain, w->k_gain,
                                  reinterpret_cast<const float*>(c.ws + c.L.rope_pp), qp, kp, vp, st),
             "gemm qkv + pack");
  }
  {
    StepTimer t(MOSS_STEP_ATTN, st);
    MOSS_TRY(launch_attention(B, H, T, d->n_txt, c.lens, qp, kp, vp, a, st), "attention");
  }
  {
    StepTimer t(MOSS_STEP_OUT, st);  // out projection + first gated add
    MOSS_TRY(launch_gemm_gated_add(R, D, D, a, D, w->w_out, D, h, mod + 2 * D, ms, T, nullptr, st),
             "gemm out + gated add");
  }
  {
    StepTimer t(MOSS_STEP_NORM2, st);
    MOSS_TRY(launch_mod_rmsnorm(h, mod + 3 * D, mod + 4 * D, ms, a, B, T, D, d->eps, st), "mod_rmsnorm");
  }
  {
    StepTimer t(MOSS_STEP_UP, st);  // up projection + SiLU gate
    MOSS_TRY(launch_gemm_silu(R, F, D, a, D, w->w_up, D, z, F, st), "gemm up + silu");
  }
  {
    StepTimer t(MOSS_STEP_DOWN, st);  // down projection + second gated add
    MOSS_TRY(launch_gemm_gated_add(R, D, F, z, F, w->w_down, F, h, mod + 5 * D, ms, T, out16, st),
             "gemm down + gated add");
  }
  return MOSS_OK;
}

bool weights_ok(const moss_block_weights* w) {
  if (!w) return false;
  const void* p[] = {w->w_mod, w->w_qkv, w->q_gain, w->k_gain, w->w_out, w->w_up, w->w_down};
  for (const void* q : p)
    if (!q || !aligned16(q)) return false;
  return true;
}

// Does any of a block's weight tensors overlap the byte range [p, p + n)?
bool weights_overlap(const moss_block_weights& w, const void* p, size_t n, size_t D, size_t F) {
  return overlaps(p, n, w.w_mod, 2 * 6 * D * D) || overlaps(p, n, w.w_qkv, 2 * 3 * D * D) ||
         overlaps(p, n, w.q_gain, 256) || overlaps(p, n, w.k_gain, 256) || overlaps(p, n, w.w_out, 2 * D * D) ||
         overlaps(p, n, w.w_up, 2 * 2 * F * D) || overlaps(p, n, w.w_down, 2 * D * F);
}

// Validation shared by the block and the stack; fills ctx on success.
int validate_forward(const moss_dims* d, int n_blocks, const uint16_t* x, const uint16_t* txt,
                     const int32_t* txt_len, const uint16_t* cond, const moss_block_weights* blocks,
                     const float* rope, uint16_t* out, void* workspace, size_t ws_bytes, Ctx* ctx) {
  if (!dims_ok(d) || n_blocks < 1 || !blocks) return MOSS_EINVAL;
  if (!cond || !rope || !out || !aligned16(cond) || !aligned16(rope) || !aligned16(out)) return MOSS_EINVAL;
  if (d->n_img > 0 && (!x || !aligned16(x))) return MOSS_EINVAL;
  if (d->n_txt > 0 && (!txt || !aligned16(txt))) return MOSS_EINVAL;
  if (!lens_ok(d, txt_len, &ctx->lens)) return MOSS_EINVAL;
  for (int i = 0; i < n_blocks; ++i)
    if (!weights_ok(&blocks[i])) return MOSS_EINVAL;
  if (!workspace || !aligned16(workspace)) return MOSS_EWORKSPACE;
  ctx->L = plan(d, n_blocks);
  if (ws_bytes < ctx->L.total) return MOSS_EWORKSPACE;
  const size_t B = d->batch, T = (size_t)d->n_txt + d->n_img, D = d->d_model, F = d->mlp_inner;
  const size_t out_bytes = 2 * B * T * D;
  if (overlaps(out, out_bytes, x, 2 * B * d->n_img * D) || overlaps(out, out_bytes, txt, 2 * B * d->n_txt * D) ||
      overlaps(out, out_bytes, cond, 2 * B * D) || overlaps(out, out_bytes, rope, 4 * 2 * T * 64) ||
      overlaps(out, out_bytes, workspace, ctx->L.total))
    return MOSS_EALIAS;
  for (int i = 0; i < n_blocks; ++i)
    if (weights_overlap(blocks[i], out, out_bytes, D, F)) return MOSS_EALIAS;
  // an input inside the workspace would be overwritten while it is still needed
  if (overlaps(workspace, ctx->L.total, x, 2 * B * d->n_img * D) ||
      overlaps(workspace, ctx->L.total, txt, 2 * B * d->n_txt * D) ||
      overlaps(workspace, ctx->L.total, cond, 2 * B * D) || overlaps(workspace, ctx->L.total, rope, 4 * 2 * T * 64))
    return MOSS_EALIAS;
  for (int i = 0; i < n_blocks; ++i)
    if (weights_overlap(blocks[i], workspace, ctx->L.total, D, F)) return MOSS_EALIAS;
  ctx->d = d;
  ctx->ws = static_cast<char*>(workspace);
  return MOSS_OK;
}

// The stack on validated arguments: cond's SiLU, then the blocks; the first
// block joins x and txt into h, the last writes bf16 `out` (or, with out
// null, leaves its result in the fp32 residual h).  skip: null, or host
// [n_blocks][batch], nonzero where block i is not applied to item b.
int run_stack(const Ctx& c, int n_blocks, const uint16_t* x, const uint16_t* txt, const uint16_t* cond,
              const moss_block_weights* blocks, const float* rope, uint16_t* out, const uint8_t* skip) {
  const moss_dims* d = c.d;
  float* h = reinterpret_cast<float*>(c.ws + c.L.h);
  // SiLU(cond), the re-laid rotary table and the packed pad rows, once per call
  MOSS_TRY(launch_call_prologue(cond, reinterpret_cast<float*>(c.ws + c.L.s_cond), d->batch * d->d_model, rope,
                                d->batch, d->n_txt + d->n_img, d->n_heads,
                                reinterpret_cast<float*>(c.ws + c.L.rope_pp),
                                reinterpret_cast<uint16_t*>(c.ws + c.L.qp),
                                reinterpret_cast<uint16_t*>(c.ws + c.L.kp),
                                reinterpret_cast<uint16_t*>(c.ws + c.L.vp), c.st),
           "call prologue");
  // every block's modulation depends only on cond: one launch streams all the W_mod matrices
  float* mod = reinterpret_cast<float*>(c.ws + c.L.mod);
  const size_t mod_stride = (size_t)d->batch * 6 * d->d_model;
  {
    StepTimer t(MOSS_STEP_ADALN, c.st);
    constexpr int kChunk = 32;  // matrices per launch_adaln_gemv_many call (no host allocation per call)
    for (int i0 = 0; i0 < n_blocks; i0 += kChunk) {
      const int k = n_blocks - i0 < kChunk ? n_blocks - i0 : kChunk;
      const uint16_t* w_mods[kChunk];
      unsigned masks[kChunk];
      for (int i = 0; i < k; ++i) {
        w_mods[i] = blocks[i0 + i].w_mod;
        masks[i] = 0u;
        if (skip)
          for (int b = 0; b < d->batch; ++b)
            if (skip[(size_t)(i0 + i) * d->batch + b]) masks[i] |= 1u << b;
      }
      MOSS_TRY(launch_adaln_gemv_many(reinterpret_cast<const float*>(c.ws + c.L.s_cond), w_mods, masks, k,
                                      mod + (size_t)i0 * mod_stride, d->batch, d->d_model, c.st),
               "adaln_gemv");
    }
  }
  const size_t item_elems = (size_t)(d->n_txt + d->n_img) * d->d_model;
  for (int i = 0; i < n_blocks; ++i) {
    const FirstRows rows{x, txt};
    uint16_t* out16 = i + 1 == n_blocks ? out : nullptr;
    // the items this block runs on: all, a contiguous run [b0, b1) (the others skip it), or another
    // pattern, which runs every item with the skipped items' gates zeroed (their residual passes
    // through exactly; the modulation launch above zeroed them)
    int b0 = 0, b1 = d->batch;
    bool contiguous = true;
    if (skip) {
      const uint8_t* sk = skip + (size_t)i * d->batch;
      b0 = 0;
      while (b0 < d->batch && sk[b0]) ++b0;
      b1 = b0;
      while (b1 < d->batch && !sk[b1]) ++b1;
      for (int b = b1; b < d->batch; ++b)
        if (!sk[b]) contiguous = false;
      if (!contiguous) b0 = 0, b1 = d->batch;
    }
    if (b0 == 0 && b1 == d->batch) {
      const int rc = run_block(c, &blocks[i], rope, h, out16, mod + i * mod_stride, i == 0 ? &rows : nullptr);
      if (rc != MOSS_OK) return rc;
      continue;
    }
    // a block skipped by some items runs on the others' rows only
    if (i == 0) {
      StepTimer t(MOSS_STEP_JOIN, c.st);  // join every item's rows (the skipped ones keep them as they are)
      MOSS_TRY(launch_join_rows(x, txt, c.lens, h, d->batch, d->n_txt, d->n_img, d->d_model, c.st), "join_rows");
    }
    if (b1 > b0) {
      moss_dims sub = *d;
      sub.batch = b1 - b0;
      Ctx cs = c;
      cs.d = &sub;
      for (int b = 0; b < sub.batch; ++b) cs.lens.len[b] = c.lens.len[b0 + b];
      const int rc = run_block(cs, &blocks[i], rope, h + b0 * item_elems, out16 ? out16 + b0 * item_elems : nullptr,
                               mod + i * mod_stride + (size_t)b0 * 6 * d->d_model, nullptr);
      if (rc != MOSS_OK) return rc;
    }
    if (out16) {
      // the call's output for the items that skip its last block: their residual, rounded
      for (int b = 0; b < d->batch; ++b)
        if (b < b0 || b >= b1)
          MOSS_TRY(launch_round_bf16(h + b * item_elems, out16 + b * item_elems, (int)item_elems, c.st),
                   "round residual");
    }
  }
  return MOSS_OK;
}

int forward(const moss_dims* d, int n_blocks, const uint16_t* x, const uint16_t* txt, const int32_t* txt_len,
            const uint16_t* cond, const moss_block_weights* blocks, const float* rope, uint16_t* out,
            void* workspace, size_t ws_bytes, hipStream_t st, const uint8_t* skip = nullptr) {
  Ctx c;
  int rc = validate_forward(d, n_blocks, x, txt, txt_len, cond, blocks, rope, out, workspace, ws_bytes, &c);
  if (rc != MOSS_OK) return rc;
  rc = check_current_device();
  if (rc != MOSS_OK) return rc;
  c.st = st;
  return run_stack(c, n_blocks, x, txt, cond, blocks, rope, out, skip);
}

// ---- the whole denoiser forward ---------------------------------------------------
constexpr int kLatent = 128;  // values per latent row
constexpr int kFreq = 256;    // timestep features

// The ends' scratch, after the stack's plan: the projected rows the stack
// joins (bf16), cond (fp32 and bf16), the timestep MLP's hidden values and the
// final modulation (fp32).
struct EndsLayout {
  size_t xrows, trows, cond32, cond16, feat, hid, modf, total;
};
EndsLayout plan_ends(const moss_dims* d, size_t start) {
  EndsLayout E;
  const size_t B = d->batch, D = d->d_model;
  size_t off = start;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round256(bytes);
    return o;
  };
  E.xrows = take(2 * B * d->n_img * D);
  E.trows = take(2 * B * (size_t)d->n_txt * D);
  E.cond32 = take(4 * B * D);
  E.cond16 = take(2 * B * D);
  E.feat = take(4 * B * kFreq);
  E.hid = take(4 * B * D);
  E.modf = take(4 * B * 2 * D);
  E.total = off;
  return E;
}

bool ends_ok(const moss_denoiser_weights* e) {
  if (!e || e->enc_dim < 64 || e->enc_dim % 64 || e->enc_dim > 16384) return false;
  const void* p[] = {e->w_t1, e->w_t2, e->w_txt, e->w_in, e->w_fmod, e->w_final};
  for (const void* q : p)
    if (!q || !aligned16(q)) return false;
  return true;
}

int denoiser(const moss_dims* d, int n_blocks, const uint16_t* latent, const uint16_t* enc, const int32_t* txt_len,
             const float* t, const moss_denoiser_weights* e, const moss_block_weights* blocks, const uint8_t* skip,
             const float* rope, uint16_t* velocity, void* workspace, size_t ws_bytes, hipStream_t st) {
  if (!dims_ok(d) || d->n_img < 1 || n_blocks < 1 || !blocks || !ends_ok(e) || !t) return MOSS_EINVAL;
  if (!latent || !aligned16(latent) || !rope || !aligned16(rope) || !velocity || !aligned16(velocity))
    return MOSS_EINVAL;
  if (d->n_txt > 0 && (!enc || !aligned16(enc))) return MOSS_EINVAL;
  ItemTimes ts{};
  for (int b = 0; b < d->batch; ++b) {
    if (!isfinite(t[b])) return MOSS_EINVAL;
    ts.t[b] = t[b];
  }
  Ctx c;
  if (!lens_ok(d, txt_len, &c.lens)) return MOSS_EINVAL;
  for (int i = 0; i < n_blocks; ++i)
    if (!weights_ok(&blocks[i])) return MOSS_EINVAL;
  if (!workspace || !aligned16(workspace)) return MOSS_EWORKSPACE;
  c.L = plan(d, n_blocks);
  const EndsLayout E = plan_ends(d, c.L.total);
  if (ws_bytes < E.total) return MOSS_EWORKSPACE;
  const size_t B = d->batch, T = (size_t)d->n_txt + d->n_img, D = d->d_model, F = d->mlp_inner;
  const size_t vb = 2 * B * d->n_img * kLatent, ed = e->enc_dim;
  const void* in[] = {latent, enc, rope, workspace, e->w_t1, e->w_t2, e->w_txt, e->w_in, e->w_fmod, e->w_final};
  const size_t len[] = {2 * B * d->n_img * kLatent, 2 * B * d->n_txt * ed, 4 * 2 * T * 64, E.total, 2 * D * kFreq,
                        2 * D * D, 2 * D * ed, 2 * D * kLatent, 2 * 2 * D * D, 2 * kLatent * D};
  for (int i = 0; i < 10; ++i)
    if (overlaps(velocity, vb, in[i], len[i])) return MOSS_EALIAS;
  for (int i = 0; i < n_blocks; ++i)
    if (weights_overlap(blocks[i], velocity, vb, D, F)) return MOSS_EALIAS;
  // no input inside the workspace (in[3] is the workspace itself)
  for (int i = 0; i < 10; ++i)
    if (i != 3 && overlaps(workspace, E.total, in[i], len[i])) return MOSS_EALIAS;
  for (int i = 0; i < n_blocks; ++i)
    if (weights_overlap(blocks[i], workspace, E.total, D, F)) return MOSS_EALIAS;
  int rc = check_current_device();
  if (rc != MOSS_OK) return rc;
  c.d = d;
  c.ws = static_cast<char*>(workspace);
  c.st = st;
  const int Bi = d->batch, Di = d->d_model;
  float* feat = reinterpret_cast<float*>(c.ws + E.feat);
  float* hid = reinterpret_cast<float*>(c.ws + E.hid);
  float* cond32 = reinterpret_cast<float*>(c.ws + E.cond32);
  uint16_t* cond16 = reinterpret_cast<uint16_t*>(c.ws + E.cond16);
  uint16_t* xrows = reinterpret_cast<uint16_t*>(c.ws + E.xrows);
  uint16_t* trows = reinterpret_cast<uint16_t*>(c.ws + E.trows);
  // cond = bf16(W_t2 SiLU(W_t1 features(t)))
  MOSS_TRY(launch_timestep_features(ts, feat, Bi, st), "timestep_features");
  MOSS_TRY(launch_gemv(feat, e->w_t1, hid, Bi, kFreq, Di, st), "gemv t1");
  MOSS_TRY(launch_silu_f32(hid, hid, Bi * Di, st), "silu");
  MOSS_TRY(launch_gemv(hid, e->w_t2, cond32, Bi, Di, Di, st), "gemv t2");
  MOSS_TRY(launch_round_bf16(cond32, cond16, Bi * Di, st), "round cond");
  // the rows the stack joins
  MOSS_TRY(launch_gemm_nt(Bi * d->n_img, Di, kLatent, latent, kLatent, e->w_in, kLatent, xrows, Di, st),
           "gemm latent rows");
  if (d->n_txt > 0)
    MOSS_TRY(launch_gemm_nt(Bi * d->n_txt, Di, (int)ed, enc, (int)ed, e->w_txt, (int)ed, trows, Di, st),
             "gemm prompt rows");
  rc = run_stack(c, n_blocks, xrows, trows, cond16, blocks, rope, nullptr, skip);
  if (rc != MOSS_OK) return rc;
  // velocity = W_final modnorm(h_img; W_fmod SiLU(cond)); the stack left SiLU(cond) in s_cond
  float* modf = reinterpret_cast<float*>(c.ws + E.modf);
  float* h = reinterpret_cast<float*>(c.ws + c.L.h);
  uint16_t* a = reinterpret_cast<uint16_t*>(c.ws + c.L.a);
  MOSS_TRY(launch_gemv(reinterpret_cast<float*>(c.ws + c.L.s_cond), e->w_fmod, modf, Bi, Di, 2 * Di, st),
           "gemv final modulation");
  MOSS_TRY(launch_mod_rmsnorm(h, modf, modf + Di, 2 * Di, a, Bi, (int)T, Di, d->eps, st), "final norm");
  for (int b = 0; b < Bi; ++b)
    MOSS_TRY(launch_gemm_nt(d->n_img, kLatent, Di, a + ((size_t)b * T + d->n_txt) * D, Di, e->w_final, Di,
                            velocity + (size_t)b * d->n_img * kLatent, kLatent, st),
             "gemm velocity");
  return MOSS_OK;
}

int single_device_check() { return check_current_device(); }

// ---- the block forward for callers that cannot allocate ----------------------------
// Its workspace is this file-scope array: one copy per GPU, held from the library's load to the
// end of the process.  Host code never passes the array's name to a kernel (in host code it is a
// host-side stand-in, not a device address): each device's address comes from
// hipGetSymbolAddress, once per device with that device current, and only that address is used.
constexpr size_t kScratchBytes = (size_t)MOSS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) __attribute__((used)) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device; null until looked up

int scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOSS_EDEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return hip_fail(hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOSS_OK;
}

int forward_noalloc(const moss_dims* d, const uint16_t* x, const uint16_t* txt, const int32_t* txt_len,
                    const uint16_t* cond, const moss_block_weights* w, const float* rope, uint16_t* out,
                    hipStream_t st) {
  // the size limit first, before any HIP call
  if (!dims_ok(d)) return MOSS_EINVAL;
  if (plan(d, 1).total > kScratchBytes) return MOSS_EWORKSPACE;
  int rc = check_current_device();
  if (rc != MOSS_OK) return rc;
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != MOSS_OK) return rc;
  Ctx c;
  rc = validate_forward(d, 1, x, txt, txt_len, cond, w, rope, out, ws, kScratchBytes, &c);
  if (rc != MOSS_OK) return rc;
  c.st = st;
  return run_stack(c, 1, x, txt, cond, w, rope, out, nullptr);
}

}  // namespace

// ============================================================================
// exported C ABI
// ============================================================================
extern "C" {

const char* moss_status_string(int status) {
  switch (status) {
    case MOSS_OK: return "ok";
    case MOSS_EINVAL: return "invalid argument";
    case MOSS_EALIAS: return "an output overlaps an input or the workspace, or an input lies in the workspace";
    case MOSS_EWORKSPACE: return "workspace missing or too small";
    case MOSS_EDEVICE: return "no gfx950 device";
    case MOSS_EHIP: return g_hip_error.empty() ? "HIP error" : g_hip_error.c_str();
    default: return "unknown status";
  }
}

int moss_device_check(int hip_device) { return check_device(hip_device); }

size_t moss_workspace_bytes(const moss_dims* dims, int32_t n_blocks) {
  if (!dims_ok(dims) || n_blocks < 1) return 0;
  return plan(dims, n_blocks).total;
}

int32_t moss_packed_rows(int32_t rows) { return rows < 1 ? 0 : packed_rows(rows); }

int moss_rope_build(int32_t n_txt, int32_t grid_h, int32_t grid_w, float theta, float* rope, hipStream_t stream) {
  if (n_txt < 0 || grid_h < 1 || grid_w < 1 || !(theta > 1.0f) || !isfinite(theta)) return MOSS_EINVAL;
  if ((long)n_txt + (long)grid_h * grid_w > MOSS_MAX_ROWS) return MOSS_EINVAL;
  if (!rope || !aligned16(rope)) return MOSS_EINVAL;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_rope_build(n_txt, grid_h, grid_w, theta, rope, stream), "rope_build");
  return MOSS_OK;
}

int moss_block_forward(const moss_dims* dims, const uint16_t* x, const uint16_t* txt, const int32_t* txt_len,
                       const uint16_t* cond, const moss_block_weights* w, const float* rope, uint16_t* out,
                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  return forward(dims, 1, x, txt, txt_len, cond, w, rope, out, workspace, ws_bytes, stream);
}

int moss_block_forward_noalloc(const moss_dims* dims, const uint16_t* x, const uint16_t* txt,
                               const int32_t* txt_len, const uint16_t* cond, const moss_block_weights* w,
                               const float* rope, uint16_t* out, hipStream_t stream) {
  return forward_noalloc(dims, x, txt, txt_len, cond, w, rope, out, stream);
}

size_t moss_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moss_stack_forward(const moss_dims* dims, int32_t n_blocks, const uint16_t* x, const uint16_t* txt,
                       const int32_t* txt_len, const uint16_t* cond, const moss_block_weights* blocks,
                       const float* rope, uint16_t* out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return forward(dims, n_blocks, x, txt, txt_len, cond, blocks, rope, out, workspace, ws_bytes, stream);
}

int moss_stack_forward_skip(const moss_dims* dims, int32_t n_blocks, const uint16_t* x, const uint16_t* txt,
                            const int32_t* txt_len, const uint16_t* cond, const moss_block_weights* blocks,
                            const uint8_t* skip, const float* rope, uint16_t* out, void* workspace,
                            size_t ws_bytes, hipStream_t stream) {
  return forward(dims, n_blocks, x, txt, txt_len, cond, blocks, rope, out, workspace, ws_bytes, stream, skip);
}

size_t moss_denoiser_workspace_bytes(const moss_dims* dims, int32_t n_blocks) {
  if (!dims_ok(dims) || n_blocks < 1 || dims->n_img < 1) return 0;
  return plan_ends(dims, plan(dims, n_blocks).total).total;
}

int moss_denoiser_forward(const moss_dims* dims, int32_t n_blocks, const uint16_t* latent, const uint16_t* enc,
                          const int32_t* txt_len, const float* t, const moss_denoiser_weights* ends,
                          const moss_block_weights* blocks, const uint8_t* skip, const float* rope,
                          uint16_t* velocity, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return denoiser(dims, n_blocks, latent, enc, txt_len, t, ends, blocks, skip, rope, velocity, workspace, ws_bytes,
                  stream);
}

int moss_guidance_euler(int32_t rows, int32_t width, const uint16_t* v_pos, const uint16_t* v_neg, float guidance,
                        float dsigma, const float* x_in, float* x_out, hipStream_t stream) {
  if (rows < 0 || width < 8 || width % 8 || (long)rows * width > (1L << 31)) return MOSS_EINVAL;
  if (!isfinite(guidance) || !isfinite(dsigma)) return MOSS_EINVAL;
  if (!v_neg && guidance != 1.0f) return MOSS_EINVAL;  // only guidance 1 may skip the negative pass
  if (!v_pos || !x_in || !x_out || !aligned16(v_pos) || !aligned16(x_in) || !aligned16(x_out)) return MOSS_EINVAL;
  if (v_neg && !aligned16(v_neg)) return MOSS_EINVAL;
  const size_t vb = 2 * (size_t)rows * width, xb = 4 * (size_t)rows * width;
  if (overlaps(x_out, xb, v_pos, vb) || overlaps(x_out, xb, v_neg, vb)) return MOSS_EALIAS;
  if (x_out != x_in && overlaps(x_out, xb, x_in, xb)) return MOSS_EALIAS;  // in place, or apart
  if (rows == 0) return MOSS_OK;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_guidance_euler(rows, width, v_pos, v_neg, guidance, dsigma, x_in, x_out, stream),
           "guidance_euler");
  return MOSS_OK;
}

int moss_k_join_rows(int32_t batch, int32_t n_txt, int32_t n_img, int32_t d_model, const uint16_t* x,
                     const uint16_t* txt, const int32_t* txt_len, float* out, hipStream_t stream) {
  moss_dims d = {batch, n_img, n_txt, d_model, d_model / MOSS_HEAD_DIM, MOSS_HEAD_DIM, 128, 1e-6f};
  if (!dims_ok(&d)) return MOSS_EINVAL;
  ItemLens lens;
  if (!lens_ok(&d, txt_len, &lens)) return MOSS_EINVAL;
  if (!out || !aligned16(out) || (n_img > 0 && (!x || !aligned16(x))) || (n_txt > 0 && (!txt || !aligned16(txt))))
    return MOSS_EINVAL;
  const size_t ob = 4ull * batch * (n_txt + n_img) * d_model;
  if (overlaps(out, ob, x, 2ull * batch * n_img * d_model) || overlaps(out, ob, txt, 2ull * batch * n_txt * d_model))
    return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_join_rows(x, txt, lens, out, batch, n_txt, n_img, d_model, stream), "join_rows");
  return MOSS_OK;
}

int moss_k_adaln_gemv(int32_t batch, int32_t d_model, const uint16_t* cond, const uint16_t* w_mod, float* mod,
                      void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (batch < 1 || batch > MOSS_MAX_BATCH || d_model < 128 || d_model % 128 || d_model > MOSS_MAX_DMODEL)
    return MOSS_EINVAL;
  if (!cond || !w_mod || !mod || !aligned16(cond) || !aligned16(w_mod) || !aligned16(mod)) return MOSS_EINVAL;
  if (!workspace || !aligned16(workspace) || ws_bytes < 4ull * batch * d_model) return MOSS_EWORKSPACE;
  if (overlaps(mod, 4ull * batch * 6 * d_model, workspace, 4ull * batch * d_model)) return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  float* s = static_cast<float*>(workspace);
  MOSS_TRY(launch_silu_cond(cond, s, batch, d_model, stream), "silu_cond");
  {
    StepTimer t(MOSS_STEP_ADALN, stream);  // the GEMV launch alone, when the probe is armed for it
    MOSS_TRY(launch_adaln_gemv(s, w_mod, mod, batch, d_model, 0u, stream), "adaln_gemv");
  }
  return MOSS_OK;
}

int moss_k_mod_rmsnorm(int32_t batch, int32_t rows, int32_t d_model, float eps, const float* h,
                       const float* shift, const float* scale, int32_t mod_stride, uint16_t* out,
                       hipStream_t stream) {
  if (batch < 1 || rows < 1 || (long)batch * rows > (long)MOSS_MAX_BATCH * MOSS_MAX_ROWS) return MOSS_EINVAL;
  if (d_model < 128 || d_model % 128 || d_model > MOSS_MAX_DMODEL || !(eps > 0.0f) || !isfinite(eps))
    return MOSS_EINVAL;
  if (mod_stride < d_model || mod_stride % 4) return MOSS_EINVAL;
  if (!h || !shift || !scale || !out || !aligned16(h) || !aligned16(shift) || !aligned16(scale) || !aligned16(out))
    return MOSS_EINVAL;
  if (overlaps(out, 2ull * batch * rows * d_model, h, 4ull * batch * rows * d_model)) return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_mod_rmsnorm(h, shift, scale, mod_stride, out, batch, rows, d_model, eps, stream), "mod_rmsnorm");
  return MOSS_OK;
}

int moss_k_gemm_nt(int32_t m, int32_t n, int32_t k, const uint16_t* a, int32_t lda, const uint16_t* w,
                   int32_t ldw, uint16_t* c, int32_t ldc, hipStream_t stream) {
  if (m < 1 || n < 128 || k < 128 || n % 128 || k % 128) return MOSS_EINVAL;
  if (lda < k || ldw < k || ldc < n || lda % 8 || ldw % 8 || ldc % 8) return MOSS_EINVAL;
  if ((long)m > (long)MOSS_MAX_BATCH * MOSS_MAX_ROWS) return MOSS_EINVAL;
  if (!a || !w || !c || !aligned16(a) || !aligned16(w) || !aligned16(c)) return MOSS_EINVAL;
  const size_t cb = 2ull * ((size_t)(m - 1) * ldc + n);
  if (overlaps(c, cb, a, 2ull * ((size_t)(m - 1) * lda + k)) || overlaps(c, cb, w, 2ull * ((size_t)(n - 1) * ldw + k)))
    return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_gemm_nt(m, n, k, a, lda, w, ldw, c, ldc, stream), "gemm_nt");
  return MOSS_OK;
}

int moss_k_qk_norm_rope_pack(int32_t batch, int32_t rows, int32_t n_heads, float eps, const uint16_t* qkv,
                             const uint16_t* q_gain, const uint16_t* k_gain, const float* rope, uint16_t* q,
                             uint16_t* k, uint16_t* v, hipStream_t stream) {
  if (batch < 1 || batch > MOSS_MAX_BATCH || rows < 1 || rows > MOSS_MAX_ROWS || n_heads < 1 ||
      n_heads * MOSS_HEAD_DIM > MOSS_MAX_DMODEL || !(eps > 0.0f) || !isfinite(eps))
    return MOSS_EINVAL;
  const void* p[] = {qkv, q_gain, k_gain, rope, q, k, v};
  for (const void* x : p)
    if (!x || !aligned16(x)) return MOSS_EINVAL;
  const size_t pk = 2ull * batch * n_heads * packed_rows(rows) * 128;
  const size_t in = 2ull * batch * rows * 3 * n_heads * 128;
  if (overlaps(q, pk, qkv, in) || overlaps(k, pk, qkv, in) || overlaps(v, pk, qkv, in) || overlaps(q, pk, k, pk) ||
      overlaps(q, pk, v, pk) || overlaps(k, pk, v, pk))
    return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_qk_norm_rope_pack(batch, rows, n_heads, eps, qkv, q_gain, k_gain, rope, q, k, v, stream),
           "qk_norm_rope_pack");
  return MOSS_OK;
}

int moss_k_gemm_qkv_pack(int32_t batch, int32_t rows, int32_t n_heads, float eps, const uint16_t* a,
                         const uint16_t* w_qkv, const uint16_t* q_gain, const uint16_t* k_gain, const float* rope,
                         uint16_t* q, uint16_t* k, uint16_t* v, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  if (batch < 1 || batch > MOSS_MAX_BATCH || rows < 1 || rows > MOSS_MAX_ROWS || n_heads < 1 ||
      n_heads * MOSS_HEAD_DIM > MOSS_MAX_DMODEL || !(eps > 0.0f) || !isfinite(eps))
    return MOSS_EINVAL;
  const void* p[] = {a, w_qkv, q_gain, k_gain, rope, q, k, v};
  for (const void* x : p)
    if (!x || !aligned16(x)) return MOSS_EINVAL;
  const size_t d = (size_t)n_heads * MOSS_HEAD_DIM;
  const size_t pk = 2ull * batch * n_heads * packed_rows(rows) * 128;
  const size_t in = 2ull * batch * rows * d, wb = 2 * 3 * d * d;
  const void* outs[] = {q, k, v};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], pk, a, in) || overlaps(outs[i], pk, w_qkv, wb) || overlaps(outs[i], pk, rope, 8ull * rows * 64))
      return MOSS_EALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], pk, outs[j], pk)) return MOSS_EALIAS;
  }
  if (!workspace || !aligned16(workspace)) return MOSS_EWORKSPACE;
  const size_t need = 512ull * packed_rows(rows);
  if (ws_bytes < need) return MOSS_EWORKSPACE;
  for (int i = 0; i < 3; ++i)
    if (overlaps(outs[i], pk, workspace, need)) return MOSS_EALIAS;
  if (overlaps(workspace, need, a, in) || overlaps(workspace, need, w_qkv, wb) ||
      overlaps(workspace, need, rope, 8ull * rows * 64))
    return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  float* rope_pp = static_cast<float*>(workspace);
  MOSS_TRY(launch_rope_pairs(rope, rows, rope_pp, stream), "rope pairs");
  MOSS_TRY(launch_gemm_qkv_pack(batch, rows, n_heads, eps, a, w_qkv, q_gain, k_gain, rope_pp, q, k, v, stream),
           "gemm qkv + pack");
  MOSS_TRY(launch_zero_packed_pads(batch, rows, n_heads, q, k, v, stream), "zero packed pads");
  return MOSS_OK;
}

int moss_k_attention(int32_t batch, int32_t n_heads, int32_t rows, int32_t n_txt, const int32_t* txt_len,
                     const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, hipStream_t stream) {
  moss_dims d = {batch, rows - n_txt, n_txt, n_heads * MOSS_HEAD_DIM, n_heads, MOSS_HEAD_DIM, 128, 1e-6f};
  if (n_txt < 0 || n_txt > rows || !dims_ok(&d)) return MOSS_EINVAL;
  ItemLens lens;
  if (!lens_ok(&d, txt_len, &lens)) return MOSS_EINVAL;
  const void* p[] = {q, k, v, o};
  for (const void* x : p)
    if (!x || !aligned16(x)) return MOSS_EINVAL;
  const size_t pk = 2ull * batch * n_heads * packed_rows(rows) * 128;
  const size_t ob = 2ull * batch * rows * n_heads * 128;
  if (overlaps(o, ob, q, pk) || overlaps(o, ob, k, pk) || overlaps(o, ob, v, pk)) return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_attention(batch, n_heads, rows, n_txt, lens, q, k, v, o, stream), "attention");
  return MOSS_OK;
}

int moss_k_silu_mul(int32_t rows, int32_t mlp_inner, const uint16_t* u, uint16_t* z, hipStream_t stream) {
  if (rows < 1 || (long)rows > (long)MOSS_MAX_BATCH * MOSS_MAX_ROWS || mlp_inner < 128 || mlp_inner % 128)
    return MOSS_EINVAL;
  if (!u || !z || !aligned16(u) || !aligned16(z)) return MOSS_EINVAL;
  if (overlaps(z, 2ull * rows * mlp_inner, u, 4ull * rows * mlp_inner)) return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_silu_mul(u, z, rows, mlp_inner, stream), "silu_mul");
  return MOSS_OK;
}

int moss_k_gated_add(int32_t batch, int32_t rows, int32_t d_model, float* h, const float* gate,
                     int32_t gate_stride, const uint16_t* y, uint16_t* out, hipStream_t stream) {
  if (batch < 1 || batch > MOSS_MAX_BATCH || rows < 1 || rows > MOSS_MAX_ROWS || d_model < 128 || d_model % 128 ||
      d_model > MOSS_MAX_DMODEL || gate_stride < d_model || gate_stride % 4)
    return MOSS_EINVAL;
  if (!h || !gate || !y || !aligned16(h) || !aligned16(gate) || !aligned16(y) || (out && !aligned16(out)))
    return MOSS_EINVAL;
  const size_t hb = 4ull * batch * rows * d_model, yb = 2ull * batch * rows * d_model;
  const size_t gb = 4ull * ((size_t)(batch - 1) * gate_stride + d_model);
  if (overlaps(h, hb, y, yb) || overlaps(h, hb, gate, gb) ||
      (out && (overlaps(out, yb, h, hb) || overlaps(out, yb, y, yb) || overlaps(out, yb, gate, gb))))
    return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_gated_add(h, gate, gate_stride, y, out, batch, rows, d_model, stream), "gated_add");
  return MOSS_OK;
}

int moss_k_gemm_silu(int32_t m, int32_t mlp_inner, int32_t k, const uint16_t* a, int32_t lda, const uint16_t* w_up,
                     int32_t ldw, uint16_t* z, int32_t ldz, hipStream_t stream) {
  if (m < 1 || mlp_inner < 128 || mlp_inner % 128 || k < 128 || k % 128) return MOSS_EINVAL;
  if (lda < k || ldw < k || ldz < mlp_inner || lda % 8 || ldw % 8 || ldz % 8) return MOSS_EINVAL;
  if ((long)m > (long)MOSS_MAX_BATCH * MOSS_MAX_ROWS) return MOSS_EINVAL;
  if (!a || !w_up || !z || !aligned16(a) || !aligned16(w_up) || !aligned16(z)) return MOSS_EINVAL;
  const size_t zb = 2ull * ((size_t)(m - 1) * ldz + mlp_inner);
  if (overlaps(z, zb, a, 2ull * ((size_t)(m - 1) * lda + k)) ||
      overlaps(z, zb, w_up, 2ull * ((size_t)(2 * mlp_inner - 1) * ldw + k)))
    return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_gemm_silu(m, mlp_inner, k, a, lda, w_up, ldw, z, ldz, stream), "gemm_silu");
  return MOSS_OK;
}

int moss_k_gemm_gated_add(int32_t m, int32_t n, int32_t k, const uint16_t* a, int32_t lda, const uint16_t* w,
                          int32_t ldw, float* h, const float* gate, int32_t gate_stride, int32_t rows_per_item,
                          uint16_t* out, hipStream_t stream) {
  if (m < 1 || n < 128 || n % 128 || k < 128 || k % 128 || lda < k || ldw < k || lda % 8 || ldw % 8)
    return MOSS_EINVAL;
  if (rows_per_item < 1 || m % rows_per_item || m / rows_per_item > MOSS_MAX_BATCH) return MOSS_EINVAL;
  if (gate_stride < n || gate_stride % 4) return MOSS_EINVAL;
  if (!a || !w || !h || !gate || !aligned16(a) || !aligned16(w) || !aligned16(h) || !aligned16(gate) ||
      (out && !aligned16(out)))
    return MOSS_EINVAL;
  const size_t hb = 4ull * m * n, ob = 2ull * m * n;
  const size_t gb = 4ull * ((size_t)(m / rows_per_item - 1) * gate_stride + n);
  const size_t ab = 2ull * ((size_t)(m - 1) * lda + k), wb = 2ull * ((size_t)(n - 1) * ldw + k);
  if (overlaps(h, hb, a, ab) || overlaps(h, hb, w, wb) || overlaps(h, hb, gate, gb) ||
      (out && (overlaps(out, ob, h, hb) || overlaps(out, ob, a, ab) || overlaps(out, ob, w, wb) ||
               overlaps(out, ob, gate, gb))))
    return MOSS_EALIAS;
  const int rc = single_device_check();
  if (rc != MOSS_OK) return rc;
  MOSS_TRY(launch_gemm_gated_add(m, n, k, a, lda, w, ldw, h, gate, gate_stride, rows_per_item, out, stream),
           "gemm_gated_add");
  return MOSS_OK;
}

int moss_probe_arm(int32_t step, int32_t max_launches, int32_t every) {
  if (step < 0 || step >= MOSS_NUM_STEPS || max_launches < 1 || max_launches > 4096 || every < 1) return MOSS_EINVAL;
  std::lock_guard<std::mutex> lk(g_probe.mu);
  while ((int)g_probe.ev.size() < 2 * max_launches) {
    hipEvent_t e;
    // timing only: no system-scope fence (cache writeback and invalidate) at each record, which
    // left a gap of about 6 us before and after the probed launch
    const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (err != hipSuccess) return hip_fail(err, "hipEventCreateWithFlags");
    g_probe.ev.push_back(e);
  }
  g_probe.step = step;
  g_probe.max = max_launches;
  g_probe.used = 0;
  g_probe.every = every;
  g_probe.seen = 0;
  return MOSS_OK;
}

int32_t moss_probe_collect(float* ms, int32_t max_out) {
  if (max_out < 0 || (max_out > 0 && !ms)) return -MOSS_EINVAL;
  std::lock_guard<std::mutex> lk(g_probe.mu);
  const int n = g_probe.used;
  g_probe.step = -1;
  g_probe.used = 0;
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipEventSynchronize(g_probe.ev[2 * i + 1]);
    if (e != hipSuccess) return -hip_fail(e, "hipEventSynchronize");
    if (i < max_out) {
      float t = 0.0f;
      e = hipEventElapsedTime(&t, g_probe.ev[2 * i], g_probe.ev[2 * i + 1]);
      if (e != hipSuccess) return -hip_fail(e, "hipEventElapsedTime");
      ms[i] = t;
    }
  }
  return n;
}

}  // extern "C"
