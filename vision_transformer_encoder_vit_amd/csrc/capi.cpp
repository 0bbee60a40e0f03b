// C ABI of the encoder block: argument validation, the host-side plan
// (workspace layout), and the kernel sequence of one forward. No device
// memory is allocated here; every buffer comes from the caller.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "../../include/vit_block.h"
#include "launch.h"

#define VIT_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_err;

vit_status fail(vit_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

vit_status ok() { return VIT_OK; }

vit_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return VIT_OK;
  return fail(VIT_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return an && bn && x < y + bn && y < x + an;
}

}  // namespace

struct vit_block_plan {
  vit_block_desc d;
  int n_in, n_out, head_dim;
  int64_t m_in, m_out;
  size_t esize;
  // workspace layout (byte offsets)
  size_t off_h, off_qkv, off_rp, off_r, off_ctx, off_x1, off_h2, off_u, off_vt, off_po, off_pml, off_qh, off_kh,
      ws_bytes;
  int attn_splits;       // key splits of the large-window attention (1: none)
  bool split_partials;   // ... over workgroups, through fp32 partials (off_po, off_pml)
  bool fused_mask_unit;  // whole block per window in one kernel (forward without seams)
  bool attn_vt;          // the large-window attention kernel runs on V^T (workspace off_vt)
  bool vt_in_gemm;       // ... written by the qkv projection's epilogue (else a transpose kernel)
  bool attn_hm;          // ... with q (scaled) and k head-major too (off_qh, off_kh): the head_dim-64 kernel
  bool pool_gemm;        // transition: the residual projection pooled in its GEMM epilogue
  bool residual_in_qkv;  // ... and computed by the qkv GEMM (a fourth weight segment)
  // Q8_ROW: workspace copies of the int8 payloads in act_dtype (exact), read
  // by the GEMMs, whose epilogues apply the row scales
  size_t off_cres, off_cqkv, off_cq, off_ck, off_cv, off_co, off_c1, off_c2;
};

static vit_status validate_desc(const vit_block_desc* d) {
  if (!d) return fail(VIT_ERR_INVALID_ARG, "desc is NULL");
  if (d->act_dtype != VIT_DTYPE_F32 && d->act_dtype != VIT_DTYPE_BF16)
    return fail(VIT_ERR_INVALID_ARG, "act_dtype %d is not VIT_DTYPE_F32 or VIT_DTYPE_BF16", d->act_dtype);
  if (d->batch < 1) return fail(VIT_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", d->batch);
  if (d->grid_h < 1 || d->grid_w < 1) return fail(VIT_ERR_INVALID_ARG, "grid %dx%d is empty", d->grid_h, d->grid_w);
  const int64_t n_in = (int64_t)d->grid_h * d->grid_w;
  if (d->dim_in < 8 || d->dim_out < 8 || d->mlp_hidden < 8 || d->dim_in % 8 || d->dim_out % 8 || d->mlp_hidden % 8)
    return fail(VIT_ERR_INVALID_ARG, "dim_in %d, dim_out %d, mlp_hidden %d must be positive multiples of 8",
                d->dim_in, d->dim_out, d->mlp_hidden);
  if (d->heads < 1 || d->dim_out % d->heads)
    return fail(VIT_ERR_INVALID_ARG, "heads %d must divide dim_out %d", d->heads, d->dim_out);
  const int hd = d->dim_out / d->heads;
  if (hd % 8) return fail(VIT_ERR_UNSUPPORTED, "head_dim %d must be a multiple of 8", hd);
  if (hd > 64) return fail(VIT_ERR_UNSUPPORTED, "head_dim %d > 64 is not supported", hd);
  if (d->q_stride != 1 && d->q_stride != 4) return fail(VIT_ERR_INVALID_ARG, "q_stride must be 1 or 4 (got %d)", d->q_stride);
  if (d->q_stride == 1 && d->dim_in != d->dim_out)
    return fail(VIT_ERR_INVALID_ARG, "dim_in %d != dim_out %d needs the q_stride-4 residual projection", d->dim_in, d->dim_out);
  if (d->q_stride == 4 && n_in % 4) return fail(VIT_ERR_INVALID_ARG, "q_stride 4 needs a token count divisible by 4");
  const int64_t n_out = n_in / d->q_stride;
  switch (d->attn_mode) {
    case VIT_ATTN_GLOBAL: break;
    case VIT_ATTN_MASK_UNIT:
      if (d->n_windows < 1 || n_in % d->n_windows || n_out % d->n_windows)
        return fail(VIT_ERR_INVALID_ARG, "n_windows %d must divide the %lld input and %lld output tokens", d->n_windows,
                    (long long)n_in, (long long)n_out);
      break;
    case VIT_ATTN_SPATIAL:
      if (d->win_h < 1 || d->win_w < 1 || d->grid_h % d->win_h || d->grid_w % d->win_w)
        return fail(VIT_ERR_INVALID_ARG, "window %dx%d must tile the %dx%d grid", d->win_h, d->win_w, d->grid_h, d->grid_w);
      if (d->q_stride != 1) return fail(VIT_ERR_UNSUPPORTED, "q_stride 4 with SPATIAL windows is not supported");
      break;
    default: return fail(VIT_ERR_INVALID_ARG, "attn_mode %d is not a VIT_ATTN_* value", d->attn_mode);
  }
  if (d->gelu != VIT_GELU_ERF && d->gelu != VIT_GELU_TANH) return fail(VIT_ERR_INVALID_ARG, "gelu %d is not a VIT_GELU_* value", d->gelu);
  if (d->qkv_layout != VIT_QKV_FUSED && d->qkv_layout != VIT_QKV_SEPARATE)
    return fail(VIT_ERR_INVALID_ARG, "qkv_layout %d is not a VIT_QKV_* value", d->qkv_layout);
  if (d->rope != VIT_ROPE_NONE && d->rope != VIT_ROPE_AXIAL_TABLE) return fail(VIT_ERR_INVALID_ARG, "rope %d is not a VIT_ROPE_* value", d->rope);
  if (d->rope == VIT_ROPE_AXIAL_TABLE) {
    if (d->attn_mode == VIT_ATTN_MASK_UNIT) return fail(VIT_ERR_UNSUPPORTED, "RoPE with mask-unit windows is not supported");
    if (d->q_stride != 1) return fail(VIT_ERR_UNSUPPORTED, "RoPE with q_stride 4 is not supported");
    if (hd % 4) return fail(VIT_ERR_INVALID_ARG, "RoPE needs head_dim %% 4 == 0 (head_dim %d)", hd);
    const int64_t want = d->attn_mode == VIT_ATTN_SPATIAL ? (int64_t)d->win_h * d->win_w : n_in;
    if (d->rope_rows != want)
      return fail(VIT_ERR_INVALID_ARG, "rope_rows %d, expected %lld (one row per %s token)", d->rope_rows, (long long)want,
                  d->attn_mode == VIT_ATTN_SPATIAL ? "in-window" : "grid");
  }
  if (!(d->ln_eps > 0.f) || !std::isfinite(d->ln_eps)) return fail(VIT_ERR_INVALID_ARG, "ln_eps must be positive and finite");
  if (!(d->attn_scale >= 0.f) || !std::isfinite(d->attn_scale)) return fail(VIT_ERR_INVALID_ARG, "attn_scale must be >= 0 and finite");
  if (d->weight_format != VIT_WEIGHTS_ACT && d->weight_format != VIT_WEIGHTS_Q8_ROW)
    return fail(VIT_ERR_INVALID_ARG, "weight_format %d is not a VIT_WEIGHTS_* value", d->weight_format);
  const int64_t widest = std::max<int64_t>(std::max<int64_t>(3LL * d->dim_out, d->mlp_hidden), d->dim_in);
  if ((int64_t)d->batch * n_in * widest >= (1LL << 40) || (int64_t)d->batch * n_in >= (1LL << 31))
    return fail(VIT_ERR_UNSUPPORTED, "problem too large");
  return VIT_OK;
}

VIT_API vit_status vit_block_create(const vit_block_desc* desc, vit_block_t* out) {
  if (!out) return fail(VIT_ERR_INVALID_ARG, "out handle pointer is NULL");
  vit_status st = validate_desc(desc);
  if (st != VIT_OK) return st;
  vit_block_plan* p = new (std::nothrow) vit_block_plan();
  if (!p) return fail(VIT_ERR_INVALID_ARG, "out of host memory");
  p->d = *desc;
  p->n_in = desc->grid_h * desc->grid_w;
  p->n_out = p->n_in / desc->q_stride;
  p->head_dim = desc->dim_out / desc->heads;
  p->m_in = (int64_t)desc->batch * p->n_in;
  p->m_out = (int64_t)desc->batch * p->n_out;
  p->esize = desc->act_dtype == VIT_DTYPE_BF16 ? 2 : 4;
  size_t o = 0;
  auto take = [&](int64_t rows, int64_t cols) {
    const size_t at = o;
    o += round256((size_t)rows * cols * p->esize);
    return at;
  };
  const vit_block_desc& d = *desc;
  p->off_h = take(p->m_in, d.dim_in);
  p->off_qkv = take(p->m_in, 3LL * d.dim_out);
  p->off_rp = d.q_stride == 4 ? take(p->m_in, d.dim_out) : 0;
  p->off_r = d.q_stride == 4 ? take(p->m_out, d.dim_out) : 0;
  p->off_ctx = take(p->m_out, d.dim_out);
  p->off_x1 = take(p->m_out, d.dim_out);
  p->off_h2 = take(p->m_out, d.dim_out);
  p->off_u = take(p->m_out, d.mlp_hidden);
  const int64_t n_q = d.attn_mode == VIT_ATTN_SPATIAL ? (int64_t)d.win_h * d.win_w : p->n_out;
  p->attn_vt = vit::attention_takes_vt(d.act_dtype == VIT_DTYPE_BF16 ? vit::DType::BF16 : vit::DType::F32,
                                       d.attn_mode, n_q, p->head_dim, d.win_w, p->n_in,
                                       p->m_in * 3LL * d.dim_out);
  // the qkv projection's MFMA path writes V^T
  p->vt_in_gemm = p->attn_vt && vit::gemm_uses_mfma(d.act_dtype == VIT_DTYPE_BF16 ? vit::DType::BF16 : vit::DType::F32,
                                                    d.dim_in, d.dim_in);
  p->off_vt = p->attn_vt ? take(p->m_in, d.dim_out) : 0;
  // At a transition the residual projection reads the same h as the qkv
  // projection. On the MFMA path it is pooled in its GEMM's epilogue, and
  // it joins the qkv GEMM as a fourth weight segment unless that GEMM's
  // epilogue is taken (RoPE, the V^T output).
  const vit::DType dtp = d.act_dtype == VIT_DTYPE_BF16 ? vit::DType::BF16 : vit::DType::F32;
  p->pool_gemm = d.q_stride == 4 && vit::gemm_uses_mfma(dtp, d.dim_in, d.dim_in);
  p->residual_in_qkv = p->pool_gemm && d.rope == VIT_ROPE_NONE && !p->vt_in_gemm;
  p->attn_hm = p->vt_in_gemm && vit::attention_takes_hm(dtp, d.attn_mode, n_q, p->head_dim, d.win_w, p->n_in,
                                                         d.q_stride);
  p->off_qh = p->attn_hm ? take(p->m_in, d.dim_out) : 0;
  p->off_kh = p->attn_hm ? take(p->m_in, d.dim_out) : 0;
  p->attn_splits = 1;
  if (p->attn_vt && !p->attn_hm) {
    const int64_t windows = d.attn_mode == VIT_ATTN_SPATIAL
                                ? (int64_t)(d.grid_h / d.win_h) * (d.grid_w / d.win_w) : 1;
    const int64_t n_kv = d.attn_mode == VIT_ATTN_SPATIAL ? (int64_t)d.win_h * d.win_w : p->n_in;
    p->attn_splits = vit::attention_splits(d.batch, windows, n_q, n_kv, d.heads);
  }
  // fp32 partials (sizes in elements of esize bytes, rounded up)
  const int64_t fp32_cols = 4 / p->esize;
  const int64_t n_kv_attn = d.attn_mode == VIT_ATTN_SPATIAL ? (int64_t)d.win_h * d.win_w : p->n_in;
  p->split_partials = p->attn_splits > 1 && !vit::attention_split_in_workgroup(p->attn_splits, n_kv_attn);
  p->off_po = p->split_partials ? take((int64_t)p->attn_splits * p->m_out, d.dim_out * fp32_cols) : 0;
  p->off_pml = p->split_partials ? take((int64_t)p->attn_splits * p->m_out, 2LL * d.heads * fp32_cols) : 0;
  if (d.weight_format == VIT_WEIGHTS_Q8_ROW) {
    const int64_t Di = d.dim_in, Do = d.dim_out, F = d.mlp_hidden;
    p->off_cres = d.q_stride == 4 ? take(Do, Di) : 0;
    p->off_cqkv = d.qkv_layout == VIT_QKV_FUSED ? take(3 * Do, Di) : 0;
    p->off_cq = d.qkv_layout == VIT_QKV_SEPARATE ? take(Do, Di) : 0;
    p->off_ck = d.qkv_layout == VIT_QKV_SEPARATE ? take(Do, Di) : 0;
    p->off_cv = d.qkv_layout == VIT_QKV_SEPARATE ? take(Do, Di) : 0;
    p->off_co = take(Do, Do);
    p->off_c1 = take(F, Do);
    p->off_c2 = take(Do, F);
  }
  p->ws_bytes = o;
  p->fused_mask_unit = d.act_dtype == VIT_DTYPE_BF16 &&
                       d.attn_mode == VIT_ATTN_MASK_UNIT && d.q_stride == 1 &&
                       d.rope == VIT_ROPE_NONE &&
                       vit::fused_mask_unit_supported(d.dim_out, d.heads, p->head_dim, d.mlp_hidden, p->n_in / d.n_windows) &&
                       vit::fused_mask_unit_lds_bytes(d.dim_out, d.mlp_hidden) <= 160 * 1024;
  *out = p;
  return ok();
}

VIT_API vit_status vit_block_workspace_size(vit_block_t plan, size_t* bytes) {
  if (!plan || !bytes) return fail(VIT_ERR_INVALID_ARG, "plan or bytes pointer is NULL");
  *bytes = plan->ws_bytes;
  return ok();
}

VIT_API vit_status vit_block_stage_mask(vit_block_t plan, uint32_t* mask) {
  if (!plan || !mask) return fail(VIT_ERR_INVALID_ARG, "plan or mask pointer is NULL");
  if (plan->fused_mask_unit) {
    *mask = 1u << VIT_STAGE_FUSED;
  } else {
    const bool residual = plan->d.q_stride == 4 && !plan->residual_in_qkv;
    *mask = ((1u << VIT_STAGE_FUSED) - 1) & ~(residual ? 0u : 1u << VIT_STAGE_RESIDUAL);
  }
  return ok();
}

VIT_API vit_status vit_block_destroy(vit_block_t plan) {
  delete plan;
  return ok();
}

VIT_API const char* vit_last_error(void) { return g_err.c_str(); }

static vit_status check_weights(const vit_block_plan* p, const vit_block_weights* w) {
  if (!w) return fail(VIT_ERR_INVALID_ARG, "weights struct is NULL");
  const vit_block_desc& d = p->d;
  const bool q8 = d.weight_format == VIT_WEIGHTS_Q8_ROW;
  struct Need {
    const void* ptr;
    const char* name;
    bool needed;
  } need[] = {
      {w->ln1_gamma, "ln1_gamma", true},
      {w->ln1_beta, "ln1_beta", true},
      {w->w_res, "w_res", d.q_stride == 4},
      {w->b_res, "b_res", d.q_stride == 4},
      {w->w_qkv, "w_qkv", d.qkv_layout == VIT_QKV_FUSED},
      {w->b_qkv, "b_qkv", d.qkv_layout == VIT_QKV_FUSED},
      {w->w_q, "w_q", d.qkv_layout == VIT_QKV_SEPARATE},
      {w->b_q, "b_q", d.qkv_layout == VIT_QKV_SEPARATE},
      {w->w_k, "w_k", d.qkv_layout == VIT_QKV_SEPARATE},
      {w->b_k, "b_k", d.qkv_layout == VIT_QKV_SEPARATE},
      {w->w_v, "w_v", d.qkv_layout == VIT_QKV_SEPARATE},
      {w->b_v, "b_v", d.qkv_layout == VIT_QKV_SEPARATE},
      {w->w_o, "w_o", true},
      {w->b_o, "b_o", true},
      {w->ln2_gamma, "ln2_gamma", true},
      {w->ln2_beta, "ln2_beta", true},
      {w->w_fc1, "w_fc1", true},
      {w->b_fc1, "b_fc1", true},
      {w->w_fc2, "w_fc2", true},
      {w->b_fc2, "b_fc2", true},
      {w->rope_table, "rope_table", d.rope == VIT_ROPE_AXIAL_TABLE},
      {w->s_res, "s_res", q8 && d.q_stride == 4},
      {w->s_qkv, "s_qkv", q8 && d.qkv_layout == VIT_QKV_FUSED},
      {w->s_q, "s_q", q8 && d.qkv_layout == VIT_QKV_SEPARATE},
      {w->s_k, "s_k", q8 && d.qkv_layout == VIT_QKV_SEPARATE},
      {w->s_v, "s_v", q8 && d.qkv_layout == VIT_QKV_SEPARATE},
      {w->s_o, "s_o", q8},
      {w->s_fc1, "s_fc1", q8},
      {w->s_fc2, "s_fc2", q8},
  };
  for (const Need& n : need) {
    if (!n.needed) continue;
    if (!n.ptr) return fail(VIT_ERR_INVALID_ARG, "weight %s is NULL", n.name);
    if (!aligned16(n.ptr)) return fail(VIT_ERR_INVALID_ARG, "weight %s is not 16-byte aligned", n.name);
  }
  return VIT_OK;
}

static vit_status forward_impl(vit_block_t plan, const vit_block_weights* w, const void* x, void* y,
                               const vit_block_seams* seams, void* ws, size_t ws_bytes, void* stream,
                               void* const* events = nullptr, int n_events = 0) {
  if (!plan) return fail(VIT_ERR_INVALID_ARG, "plan is NULL");
  const vit_block_plan& P = *plan;
  const vit_block_desc& d = P.d;
  const bool q8 = d.weight_format == VIT_WEIGHTS_Q8_ROW;
  vit_status st = check_weights(&P, w);
  if (st != VIT_OK) return st;
  if (!x || !y) return fail(VIT_ERR_INVALID_ARG, "x or y is NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(VIT_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  if (ws_bytes < P.ws_bytes) return fail(VIT_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, P.ws_bytes);
  if (P.ws_bytes && !ws) return fail(VIT_ERR_WORKSPACE, "workspace is NULL");
  if (ws && !aligned16(ws)) return fail(VIT_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const size_t x_bytes = (size_t)P.m_in * d.dim_in * P.esize;
  const size_t y_bytes = (size_t)P.m_out * d.dim_out * P.esize;
  if (x == y) {
    if (d.q_stride != 1) return fail(VIT_ERR_INVALID_ARG, "y == x is allowed only with q_stride 1");
  } else if (overlaps(x, x_bytes, y, y_bytes)) {
    return fail(VIT_ERR_INVALID_ARG, "x and y overlap");
  }
  if (overlaps(ws, P.ws_bytes, y, y_bytes) || overlaps(ws, P.ws_bytes, x, x_bytes))
    return fail(VIT_ERR_INVALID_ARG, "workspace overlaps x or y");
  vit_block_seams S;
  std::memset(&S, 0, sizeof S);
  if (seams) {
    S = *seams;
    void* const all[] = {S.h, S.qkv, S.q_pooled, S.r, S.ctx, S.attn_branch, S.x1, S.h2, S.u, S.mlp_branch};
    for (void* s : all)
      if (s && !aligned16(s)) return fail(VIT_ERR_INVALID_ARG, "seam buffers must be 16-byte aligned");
  }

  const vit::DType dt = d.act_dtype == VIT_DTYPE_BF16 ? vit::DType::BF16 : vit::DType::F32;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  void* h = S.h ? S.h : base + P.off_h;
  void* qkv = S.qkv ? S.qkv : base + P.off_qkv;
  void* ctx = S.ctx ? S.ctx : base + P.off_ctx;
  void* x1 = S.x1 ? S.x1 : base + P.off_x1;
  void* h2 = S.h2 ? S.h2 : base + P.off_h2;
  void* u = S.u ? S.u : base + P.off_u;
  const int Di = d.dim_in, Do = d.dim_out, F = d.mlp_hidden, hd = P.head_dim;
  hipError_t e;
  // measurement events of stage i: events[2i] (first kernel's start) and
  // events[2i+1] (last kernel's end)
  auto stage_ev = [&](int stage) {
    vit::StageEvents ev;
    if (events && 2 * stage + 1 < n_events) {
      ev.start = (hipEvent_t)events[2 * stage];
      ev.stop = (hipEvent_t)events[2 * stage + 1];
    }
    return ev;
  };
  auto only_start = [](vit::StageEvents ev) { ev.stop = nullptr; return ev; };
  auto mark_empty = [&](int stage) -> vit_status {
    const vit::StageEvents ev = stage_ev(stage);
    if (!ev.start) return VIT_OK;
    vit_status r = device_status(hipEventRecord(ev.start, s), "hipEventRecord");
    return r != VIT_OK ? r : device_status(hipEventRecord(ev.stop, s), "hipEventRecord");
  };

  // Small mask units: the whole block in one kernel per window (no seams:
  // the step-by-step path below produces those).
  if (!seams && P.fused_mask_unit) {
    vit::FusedMUArgs f;
    f.x = x;
    f.y = y;
    f.ln1_g = w->ln1_gamma;
    f.ln1_b = w->ln1_beta;
    f.ln2_g = w->ln2_gamma;
    f.ln2_b = w->ln2_beta;
    // q8_row: the kernel reads the int8 payloads itself (1-byte elements)
    const bool q8w = d.weight_format == VIT_WEIGHTS_Q8_ROW;
    if (d.qkv_layout == VIT_QKV_FUSED) {
      const size_t wseg = (size_t)Do * Di * (q8w ? 1 : P.esize);
      f.wq = w->w_qkv;
      f.wk = (const char*)w->w_qkv + wseg;
      f.wv = (const char*)w->w_qkv + 2 * wseg;
      f.bq = w->b_qkv;
      f.bk = w->b_qkv + Do;
      f.bv = w->b_qkv + 2 * Do;
      if (q8w) {
        f.sq = w->s_qkv;
        f.sk = static_cast<const uint16_t*>(w->s_qkv) + Do;
        f.sv = static_cast<const uint16_t*>(w->s_qkv) + 2 * Do;
      }
    } else {
      f.wq = w->w_q;
      f.wk = w->w_k;
      f.wv = w->w_v;
      f.bq = w->b_q;
      f.bk = w->b_k;
      f.bv = w->b_v;
      if (q8w) {
        f.sq = w->s_q;
        f.sk = w->s_k;
        f.sv = w->s_v;
      }
    }
    f.q8 = q8w;
    if (q8w) {
      f.so = w->s_o;
      f.s1 = w->s_fc1;
      f.s2 = w->s_fc2;
    }
    f.wo = w->w_o;
    f.bo = w->b_o;
    f.w1 = w->w_fc1;
    f.b1 = w->b_fc1;
    f.w2 = w->w_fc2;
    f.b2 = w->b_fc2;
    f.batch = d.batch;
    f.tokens = P.n_in;
    f.n_windows = d.n_windows;
    f.dim = Do;
    f.heads = d.heads;
    f.head_dim = hd;
    f.mlp = F;
    f.eps = d.ln_eps;
    f.scale = d.attn_scale > 0.f ? d.attn_scale : 1.0f / std::sqrt((float)hd);
    f.gelu_tanh = d.gelu == VIT_GELU_TANH;
    for (int stg = 0; stg < VIT_STAGE_FUSED; ++stg)
      if ((st = mark_empty(stg)) != VIT_OK) return st;
    e = vit::launch_block_mask_unit_fused(f, s, stage_ev(VIT_STAGE_FUSED));
    if ((st = device_status(e, "fused mask-unit block")) != VIT_OK) return st;
    return ok();
  }
  auto only_stop = [](vit::StageEvents ev) { ev.start = nullptr; return ev; };

  // 0. Q8_ROW: the int8 payloads to act_dtype (exact) in the workspace, one
  // launch for all matrices (timed with LN1's stage)
  const void* Wres = w->w_res;
  const void *Wqkv = w->w_qkv, *Wq = w->w_q, *Wk = w->w_k, *Wv = w->w_v;
  const void *Wo = w->w_o, *W1 = w->w_fc1, *W2 = w->w_fc2;
  if (q8) {
    vit::I8Segments sg;
    auto add = [&](const void*& wp, size_t off, int64_t n) {
      sg.src[sg.count] = static_cast<const int8_t*>(wp);
      sg.dst[sg.count] = base + off;
      sg.n[sg.count] = n;
      ++sg.count;
      wp = base + off;
    };
    if (d.q_stride == 4) add(Wres, P.off_cres, (int64_t)Do * Di);
    if (d.qkv_layout == VIT_QKV_FUSED) {
      add(Wqkv, P.off_cqkv, 3LL * Do * Di);
    } else {
      add(Wq, P.off_cq, (int64_t)Do * Di);
      add(Wk, P.off_ck, (int64_t)Do * Di);
      add(Wv, P.off_cv, (int64_t)Do * Di);
    }
    add(Wo, P.off_co, (int64_t)Do * Do);
    add(W1, P.off_c1, (int64_t)F * Do);
    add(W2, P.off_c2, (int64_t)Do * F);
    e = vit::launch_i8_convert(sg, dt, s, only_start(stage_ev(VIT_STAGE_LN1)));
    if ((st = device_status(e, "q8_row payload conversion")) != VIT_OK) return st;
  }

  // 1. LN1
  e = vit::launch_layernorm(x, h, w->ln1_gamma, w->ln1_beta, P.m_in, Di, d.ln_eps, dt, s,
                            q8 ? only_stop(stage_ev(VIT_STAGE_LN1)) : stage_ev(VIT_STAGE_LN1));
  if ((st = device_status(e, "layernorm (LN1)")) != VIT_OK) return st;

  // 2. qkv projection (+ bias, + RoPE)
  vit::GemmArgs g;
  g.A = h;
  g.lda = Di;
  g.M = (int)P.m_in;
  g.N = 3 * Do;
  g.K = Di;
  g.C = qkv;
  g.ldc = 3 * Do;
  if (d.qkv_layout == VIT_QKV_FUSED) {
    g.W[0] = Wqkv;
    g.bias[0] = w->b_qkv;
    g.wscale[0] = q8 ? w->s_qkv : nullptr;
    g.seg_cols = 3 * Do;
  } else {
    g.W[0] = Wq;
    g.W[1] = Wk;
    g.W[2] = Wv;
    g.bias[0] = w->b_q;
    g.bias[1] = w->b_k;
    g.bias[2] = w->b_v;
    if (q8) {
      g.wscale[0] = w->s_q;
      g.wscale[1] = w->s_k;
      g.wscale[2] = w->s_v;
    }
    g.seg_cols = Do;
  }
  if (d.rope == VIT_ROPE_AXIAL_TABLE) {
    g.epi = vit::EPI_BIAS_ROPE;
    g.rope = w->rope_table;
    g.rope_cols = 2 * Do;
    g.head_dim = hd;
    g.rope_mode = d.attn_mode == VIT_ATTN_SPATIAL ? 1 : 0;
    g.tokens_per_frame = P.n_in;
    g.grid_w = d.grid_w;
    g.win_h = d.attn_mode == VIT_ATTN_SPATIAL ? d.win_h : 1;
    g.win_w = d.attn_mode == VIT_ATTN_SPATIAL ? d.win_w : 1;
  } else {
    g.epi = vit::EPI_BIAS;
  }
  // the residual projection as a fourth weight segment whose columns the
  // epilogue max-pools over the four quarters of each frame straight into r
  // (Hiera's query pool; no unpooled copy, no separate launches)
  const bool pool_gemm = P.pool_gemm, merged = P.residual_in_qkv;
  void* r_out = S.r ? S.r : base + P.off_r;
  if (merged) {
    if (d.qkv_layout == VIT_QKV_FUSED) {
      for (int k = 0; k < 3; ++k) {
        g.W[k] = static_cast<const char*>(Wqkv) + (size_t)k * Do * Di * P.esize;
        g.bias[k] = w->b_qkv + (size_t)k * Do;
        g.wscale[k] = q8 ? static_cast<const void*>(static_cast<const uint16_t*>(w->s_qkv) + (size_t)k * Do) : nullptr;
      }
    }
    g.W[3] = Wres;
    g.bias[3] = w->b_res;
    g.wscale[3] = q8 ? w->s_res : nullptr;
    g.seg_cols = Do;
    g.N = 4 * Do;
    g.epi = vit::EPI_POOL;
    g.tokens_per_frame = P.n_in;
    g.pool_out = r_out;
    g.ld_pool = Do;
    g.pool_col0 = 3 * Do;
  }
  const float attn_scale = d.attn_scale > 0.f ? d.attn_scale : 1.0f / std::sqrt((float)hd);
  if (P.vt_in_gemm) {
    g.vt = base + P.off_vt;
    g.vt_col0 = 2 * Do;
    g.vt_tokens = P.n_in;
    g.vt_heads = d.heads;
    g.vt_hd = hd;
    g.vt_only = !seams;  // the qkv seam keeps q, k and v in row layout too
  }
  if (P.attn_hm) {
    // q (times scale * log2 e) and k head-major in window order as well
    g.hm_q = base + P.off_qh;
    g.hm_k = base + P.off_kh;
    g.hm_qscale = attn_scale * 1.4426950408889634f;
    g.hm_spatial = d.attn_mode == VIT_ATTN_SPATIAL;
    g.grid_w = d.grid_w;
    g.win_h = g.hm_spatial ? d.win_h : 1;
    g.win_w = g.hm_spatial ? d.win_w : 1;
  }
  if (P.attn_vt && !P.vt_in_gemm) {
    e = vit::launch_gemm(g, dt, s, only_start(stage_ev(VIT_STAGE_QKV)));
    if ((st = device_status(e, "gemm (qkv)")) != VIT_OK) return st;
    e = vit::launch_v_transpose(qkv, 3LL * Do, 2 * Do, base + P.off_vt, d.batch, (int)P.n_in, d.heads, hd, s,
                                only_stop(stage_ev(VIT_STAGE_QKV)));
    if ((st = device_status(e, "V transpose")) != VIT_OK) return st;
  } else {
    e = vit::launch_gemm(g, dt, s, stage_ev(VIT_STAGE_QKV));
    if ((st = device_status(e, "gemm (qkv)")) != VIT_OK) return st;
  }

  // 3. residual: x, or pool4(h W_res^T + b_res) at a transition
  const void* r = x;
  if (d.q_stride == 4 && merged) {
    // written by the qkv GEMM
    if ((st = mark_empty(VIT_STAGE_RESIDUAL)) != VIT_OK) return st;
    r = r_out;
  } else if (d.q_stride == 4 && pool_gemm) {
    vit::GemmArgs gr;
    gr.A = h;
    gr.lda = Di;
    gr.M = (int)P.m_in;
    gr.N = Do;
    gr.K = Di;
    gr.W[0] = Wres;
    gr.bias[0] = w->b_res;
    gr.wscale[0] = q8 ? w->s_res : nullptr;
    gr.seg_cols = Do;
    gr.ldc = Do;
    gr.epi = vit::EPI_POOL;
    gr.tokens_per_frame = P.n_in;
    gr.pool_out = r_out;
    gr.ld_pool = Do;
    gr.pool_col0 = 0;
    e = vit::launch_gemm(gr, dt, s, stage_ev(VIT_STAGE_RESIDUAL));
    if ((st = device_status(e, "gemm (pooled residual projection)")) != VIT_OK) return st;
    r = r_out;
  } else if (d.q_stride == 4) {
    vit::GemmArgs gr;
    gr.A = h;
    gr.lda = Di;
    gr.M = (int)P.m_in;
    gr.N = Do;
    gr.K = Di;
    gr.W[0] = Wres;
    gr.bias[0] = w->b_res;
    gr.wscale[0] = q8 ? w->s_res : nullptr;
    gr.seg_cols = Do;
    gr.C = base + P.off_rp;
    gr.ldc = Do;
    gr.epi = vit::EPI_BIAS;
    e = vit::launch_gemm(gr, dt, s, only_start(stage_ev(VIT_STAGE_RESIDUAL)));
    if ((st = device_status(e, "gemm (residual projection)")) != VIT_OK) return st;
    void* rr = S.r ? S.r : base + P.off_r;
    e = vit::launch_pool4(base + P.off_rp, Do, rr, Do, d.batch, P.n_in, Do, dt, s,
                          only_stop(stage_ev(VIT_STAGE_RESIDUAL)));
    if ((st = device_status(e, "pool4 (residual)")) != VIT_OK) return st;
    r = rr;
  } else {
    // no kernel in this stage: mark it empty
    if ((st = mark_empty(VIT_STAGE_RESIDUAL)) != VIT_OK) return st;
    if (S.r) {
      e = hipMemcpyAsync(S.r, x, x_bytes, hipMemcpyDeviceToDevice, s);
      if ((st = device_status(e, "copy (r seam)")) != VIT_OK) return st;
    }
  }
  if (d.q_stride == 4 && S.q_pooled) {
    e = vit::launch_pool4(qkv, 3LL * Do, S.q_pooled, Do, d.batch, P.n_in, Do, dt, s);
    if ((st = device_status(e, "pool4 (q seam)")) != VIT_OK) return st;
  }


  // 4. attention
  vit::AttnArgs a;
  a.qkv = qkv;
  a.ld_qkv = 3 * Do;
  a.vt = P.attn_vt ? base + P.off_vt : nullptr;
  if (P.attn_hm) {
    a.qh = base + P.off_qh;
    a.kh = base + P.off_kh;
  }
  if (P.split_partials) {
    a.part_o = reinterpret_cast<float*>(base + P.off_po);
    a.part_ml = reinterpret_cast<float*>(base + P.off_pml);
  }
  a.ctx = ctx;
  a.ld_ctx = Do;
  a.batch = d.batch;
  a.tokens_in = P.n_in;
  a.tokens_out = P.n_out;
  a.dim = Do;
  a.heads = d.heads;
  a.head_dim = hd;
  a.mode = d.attn_mode;
  a.n_windows = d.n_windows;
  a.grid_w = d.grid_w;
  a.win_h = d.win_h;
  a.win_w = d.win_w;
  a.q_stride = d.q_stride;
  a.scale = attn_scale;
  e = vit::launch_attention(a, dt, s, stage_ev(VIT_STAGE_ATTN));
  if ((st = device_status(e, "attention")) != VIT_OK) return st;

  // 5. x1 = r + ctx W_o^T + b_o
  vit::GemmArgs go;
  go.A = ctx;
  go.lda = Do;
  go.M = (int)P.m_out;
  go.N = Do;
  go.K = Do;
  go.W[0] = Wo;
  go.bias[0] = w->b_o;
  go.wscale[0] = q8 ? w->s_o : nullptr;
  go.seg_cols = Do;
  go.C = x1;
  go.ldc = Do;
  go.epi = vit::EPI_BIAS_RES;
  go.res = r;
  go.ldres = Do;
  go.branch = S.attn_branch;
  go.ldbranch = Do;
  e = vit::launch_gemm(go, dt, s, stage_ev(VIT_STAGE_PROJ));
  if ((st = device_status(e, "gemm (out projection)")) != VIT_OK) return st;

  // 6. LN2
  e = vit::launch_layernorm(x1, h2, w->ln2_gamma, w->ln2_beta, P.m_out, Do, d.ln_eps, dt, s,
                            stage_ev(VIT_STAGE_LN2));
  if ((st = device_status(e, "layernorm (LN2)")) != VIT_OK) return st;

  // 7. u = GELU(h2 W_1^T + b_1)
  vit::GemmArgs g1;
  g1.A = h2;
  g1.lda = Do;
  g1.M = (int)P.m_out;
  g1.N = F;
  g1.K = Do;
  g1.W[0] = W1;
  g1.bias[0] = w->b_fc1;
  g1.wscale[0] = q8 ? w->s_fc1 : nullptr;
  g1.seg_cols = F;
  g1.C = u;
  g1.ldc = F;
  g1.epi = d.gelu == VIT_GELU_ERF ? vit::EPI_GELU_ERF : vit::EPI_GELU_TANH;
  e = vit::launch_gemm(g1, dt, s, stage_ev(VIT_STAGE_FC1));
  if ((st = device_status(e, "gemm (fc1)")) != VIT_OK) return st;

  // 8. y = x1 + u W_2^T + b_2
  vit::GemmArgs g2;
  g2.A = u;
  g2.lda = F;
  g2.M = (int)P.m_out;
  g2.N = Do;
  g2.K = F;
  g2.W[0] = W2;
  g2.bias[0] = w->b_fc2;
  g2.wscale[0] = q8 ? w->s_fc2 : nullptr;
  g2.seg_cols = Do;
  g2.C = y;
  g2.ldc = Do;
  g2.epi = vit::EPI_BIAS_RES;
  g2.res = x1;
  g2.ldres = Do;
  g2.branch = S.mlp_branch;
  g2.ldbranch = Do;
  e = vit::launch_gemm(g2, dt, s, stage_ev(VIT_STAGE_FC2));
  if ((st = device_status(e, "gemm (fc2)")) != VIT_OK) return st;
  if ((st = mark_empty(VIT_STAGE_FUSED)) != VIT_OK) return st;
  return ok();
}

VIT_API vit_status vit_block_forward(vit_block_t plan, const vit_block_weights* w, const void* x, void* y,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(plan, w, x, y, nullptr, workspace, workspace_bytes, stream);
}

VIT_API vit_status vit_block_forward_static(vit_block_t plan, const vit_block_weights* w, const void* x, void* y,
                                            void* stream) {
  if (!plan) return fail(VIT_ERR_INVALID_ARG, "plan is NULL");
  if (plan->ws_bytes > vit::STATIC_SCRATCH_BYTES)
    return fail(VIT_ERR_WORKSPACE,
                "this block needs %zu bytes of workspace; the library's static scratch holds %zu "
                "(use vit_block_forward with a caller workspace)",
                plan->ws_bytes, vit::STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  vit_status st = device_status(vit::static_scratch(&ws), "static scratch lookup");
  if (st != VIT_OK) return st;
  return forward_impl(plan, w, x, y, nullptr, ws, vit::STATIC_SCRATCH_BYTES, stream);
}

VIT_API vit_status vit_block_forward_timed(vit_block_t plan, const vit_block_weights* w, const void* x, void* y,
                                           void* workspace, size_t workspace_bytes, void* stream,
                                           void* const* events, int32_t n_events) {
  if (n_events < 0 || (n_events > 0 && !events)) return fail(VIT_ERR_INVALID_ARG, "bad events array");
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return fail(VIT_ERR_INVALID_ARG, "event %d is NULL", i);
  return forward_impl(plan, w, x, y, nullptr, workspace, workspace_bytes, stream, events, n_events);
}

VIT_API vit_status vit_block_forward_seams(vit_block_t plan, const vit_block_weights* w, const void* x, void* y,
                                           const vit_block_seams* seams, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (!seams) return fail(VIT_ERR_INVALID_ARG, "seams struct is NULL");
  return forward_impl(plan, w, x, y, seams, workspace, workspace_bytes, stream);
}

// ---- stack of blocks

struct vit_stack_plan {
  std::vector<vit_block_plan*> blocks;
  std::vector<int> taps, tap_levels, tap_grid_h, tap_grid_w;
  int levels0 = 0, batch = 0, esize = 2;
  int64_t tokens0 = 0;
  int dim0 = 0;
  size_t act_bytes = 0, ws_block = 0, ws_bytes = 0;
  ~vit_stack_plan() {
    for (vit_block_plan* b : blocks) delete b;
  }
};

VIT_API vit_status vit_stack_create(const vit_block_desc* blocks, int32_t n_blocks, int32_t unroll_levels,
                                    const int32_t* taps, int32_t n_taps, vit_stack_t* out) {
  if (!out) return fail(VIT_ERR_INVALID_ARG, "out handle pointer is NULL");
  if (!blocks || n_blocks < 1) return fail(VIT_ERR_INVALID_ARG, "need at least one block descriptor");
  if (unroll_levels < 0 || unroll_levels > 8) return fail(VIT_ERR_INVALID_ARG, "unroll_levels %d outside 0..8", unroll_levels);
  if (n_taps < 0 || (n_taps > 0 && !taps)) return fail(VIT_ERR_INVALID_ARG, "bad taps array");
  for (int k = 0; k < n_taps; ++k)
    if (taps[k] < 0 || taps[k] >= n_blocks || (k > 0 && taps[k] <= taps[k - 1]))
      return fail(VIT_ERR_INVALID_ARG, "taps must be increasing block indices (tap %d = %d)", k, taps[k]);
  const vit_block_desc& b0 = blocks[0];
  if (b0.grid_h % (1 << unroll_levels) || b0.grid_w % (1 << unroll_levels))
    return fail(VIT_ERR_INVALID_ARG, "grid %dx%d not divisible by 2^%d", b0.grid_h, b0.grid_w, unroll_levels);
  auto* sp = new (std::nothrow) vit_stack_plan();
  if (!sp) return fail(VIT_ERR_INVALID_ARG, "out of host memory");
  std::unique_ptr<vit_stack_plan> guard(sp);
  sp->levels0 = unroll_levels;
  sp->batch = b0.batch;
  sp->esize = b0.act_dtype == VIT_DTYPE_BF16 ? 2 : 4;
  sp->tokens0 = (int64_t)b0.grid_h * b0.grid_w;
  sp->dim0 = b0.dim_in;
  int levels = unroll_levels, k = 0;
  size_t act = 0;
  for (int i = 0; i < n_blocks; ++i) {
    const vit_block_desc& d = blocks[i];
    if (i > 0) {
      const vit_block_desc& pd = blocks[i - 1];
      const int gh = pd.grid_h / (pd.q_stride == 4 ? 2 : 1), gw = pd.grid_w / (pd.q_stride == 4 ? 2 : 1);
      if (d.batch != pd.batch || d.act_dtype != pd.act_dtype || d.grid_h != gh || d.grid_w != gw ||
          d.dim_in != pd.dim_out)
        return fail(VIT_ERR_INVALID_ARG, "block %d does not take block %d's output (batch, dtype, %dx%d grid, dim %d)",
                    i, i - 1, gh, gw, pd.dim_out);
    }
    if (d.attn_mode == VIT_ATTN_MASK_UNIT && levels < 1)
      return fail(VIT_ERR_INVALID_ARG, "block %d: mask units need an unrolled order, no level left", i);
    if (d.q_stride == 4 && levels < 1)
      return fail(VIT_ERR_INVALID_ARG, "block %d: a 2x2 pool needs an unroll level, none left", i);
    vit_block_t bp = nullptr;
    vit_status st = vit_block_create(&d, &bp);
    if (st != VIT_OK) {
      const std::string msg = g_err;
      return fail(st, "block %d: %s", i, msg.c_str());
    }
    sp->blocks.push_back(bp);
    const int64_t n_in = (int64_t)d.grid_h * d.grid_w, n_out = n_in / d.q_stride;
    act = std::max(act, (size_t)d.batch * n_in * d.dim_in * sp->esize);
    act = std::max(act, (size_t)d.batch * n_out * d.dim_out * sp->esize);
    sp->ws_block = std::max(sp->ws_block, bp->ws_bytes);
    if (d.q_stride == 4) --levels;
    if (k < n_taps && taps[k] == i) {
      sp->taps.push_back(i);
      sp->tap_levels.push_back(levels);
      sp->tap_grid_h.push_back(d.grid_h / (d.q_stride == 4 ? 2 : 1));
      sp->tap_grid_w.push_back(d.grid_w / (d.q_stride == 4 ? 2 : 1));
      ++k;
    }
  }
  sp->act_bytes = round256(act);
  sp->ws_bytes = 2 * sp->act_bytes + round256(sp->ws_block);
  *out = guard.release();
  return ok();
}

VIT_API vit_status vit_stack_workspace_size(vit_stack_t plan, size_t* bytes) {
  if (!plan || !bytes) return fail(VIT_ERR_INVALID_ARG, "plan or bytes pointer is NULL");
  *bytes = plan->ws_bytes;
  return ok();
}

VIT_API vit_status vit_stack_forward(vit_stack_t plan, const vit_block_weights* weights, const void* x,
                                     void* const* features, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(VIT_ERR_INVALID_ARG, "plan is NULL");
  const vit_stack_plan& P = *plan;
  if (!weights || !x) return fail(VIT_ERR_INVALID_ARG, "weights or x is NULL");
  if (!P.taps.empty() && !features) return fail(VIT_ERR_INVALID_ARG, "features array is NULL");
  if (workspace_bytes < P.ws_bytes) return fail(VIT_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, P.ws_bytes);
  if (!workspace || !aligned16(workspace)) return fail(VIT_ERR_WORKSPACE, "workspace is NULL or not 16-byte aligned");
  if (!aligned16(x)) return fail(VIT_ERR_INVALID_ARG, "x must be 16-byte aligned");
  const size_t x_bytes = (size_t)P.batch * P.tokens0 * P.dim0 * P.esize;
  if (overlaps(workspace, P.ws_bytes, x, x_bytes)) return fail(VIT_ERR_INVALID_ARG, "workspace overlaps x");
  for (size_t k = 0; k < P.taps.size(); ++k) {
    const vit_block_desc& d = P.blocks[P.taps[k]]->d;
    const size_t fb = (size_t)P.blocks[P.taps[k]]->m_out * d.dim_out * P.esize;
    if (!features[k] || !aligned16(features[k])) return fail(VIT_ERR_INVALID_ARG, "feature %zu is NULL or misaligned", k);
    if (overlaps(features[k], fb, workspace, P.ws_bytes) || overlaps(features[k], fb, x, x_bytes))
      return fail(VIT_ERR_INVALID_ARG, "feature %zu overlaps x or the workspace", k);
  }
  for (size_t i = 0; i < P.blocks.size(); ++i) {
    vit_status st = check_weights(P.blocks[i], &weights[i]);
    if (st != VIT_OK) {
      const std::string msg = g_err;
      return fail(st, "block %zu: %s", i, msg.c_str());
    }
  }
  char* base = (char*)workspace;
  void* buf[2] = {base, base + P.act_bytes};
  void* ws_b = base + 2 * P.act_bytes;
  const int32_t dt = P.blocks[0]->d.act_dtype;
  const vit_block_desc& b0 = P.blocks[0]->d;
  vit_status st = vit_unroll(x, buf[0], P.batch, b0.grid_h, b0.grid_w, P.levels0, P.dim0, dt, stream);
  if (st != VIT_OK) return st;
  int cur = 0;
  size_t k = 0;
  for (size_t i = 0; i < P.blocks.size(); ++i) {
    st = vit_block_forward(P.blocks[i], &weights[i], buf[cur], buf[cur ^ 1], ws_b, P.ws_block, stream);
    if (st != VIT_OK) {
      const std::string msg = g_err;
      return fail(st, "block %zu: %s", i, msg.c_str());
    }
    cur ^= 1;
    if (k < P.taps.size() && P.taps[k] == (int)i) {
      st = vit_reroll(buf[cur], features[k], P.batch, P.tap_grid_h[k], P.tap_grid_w[k], P.tap_levels[k],
                      P.blocks[i]->d.dim_out, dt, stream);
      if (st != VIT_OK) return st;
      ++k;
    }
  }
  return ok();
}

VIT_API vit_status vit_stack_destroy(vit_stack_t plan) {
  delete plan;
  return ok();
}

// ---- single steps

static vit_status check_dtype(int32_t dtype) {
  if (dtype != VIT_DTYPE_F32 && dtype != VIT_DTYPE_BF16) return fail(VIT_ERR_INVALID_ARG, "dtype %d is not a VIT_DTYPE_* value", dtype);
  return VIT_OK;
}

VIT_API vit_status vit_layernorm(const void* x, void* y, const float* gamma, const float* beta, int64_t rows,
                                 int32_t dim, float eps, int32_t dtype, void* stream) {
  vit_status st = check_dtype(dtype);
  if (st != VIT_OK) return st;
  if (rows < 0) return fail(VIT_ERR_INVALID_ARG, "rows < 0");
  if (dim < 8 || dim % 8 || dim > 8192) return fail(VIT_ERR_INVALID_ARG, "dim %d must be a multiple of 8 in [8, 8192]", dim);
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(VIT_ERR_INVALID_ARG, "eps must be positive and finite");
  if (rows == 0) return ok();
  if (!x || !y || !gamma || !beta) return fail(VIT_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(x) || !aligned16(y) || !aligned16(gamma) || !aligned16(beta))
    return fail(VIT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t bytes = (size_t)rows * dim * (dtype == VIT_DTYPE_BF16 ? 2 : 4);
  if (x != y && overlaps(x, bytes, y, bytes)) return fail(VIT_ERR_INVALID_ARG, "x and y overlap");
  const vit::DType dt = dtype == VIT_DTYPE_BF16 ? vit::DType::BF16 : vit::DType::F32;
  st = device_status(vit::launch_layernorm(x, y, gamma, beta, rows, dim, eps, dt, (hipStream_t)stream), "layernorm");
  return st == VIT_OK ? ok() : st;
}

static vit_status permute_common(const void* x, void* y, int32_t batch, int32_t gh, int32_t gw, int32_t levels,
                                 int32_t channels, int32_t dtype, void* stream, bool inverse) {
  vit_status st = check_dtype(dtype);
  if (st != VIT_OK) return st;
  if (batch < 0 || gh < 1 || gw < 1) return fail(VIT_ERR_INVALID_ARG, "bad batch or grid");
  if (levels < 0 || levels > 8) return fail(VIT_ERR_INVALID_ARG, "levels %d outside 0..8", levels);
  if (gh % (1 << levels) || gw % (1 << levels))
    return fail(VIT_ERR_INVALID_ARG, "grid %dx%d not divisible by 2^%d", gh, gw, levels);
  if (channels < 8 || channels % 8) return fail(VIT_ERR_INVALID_ARG, "channels %d must be a positive multiple of 8", channels);
  if (batch == 0) return ok();
  if (!x || !y) return fail(VIT_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(x) || !aligned16(y)) return fail(VIT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t bytes = (size_t)batch * gh * gw * channels * (dtype == VIT_DTYPE_BF16 ? 2 : 4);
  if (overlaps(x, bytes, y, bytes)) return fail(VIT_ERR_INVALID_ARG, "x and y overlap");
  const vit::DType dt = dtype == VIT_DTYPE_BF16 ? vit::DType::BF16 : vit::DType::F32;
  st = device_status(vit::launch_permute(x, y, batch, gh, gw, levels, channels, inverse, dt, (hipStream_t)stream),
                     inverse ? "reroll" : "unroll");
  return st == VIT_OK ? ok() : st;
}

VIT_API vit_status vit_unroll(const void* x, void* y, int32_t batch, int32_t grid_h, int32_t grid_w, int32_t levels,
                              int32_t channels, int32_t dtype, void* stream) {
  return permute_common(x, y, batch, grid_h, grid_w, levels, channels, dtype, stream, false);
}

VIT_API vit_status vit_reroll(const void* x, void* y, int32_t batch, int32_t grid_h, int32_t grid_w, int32_t levels,
                              int32_t channels, int32_t dtype, void* stream) {
  return permute_common(x, y, batch, grid_h, grid_w, levels, channels, dtype, stream, true);
}

VIT_API vit_status vit_pool4(const void* x, int64_t x_row_stride, void* y, int64_t y_row_stride, int32_t batch,
                             int32_t tokens, int32_t channels, int32_t dtype, void* stream) {
  vit_status st = check_dtype(dtype);
  if (st != VIT_OK) return st;
  if (batch < 0 || tokens < 0 || tokens % 4) return fail(VIT_ERR_INVALID_ARG, "tokens must be a non-negative multiple of 4");
  if (channels < 8 || channels % 8) return fail(VIT_ERR_INVALID_ARG, "channels %d must be a positive multiple of 8", channels);
  if (x_row_stride < channels || y_row_stride < channels || x_row_stride % 8 || y_row_stride % 8)
    return fail(VIT_ERR_INVALID_ARG, "row strides must be multiples of 8 and >= channels");
  if (batch == 0 || tokens == 0) return ok();
  if (!x || !y) return fail(VIT_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(x) || !aligned16(y)) return fail(VIT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t es = dtype == VIT_DTYPE_BF16 ? 2 : 4;
  if (overlaps(x, (size_t)batch * tokens * x_row_stride * es, y, (size_t)batch * (tokens / 4) * y_row_stride * es))
    return fail(VIT_ERR_INVALID_ARG, "x and y overlap");
  const vit::DType dt = dtype == VIT_DTYPE_BF16 ? vit::DType::BF16 : vit::DType::F32;
  st = device_status(vit::launch_pool4(x, x_row_stride, y, y_row_stride, batch, tokens, channels, dt, (hipStream_t)stream),
                     "pool4");
  return st == VIT_OK ? ok() : st;
}

// ---- patch-embedding stems ------------------------------------------------

static_assert(VIT_POS_NONE == vit::POS_NONE && VIT_POS_ROWS == vit::POS_ROWS && VIT_POS_BUCKET == vit::POS_BUCKET &&
                  VIT_POS_TILE == vit::POS_TILE,
              "position modes of the ABI and the GEMM epilogue");

namespace {

struct stem_geom {
  int out_h, out_w, K, Kp;
  int64_t M;
  size_t esize, a_bytes, w_bytes;  // workspace: gathered pixels, padded weight
  bool pad_weight;
};

vit_status stem_check(const vit_patch_embed_desc* d, stem_geom* g) {
  if (!d) return fail(VIT_ERR_INVALID_ARG, "desc is NULL");
  vit_status st = check_dtype(d->act_dtype);
  if (st != VIT_OK) return st;
  if (d->batch < 1) return fail(VIT_ERR_INVALID_ARG, "batch %d < 1", d->batch);
  if (d->in_h < 1 || d->in_w < 1 || d->in_ch < 1 || d->in_ch > 64)
    return fail(VIT_ERR_INVALID_ARG, "bad pixel shape %dx%dx%d", d->in_h, d->in_w, d->in_ch);
  if (d->pixel_layout != VIT_PIXELS_NCHW && d->pixel_layout != VIT_PIXELS_NHWC)
    return fail(VIT_ERR_INVALID_ARG, "unknown pixel layout %d", d->pixel_layout);
  if (d->weight_layout != VIT_CONV_OIHW && d->weight_layout != VIT_CONV_OHWI)
    return fail(VIT_ERR_INVALID_ARG, "unknown weight layout %d", d->weight_layout);
  if (d->kernel < 1 || d->kernel > 32 || d->stride < 1 || d->pad < 0 || d->pad >= d->kernel)
    return fail(VIT_ERR_INVALID_ARG, "kernel %d, stride %d, pad %d: need 1 <= kernel <= 32, stride >= 1, 0 <= pad < kernel",
                d->kernel, d->stride, d->pad);
  if (d->dim < 8 || d->dim % 8 || d->dim > 8192) return fail(VIT_ERR_INVALID_ARG, "dim %d must be a multiple of 8 in [8, 8192]", d->dim);
  g->out_h = d->in_h + 2 * d->pad >= d->kernel ? (d->in_h + 2 * d->pad - d->kernel) / d->stride + 1 : 0;
  g->out_w = d->in_w + 2 * d->pad >= d->kernel ? (d->in_w + 2 * d->pad - d->kernel) / d->stride + 1 : 0;
  if (g->out_h < 1 || g->out_w < 1) return fail(VIT_ERR_INVALID_ARG, "the kernel does not fit the padded image");
  switch (d->pos_mode) {
    case VIT_POS_NONE:
    case VIT_POS_ROWS: break;
    case VIT_POS_BUCKET:
      if (d->pos_side != g->out_h || d->pos_side != g->out_w)
        return fail(VIT_ERR_INVALID_ARG, "BUCKET positions need a square grid equal to pos_side (%d), got %dx%d",
                    d->pos_side, g->out_h, g->out_w);
      break;
    case VIT_POS_TILE:
      if (d->pos_side < 1) return fail(VIT_ERR_INVALID_ARG, "TILE positions need pos_side >= 1");
      break;
    default: return fail(VIT_ERR_INVALID_ARG, "unknown pos_mode %d", d->pos_mode);
  }
  g->K = d->in_ch * d->kernel * d->kernel;
  g->Kp = (g->K + 63) / 64 * 64;
  g->M = (int64_t)d->batch * g->out_h * g->out_w;
  if (g->M * g->Kp >= (int64_t(1) << 31)) return fail(VIT_ERR_UNSUPPORTED, "gathered matrix of %lld entries is too large",
                                                      (long long)(g->M * g->Kp));
  g->esize = d->act_dtype == VIT_DTYPE_BF16 ? 2 : 4;
  g->pad_weight = g->K != g->Kp;
  g->a_bytes = round256((size_t)g->M * g->Kp * g->esize);
  g->w_bytes = g->pad_weight ? round256((size_t)d->dim * g->Kp * g->esize) : 0;
  return VIT_OK;
}

}  // namespace

VIT_API vit_status vit_patch_embed_workspace_size(const vit_patch_embed_desc* desc, size_t* bytes) {
  if (!bytes) return fail(VIT_ERR_INVALID_ARG, "bytes is NULL");
  stem_geom g;
  vit_status st = stem_check(desc, &g);
  if (st != VIT_OK) return st;
  *bytes = g.a_bytes + g.w_bytes;
  return ok();
}

VIT_API vit_status vit_patch_embed(const vit_patch_embed_desc* desc, const float* pixels, const void* weight,
                                   const float* bias, const float* pos, void* tokens, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  stem_geom g;
  vit_status st = stem_check(desc, &g);
  if (st != VIT_OK) return st;
  const vit_patch_embed_desc& d = *desc;
  if (!pixels || !weight || !tokens) return fail(VIT_ERR_INVALID_ARG, "pixels, weight and tokens must not be NULL");
  if (d.pos_mode != VIT_POS_NONE && !pos) return fail(VIT_ERR_INVALID_ARG, "pos is NULL but pos_mode is not NONE");
  if (!aligned16(pixels) || !aligned16(weight) || !aligned16(tokens) || (bias && !aligned16(bias)) ||
      (pos && !aligned16(pos)))
    return fail(VIT_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (workspace_bytes < g.a_bytes + g.w_bytes)
    return fail(VIT_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, g.a_bytes + g.w_bytes);
  if (!workspace || !aligned16(workspace)) return fail(VIT_ERR_WORKSPACE, "workspace is NULL or not 16-byte aligned");
  const size_t pix_bytes = (size_t)d.batch * d.in_h * d.in_w * d.in_ch * 4;
  const size_t tok_bytes = (size_t)g.M * d.dim * g.esize;
  const size_t ws = g.a_bytes + g.w_bytes;
  if (overlaps(tokens, tok_bytes, pixels, pix_bytes) || overlaps(tokens, tok_bytes, workspace, ws) ||
      overlaps(workspace, ws, pixels, pix_bytes))
    return fail(VIT_ERR_INVALID_ARG, "tokens, pixels and workspace must not overlap");
  const vit::DType dt = d.act_dtype == VIT_DTYPE_BF16 ? vit::DType::BF16 : vit::DType::F32;
  const hipStream_t s = (hipStream_t)stream;
  char* base = static_cast<char*>(workspace);
  void* A = base;
  const void* W = weight;
  void* Wp = g.pad_weight ? base + g.a_bytes : nullptr;
  st = device_status(vit::launch_im2col(pixels, d.pixel_layout == VIT_PIXELS_NHWC, d.batch, d.in_ch, d.in_h, d.in_w,
                                        d.kernel, d.stride, d.pad, d.weight_layout == VIT_CONV_OHWI, A, g.Kp, dt, s,
                                        g.pad_weight ? weight : nullptr, Wp, d.dim),
                     "im2col");
  if (st != VIT_OK) return st;
  if (g.pad_weight) W = Wp;
  vit::GemmArgs a;
  a.A = A;
  a.lda = g.Kp;
  a.W[0] = W;
  a.bias[0] = bias;
  a.seg_cols = d.dim;
  a.C = tokens;
  a.ldc = d.dim;
  a.M = (int)g.M;
  a.N = d.dim;
  a.K = g.Kp;
  a.epi = vit::EPI_BIAS_POS;
  a.tokens_per_frame = g.out_h * g.out_w;
  a.grid_w = g.out_w;
  a.pos = d.pos_mode == VIT_POS_NONE ? nullptr : pos;
  a.pos_mode = d.pos_mode;
  a.pos_side = d.pos_side;
  st = device_status(vit::launch_gemm(a, dt, s), "patch-embed GEMM");
  return st == VIT_OK ? ok() : st;
}
