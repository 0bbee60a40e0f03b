// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vit {

enum class DType { F32 = 0, BF16 = 1 };

// The library's own device scratch (scratch.hip): STATIC_SCRATCH_BYTES on
// every GPU, for vit_block_forward_static. static_scratch() returns its
// address on the current device (looked up on the first call there).
constexpr size_t STATIC_SCRATCH_BYTES = size_t(256) << 20;
hipError_t static_scratch(void** ptr);

// Optional events for measurement: `start` takes the first kernel's begin
// time and `stop` the last kernel's end time (hipExtLaunchKernel timestamps
// from the dispatch packets, so no extra packets enter the stream).
struct StageEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

enum Epilogue {
  EPI_BIAS = 0,        // C = acc + bias
  EPI_BIAS_ROPE = 1,   // C = rope(acc + bias) on columns < rope_cols
  EPI_GELU_ERF = 2,    // C = gelu_erf(acc + bias)
  EPI_GELU_TANH = 3,   // C = gelu_tanh(acc + bias)
  EPI_BIAS_RES = 4,    // C = res + (acc + bias); branch = acc + bias if set
  EPI_BIAS_POS = 5,    // C = acc + bias + pos[row(token)] (bias and pos may be NULL)
  EPI_POOL = 6,        // columns < pool_col0: C = acc + bias; the rest 2x2-max-pooled
                       // into pool_out (see GemmArgs)
};

// Position-table row of token t = y * grid_w + x of a frame (EPI_BIAS_POS):
// POS_ROWS t; POS_BUCKET max(y-1,0) * pos_side + max(x-1,0); POS_TILE
// (y mod pos_side) * pos_side + (x mod pos_side). Values match the C ABI's
// VIT_POS_*.
enum PosMode { POS_NONE = 0, POS_ROWS = 1, POS_BUCKET = 2, POS_TILE = 3 };

// C[M, N] = epilogue(A[M, K] * W[N, K]^T + bias). W and bias may be split
// into up to three column segments of seg_cols columns each (separate q/k/v
// weights), four with EPI_POOL; with one segment seg_cols = N.
struct GemmArgs {
  const void* A = nullptr;
  int64_t lda = 0;
  const void* W[4] = {nullptr, nullptr, nullptr, nullptr};
  const float* bias[4] = {nullptr, nullptr, nullptr, nullptr};
  int seg_cols = 0;
  void* C = nullptr;
  int64_t ldc = 0;
  int M = 0, N = 0, K = 0;
  int epi = EPI_BIAS;
  // EPI_BIAS_RES
  const void* res = nullptr;
  int64_t ldres = 0;
  void* branch = nullptr;
  int64_t ldbranch = 0;
  // EPI_BIAS_ROPE: table [rows, head_dim/2, 2]; token t of a frame uses row
  // t (rope_mode 0) or its in-window raster index (rope_mode 1).
  const float* rope = nullptr;
  int rope_cols = 0, head_dim = 0, rope_mode = 0;
  int tokens_per_frame = 1, grid_w = 1, win_h = 1, win_w = 1;
  // EPI_BIAS / EPI_BIAS_ROPE: columns >= vt_col0 (V, bias only) are also
  // written transposed to vt [M / vt_tokens, vt_heads, vt_hd, vt_tokens];
  // with vt_only they are not written to C. Needs the bf16 MFMA path
  // (gemm_uses_mfma), M and vt_tokens multiples of 8, vt_col0 a multiple of 8.
  void* vt = nullptr;
  int vt_col0 = 0, vt_tokens = 0, vt_heads = 0, vt_hd = 0;
  bool vt_only = false;
  // Head-major attention operands (with vt, head_dim vt_hd = 64): columns
  // < vt_col0 / 2 (q, after RoPE) times hm_qscale go to hm_q, columns
  // vt_col0 / 2 .. vt_col0 - 1 (k) to hm_k, both [frame, window, head, i, 64]
  // with i the token's index inside its attention window; vt then takes the
  // same window order, [frame, window, head, 64, i]. Windows are the whole
  // frame, or (hm_spatial) the win_h x win_w tiles of a grid grid_w wide
  // (win_w a multiple of 8). With vt_only, q and k are not written to C.
  void* hm_q = nullptr;
  void* hm_k = nullptr;
  float hm_qscale = 1.f;
  bool hm_spatial = false;
  // EPI_BIAS_POS: float32 table [rows, N]; frames of tokens_per_frame tokens
  // on a grid grid_w wide
  const float* pos = nullptr;
  int pos_mode = POS_NONE, pos_side = 0;
  // optional float16 scale per weight row (output column), segment-wise
  // like W: acc[m, n] * wscale[n] before the bias (integer-valued W rows
  // of q8_row weights)
  const void* wscale[4] = {nullptr, nullptr, nullptr, nullptr};
  // EPI_POOL (bf16 MFMA path only): A rows are frames of tokens_per_frame
  // tokens (a multiple of 4; M a multiple of it). Columns >= pool_col0 (a
  // multiple of 8) are not written to C: pool_out[f * T/4 + t, n - pool_col0]
  // = max over s < 4 of (acc + bias)[f * T + s * T/4 + t, n] (the Hiera
  // query pool over the four unrolled quarters of a frame), ld_pool apart.
  void* pool_out = nullptr;
  int64_t ld_pool = 0;
  int pool_col0 = 0;
};
hipError_t launch_gemm(const GemmArgs& a, DType dt, hipStream_t s, StageEvents ev = {});
// The bf16 MFMA path takes K >= 64 with K % 16 == 0 (a last K tile of 16,
// 32 or 48 columns runs that many MFMA K steps) and 16-byte aligned A rows;
// other shapes and fp32 run the VALU kernel. The V^T output needs this path.
inline bool gemm_uses_mfma(DType dt, int K, int64_t lda) {
  return dt == DType::BF16 && K >= 64 && K % 16 == 0 && lda % 8 == 0;
}

enum AttnMode { ATTN_GLOBAL = 0, ATTN_MASK_UNIT = 1, ATTN_SPATIAL = 2 };

struct AttnArgs {
  const void* qkv = nullptr;  // [B * tokens_in, 3 * dim], rows [q | k | v]
  // Head-major operands written by the qkv projection (GemmArgs::hm_q):
  // when qh is set, q (pre-multiplied by scale * log2 e), k and vt are read
  // in window order, [B, windows, heads, n, 64] and [B, windows, heads, 64,
  // n]; needs attention_takes_hm()
  const void* qh = nullptr;
  const void* kh = nullptr;
  // V transposed, [B, heads, head_dim, tokens_in]: given exactly when
  // attention_takes_vt() holds, and then read in place of qkv's V columns
  const void* vt = nullptr;
  // key-split partials, needed when attention_splits() > 1 (vt path):
  // part_o [splits, B*tokens_out, dim], part_ml [splits, B*tokens_out, heads, 2], fp32
  float* part_o = nullptr;
  float* part_ml = nullptr;
  int64_t ld_qkv = 0;
  void* ctx = nullptr;        // [B * tokens_out, dim]
  int64_t ld_ctx = 0;
  int batch = 1, tokens_in = 0, tokens_out = 0, dim = 0, heads = 1, head_dim = 0;
  int mode = ATTN_GLOBAL, n_windows = 1, grid_w = 1, win_h = 1, win_w = 1;
  int q_stride = 1;
  float scale = 1.f;
};
// Patch-embedding gather: A[m, kk] (m = (frame, y, x) of the output grid,
// kk < C*k*k in the weight's flattening order, (c, ky, kx) for OIHW or
// (ky, kx, c) for OHWI; zero outside the image and for kk >= C*k*k) for
// float32 pixels [B, C, H, W] (nhwc false) or [B, H, W, C]; A is [M, Kp].
// With wsrc, the same launch also copies the weight rows wsrc [wrows, C*k*k]
// into wdst [wrows, Kp], zero-filling the tail.
hipError_t launch_im2col(const float* pixels, bool nhwc, int batch, int C, int H, int W, int k, int s, int p,
                         bool ohwi, void* A, int Kp, DType dt, hipStream_t st, const void* wsrc = nullptr,
                         void* wdst = nullptr, int wrows = 0, StageEvents ev = {});

// Exact conversion of int8 arrays to the activation type (q8_row payloads
// before their GEMMs): up to 6 segments, each a multiple of 16 elements,
// 16-byte aligned, in one launch.
struct I8Segments {
  const int8_t* src[6] = {};
  void* dst[6] = {};
  int64_t n[6] = {};
  int count = 0;
};
hipError_t launch_i8_convert(const I8Segments& sg, DType dt, hipStream_t s, StageEvents ev = {});

hipError_t launch_attention(const AttnArgs& a, DType dt, hipStream_t s, StageEvents ev = {});

// Large global or spatial windows go to the 32x32-MFMA attention kernel,
// which streams K and V^T tiles straight into LDS: bf16, >= 128 queries per
// window, head_dim <= 64, frame token count and (spatial) window width
// multiples of 8 (16-byte runs of consecutive keys in V^T), 32-bit element
// offsets into qkv.
// Large-window attention on a small grid (fewer than 256 workgroups of 128
// queries) splits each window's keys over several workgroups, each with at
// least two 64-key tiles; a second kernel merges the partial softmaxes.
inline int attention_splits(int64_t batch, int64_t windows, int64_t n_q, int64_t n_kv, int64_t heads) {
  const int64_t blocks = batch * windows * ((n_q + 127) / 128) * heads;
  const int64_t tiles = (n_kv + 63) / 64;
  if (blocks <= 0 || blocks >= 256) return 1;
  int64_t s = (256 + blocks - 1) / blocks;
  s = s < tiles / 2 ? s : tiles / 2;
  s = s < 8 ? s : 8;
  return s >= 2 ? (int)s : 1;
}

// A split of 2 or 4 over at most 1024 keys runs among the four waves of one
// workgroup (no fp32 partials, no combine launch); other splits write
// partials (AttnArgs::part_o, part_ml) that a combine launch merges.
inline bool attention_split_in_workgroup(int splits, int64_t n_kv) {
  return (splits == 2 || splits == 4) && n_kv <= 16 * 64;
}

// Large windows with head_dim 64 and no query pool: the head-major kernel
// (operands in window order from the qkv projection; no key split).
inline bool attention_takes_hm(DType dt, int mode, int64_t n_q, int head_dim, int win_w, int64_t tokens_in,
                               int q_stride) {
  return dt == DType::BF16 && (mode == ATTN_GLOBAL || (mode == ATTN_SPATIAL && win_w % 8 == 0)) && n_q >= 128 &&
         head_dim == 64 && tokens_in % 8 == 0 && q_stride == 1;
}

inline bool attention_takes_vt(DType dt, int mode, int64_t n_q, int head_dim, int win_w, int64_t tokens_in,
                               int64_t qkv_elems) {
  return dt == DType::BF16 && (mode == ATTN_GLOBAL || (mode == ATTN_SPATIAL && win_w % 8 == 0)) && n_q >= 128 &&
         head_dim <= 64 && tokens_in % 8 == 0 && qkv_elems < (1LL << 31);
}

// Whole block for 64-token mask units of width <= 128 in one kernel
// (q_stride 1): x [B*tokens, dim] -> y, one workgroup per (frame, window).
struct FusedMUArgs {
  const void* x = nullptr;
  void* y = nullptr;
  const float *ln1_g = nullptr, *ln1_b = nullptr, *ln2_g = nullptr, *ln2_b = nullptr;
  const void *wq = nullptr, *wk = nullptr, *wv = nullptr;
  const float *bq = nullptr, *bk = nullptr, *bv = nullptr;
  const void* wo = nullptr;
  const float* bo = nullptr;
  const void* w1 = nullptr;
  const float* b1 = nullptr;
  const void* w2 = nullptr;
  const float* b2 = nullptr;
  int batch = 1, tokens = 0, n_windows = 1, dim = 0, heads = 1, head_dim = 0, mlp = 0;
  float eps = 1e-6f, scale = 1.f;
  bool gelu_tanh = false;
  // q8_row weights: the w* are int8 payloads, these their float16 row scales
  bool q8 = false;
  const void *sq = nullptr, *sk = nullptr, *sv = nullptr, *so = nullptr, *s1 = nullptr, *s2 = nullptr;
};
bool fused_mask_unit_supported(int dim, int heads, int head_dim, int mlp, int window_tokens);
size_t fused_mask_unit_lds_bytes(int dim, int mlp);
hipError_t launch_block_mask_unit_fused(const FusedMUArgs& a, hipStream_t s, StageEvents ev = {});

hipError_t launch_layernorm(const void* x, void* y, const float* g, const float* b,
                            int64_t rows, int dim, float eps, DType dt, hipStream_t s,
                            StageEvents ev = {});
hipError_t launch_permute(const void* x, void* y, int batch, int grid_h, int grid_w,
                          int levels, int channels, bool inverse, DType dt, hipStream_t s);
// vt [B, heads, head_dim, tokens] from the V columns (col0 + h*head_dim + d)
// of qkv rows [B*tokens, ld] (bf16; tokens and head_dim multiples of 8).
hipError_t launch_v_transpose(const void* qkv, int64_t ld, int col0, void* vt, int batch, int tokens, int heads,
                              int head_dim, hipStream_t s, StageEvents ev = {});
hipError_t launch_pool4(const void* x, int64_t x_stride, void* y, int64_t y_stride,
                        int batch, int tokens, int channels, DType dt, hipStream_t s,
                        StageEvents ev = {});

}  // namespace vit
