/*
 * vit_block.h -- C ABI of the MI355X (gfx950) pre-LayerNorm ViT encoder block.
 *
 * The operation (one block over the patch tokens of B frames):
 *
 *   h   = LN1(x)                         row LayerNorm, biased variance
 *   r   = x                              or, at a Hiera stage transition
 *                                        (q_stride 4): r = pool4(h W_res^T + b_res)
 *   qkv = h W_qkv^T + b_qkv              one fused projection, rows [q | k | v],
 *                                        or three separate projections
 *   q,k <- axial RoPE(q, k)              optional, (cos, sin) table per token
 *   q   <- pool4(q)                      q_stride 4 only
 *   ctx = softmax(q k^T * scale) v       per frame, window and head, non-causal
 *   x1  = r + ctx W_o^T + b_o
 *   y   = x1 + GELU(LN2(x1) W_1^T + b_1) W_2^T + b_2     GELU: erf or tanh form
 *
 * Sources of each step (the pages this library was built from):
 *  - SigLIP-B/16 vision tower (franken_ocr 0.8.0 vision_siglip.rs): the
 *    pre-LN block `encoder_block`, separate q/k/v/out projections with bias
 *    and non-causal attention `self_attention`, tanh-GELU, LN eps 1e-6,
 *    frames batched with no cross-frame attention.
 *  - SAM3 image model (cortiq-engine 0.8.44 sam3.rs): `layer_norm_rows`,
 *    fused qkv with rows laid out [q | k | v] and per-head column blocks
 *    (`run_attn`), stable softmax, `apply_rope` (pairs (2j, 2j+1) of each
 *    head, first half of the pairs on the x position, second half on y),
 *    24x24 windows of the 72x72 trunk grid (`vit_windows`), erf-GELU.
 *  - Hiera backbone plan (corridorkey-mrp-mlx "Phase 4: Hiera Backbone MLX
 *    Port"): MaskUnitAttention (windows over the unrolled token order, max
 *    pool of the queries over the q_stride axis at stage transitions), the
 *    transition's projection + max-pool of the residual, MLP fc1-GELU-fc2,
 *    Unroll/Reroll token permutations.
 *
 * Conventions for every entry point
 *  - Every pointer argument that names a tensor is a DEVICE pointer (memory
 *    from hipMalloc or a torch tensor on the GPU), 16-byte aligned. The
 *    caller owns all device memory; the library never allocates device
 *    memory and keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls enqueue kernels and return without synchronising; errors found on
 *    the host (arguments, shapes) are reported before anything is enqueued,
 *    and then no output is touched. A failed kernel launch returns
 *    VIT_ERR_DEVICE.
 *  - Activations and weight matrices are in the block's activation dtype
 *    (VIT_DTYPE_F32 = IEEE float32, VIT_DTYPE_BF16 = bfloat16 bits);
 *    LayerNorm gamma/beta, biases and the RoPE table are always float32.
 *    Accumulation is float32 in both cases.
 *  - Matrices are row-major. Weights use the PyTorch Linear layout
 *    [out_features, in_features].
 *  - Token rows are row-major [B, N, C] with frames contiguous. In GLOBAL and
 *    SPATIAL modes token n of a frame is the grid position (n / grid_w,
 *    n % grid_w). In MASK_UNIT mode the tokens are in Hiera's unrolled order
 *    (see vit_unroll), and the block's output is in the unrolled order of its
 *    output grid.
 *  - vit_last_error() returns a message for the last failed call on the
 *    calling thread ("" if none). The string is valid until the next call.
 */
#ifndef VIT_BLOCK_H
#define VIT_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vit_status {
  VIT_OK = 0,
  VIT_ERR_INVALID_ARG = 1, /* bad pointer, size, shape or alignment */
  VIT_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels cover */
  VIT_ERR_WORKSPACE = 3,   /* workspace pointer missing or too small */
  VIT_ERR_DEVICE = 4       /* a HIP call or kernel launch failed */
} vit_status;

enum { VIT_DTYPE_F32 = 0, VIT_DTYPE_BF16 = 1 };
enum { VIT_ATTN_GLOBAL = 0, VIT_ATTN_MASK_UNIT = 1, VIT_ATTN_SPATIAL = 2 };
enum { VIT_GELU_ERF = 0, VIT_GELU_TANH = 1 };
enum { VIT_QKV_FUSED = 0, VIT_QKV_SEPARATE = 1 };
enum { VIT_ROPE_NONE = 0, VIT_ROPE_AXIAL_TABLE = 1 };
/* Weight matrix storage. Q8_ROW is the SAM3 page's `q8_row` tensor type
 * (cortiq-engine sam3.rs, `bad_scales`: a [rows, cols] payload of one byte
 * per element followed by one float16 scale per row): here the int8 payload
 * and the scales are two arrays, and W[r, c] = payload[r, c] * scale[r].
 * Each forward first copies the payloads into the workspace as act_dtype
 * (exact: |q| <= 128 has at most 8 significant bits), the GEMMs multiply
 * them with float32 accumulation and apply the scale per output column
 * before the bias, so the result is that of the dequantized matrix up to
 * float32 rounding. Any act_dtype; the single-kernel mask-unit path is not
 * used with Q8_ROW. */
enum { VIT_WEIGHTS_ACT = 0, VIT_WEIGHTS_Q8_ROW = 1 };

/* Shape and options of one block. Validated by vit_block_create. */
typedef struct vit_block_desc {
  int32_t batch;       /* frames B >= 1 (zero frames is an error, as in the
                          SigLIP tower's frame-count check)                */
  int32_t grid_h;      /* input token grid; N_in = grid_h * grid_w          */
  int32_t grid_w;
  int32_t dim_in;      /* D_in: width of x, LN1, the qkv/res projections' K */
  int32_t dim_out;     /* D_out: attention, LN2 and MLP width (= dim_in
                          unless q_stride == 4)                             */
  int32_t heads;       /* head_dim = dim_out / heads, a multiple of 8, <= 64 */
  int32_t mlp_hidden;  /* fc1 output width                                  */
  int32_t attn_mode;   /* VIT_ATTN_*                                        */
  int32_t n_windows;   /* MASK_UNIT: windows per frame; kv token n belongs to
                          window n mod n_windows (query token m likewise, in
                          the pooled order when q_stride == 4)              */
  int32_t win_h;       /* SPATIAL: window size; the grid must divide evenly */
  int32_t win_w;
  int32_t q_stride;    /* 1, or 4 (Hiera transition: 2x2 max-pool of the
                          queries and of the projected residual; N_out = N_in/4;
                          MASK_UNIT or GLOBAL only)                          */
  int32_t gelu;        /* VIT_GELU_ERF or VIT_GELU_TANH                     */
  int32_t qkv_layout;  /* VIT_QKV_FUSED or VIT_QKV_SEPARATE                 */
  int32_t rope;        /* VIT_ROPE_NONE or VIT_ROPE_AXIAL_TABLE (GLOBAL or
                          SPATIAL, head_dim % 4 == 0)                        */
  int32_t rope_rows;   /* table rows: win_h*win_w (SPATIAL) or N_in (GLOBAL) */
  float ln_eps;        /* LayerNorm epsilon (> 0), e.g. 1e-6                */
  float attn_scale;    /* softmax scale; 0 means head_dim^-1/2              */
  int32_t act_dtype;   /* VIT_DTYPE_F32 or VIT_DTYPE_BF16                   */
  int32_t weight_format; /* VIT_WEIGHTS_ACT (0): matrices in act_dtype;
                          VIT_WEIGHTS_Q8_ROW: int8 matrices with a float16
                          scale per output row (see vit_block_weights)     */
} vit_block_desc;

/* Device pointers to one block's parameters. Unused members may be NULL.
 * Matrices in act_dtype, [out, in] row-major; vectors float32. */
typedef struct vit_block_weights {
  const float* ln1_gamma;  /* [dim_in]  */
  const float* ln1_beta;   /* [dim_in]  */
  const void* w_res;       /* [dim_out, dim_in]  (q_stride 4 only) */
  const float* b_res;      /* [dim_out]          (q_stride 4 only) */
  const void* w_qkv;       /* [3*dim_out, dim_in] (FUSED)    */
  const float* b_qkv;      /* [3*dim_out]         (FUSED)    */
  const void* w_q;         /* [dim_out, dim_in]   (SEPARATE) */
  const float* b_q;
  const void* w_k;
  const float* b_k;
  const void* w_v;
  const float* b_v;
  const void* w_o;         /* [dim_out, dim_out] */
  const float* b_o;        /* [dim_out] */
  const float* ln2_gamma;  /* [dim_out] */
  const float* ln2_beta;   /* [dim_out] */
  const void* w_fc1;       /* [mlp_hidden, dim_out] */
  const float* b_fc1;      /* [mlp_hidden] */
  const void* w_fc2;       /* [dim_out, mlp_hidden] */
  const float* b_fc2;      /* [dim_out] */
  const float* rope_table; /* [rope_rows, head_dim/2, 2] (cos, sin) */
  /* VIT_WEIGHTS_Q8_ROW only: float16 scale per row of the matching int8
   * matrix ([out_features] each); ignored otherwise */
  const void* s_res;
  const void* s_qkv;
  const void* s_q;
  const void* s_k;
  const void* s_v;
  const void* s_o;
  const void* s_fc1;
  const void* s_fc2;
} vit_block_weights;

/* Optional caller buffers for the block's intermediates (all act_dtype,
 * row-major, NULL = not wanted). Rows: M_in = B*N_in, M_out = B*N_out.
 *   h           [M_in,  dim_in]     LN1 output
 *   qkv         [M_in,  3*dim_out]  projections after bias and RoPE, [q|k|v]
 *   q_pooled    [M_out, dim_out]    pooled queries (q_stride 4)
 *   r           [M_out, dim_out]    residual: x, or the pooled projection
 *   ctx         [M_out, dim_out]    attention output before W_o
 *   attn_branch [M_out, dim_out]    ctx W_o^T + b_o (before the residual)
 *   x1          [M_out, dim_out]
 *   h2          [M_out, dim_out]    LN2 output
 *   u           [M_out, mlp_hidden] GELU(fc1) output
 *   mlp_branch  [M_out, dim_out]    u W_2^T + b_2 (before the residual)   */
typedef struct vit_block_seams {
  void* h;
  void* qkv;
  void* q_pooled;
  void* r;
  void* ctx;
  void* attn_branch;
  void* x1;
  void* h2;
  void* u;
  void* mlp_branch;
} vit_block_seams;

typedef struct vit_block_plan* vit_block_t;

/* Validate `desc` and build a host-side plan (tile choices, workspace
 * layout). `*out` receives the handle. The plan holds no device memory and
 * is immutable: forwards on different streams with distinct workspaces may
 * run concurrently. */
vit_status vit_block_create(const vit_block_desc* desc, vit_block_t* out);

/* Bytes of device workspace a forward needs (a multiple of 256). */
vit_status vit_block_workspace_size(vit_block_t plan, size_t* bytes);

/* One block forward: x [B*N_in, dim_in] -> y [B*N_out, dim_out].
 * y may equal x when q_stride == 1 (in place); any other overlap between
 * y, x, the weights and the workspace is an error. */
vit_status vit_block_forward(vit_block_t plan, const vit_block_weights* w,
                             const void* x, void* y, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Maximum workspace of vit_block_forward_static: the library's own device
 * scratch, 256 MiB on every GPU the library runs on (held from the first
 * call on that GPU until the process ends). */
#define VIT_STATIC_SCRATCH_BYTES ((size_t)256 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): as
 * vit_block_forward, with the workspace taken from the library's static
 * device scratch instead of the caller. Allocates nothing (no hipMalloc,
 * hipFree or allocating library call); the first call on a device looks the
 * scratch up there. Fails with VIT_ERR_WORKSPACE, before any launch, when
 * the plan's workspace (vit_block_workspace_size) exceeds
 * VIT_STATIC_SCRATCH_BYTES. Every call on one GPU uses that GPU's single
 * scratch and leaves its contents behind; nothing in it needs to start at
 * zero. Calls that overlap on one GPU (other streams, other threads) race
 * on the scratch: the caller serialises them. */
vit_status vit_block_forward_static(vit_block_t plan, const vit_block_weights* w,
                                    const void* x, void* y, void* stream);

/* As vit_block_forward, and also writes every non-NULL seam buffer. It
 * always runs the step-by-step kernels (one per stage), so where
 * vit_block_forward uses the single fused kernel (bf16 mask units of 64
 * tokens, width <= 128, q_stride 1) y differs from it by rounding only;
 * otherwise the two are bit-identical. */
vit_status vit_block_forward_seams(vit_block_t plan, const vit_block_weights* w,
                                   const void* x, void* y,
                                   const vit_block_seams* seams, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Stages of one forward, in launch order (for vit_block_forward_timed). */
enum {
  VIT_STAGE_LN1 = 0,      /* LayerNorm of x                              */
  VIT_STAGE_QKV = 1,      /* qkv projection (+ bias, + RoPE); at a bf16
                             transition without RoPE or V^T output it also
                             computes the pooled residual projection, and
                             VIT_STAGE_RESIDUAL is then empty           */
  VIT_STAGE_RESIDUAL = 2, /* transition: residual projection + 4x pool    */
  VIT_STAGE_ATTN = 3,     /* windowed / global attention                  */
  VIT_STAGE_PROJ = 4,     /* out projection + bias + residual             */
  VIT_STAGE_LN2 = 5,      /* LayerNorm of x1                              */
  VIT_STAGE_FC1 = 6,      /* fc1 + bias + GELU                            */
  VIT_STAGE_FC2 = 7,      /* fc2 + bias + residual                        */
  VIT_STAGE_FUSED = 8,    /* the whole block in one kernel (small mask units;
                             the other stages are then empty)              */
  VIT_NSTAGES = 9
};

/* As vit_block_forward, for measurement: `events` holds n_events hipEvent_t
 * handles created by the caller (hipEventCreate); for stage i (VIT_STAGE_*)
 * with 2i+1 < n_events, events[2i] takes the begin timestamp of the stage's
 * first kernel and events[2i+1] the end timestamp of its last kernel (the
 * kernels are launched with hipExtLaunchKernel's start/stop events, so no
 * marker packets are added to the stream), and hipEventElapsedTime(events[2i],
 * events[2i+1]) is the stage's device time. A stage with no kernel (the
 * residual stage outside transitions) records both events back to back on
 * `stream`. The result is bit-identical to vit_block_forward. */
vit_status vit_block_forward_timed(vit_block_t plan, const vit_block_weights* w,
                                   const void* x, void* y, void* workspace,
                                   size_t workspace_bytes, void* stream,
                                   void* const* events, int32_t n_events);

/* Which stages (bit i = VIT_STAGE_i) launch kernels in vit_block_forward
 * and vit_block_forward_timed for this plan; the others record empty
 * events. */
vit_status vit_block_stage_mask(vit_block_t plan, uint32_t* mask);

vit_status vit_block_destroy(vit_block_t plan);

const char* vit_last_error(void);

/* ---- a stack of blocks over one token grid (Hiera plan, "Architecture
 * Summary" and "Implementation Plan" item 8: Unroll once, the blocks in
 * order, Reroll at each stage end) ---- */

typedef struct vit_stack_plan* vit_stack_t;

/* Plan `n_blocks` blocks applied in order. Block 0 reads x [B, grid_h*grid_w,
 * dim_in] in raster order, which is first unrolled with `unroll_levels` 2x2
 * levels (the block descriptors see the unrolled order, as MASK_UNIT needs);
 * every block with q_stride 4 halves the grid and uses up one level. After
 * block taps[k] (increasing) its output is rerolled with the levels left
 * into feature k, raster order [B, H_k*W_k, dim_out]. Block i+1 must take
 * block i's output: same batch and dtype, its grid_h/grid_w the halved grid
 * after a transition, dim_in = dim_out. Errors as vit_block_create, plus a
 * chain that does not connect, levels that run out (q_stride 4 or
 * MASK_UNIT with no level left) or bad taps. Holds no device memory. */
vit_status vit_stack_create(const vit_block_desc* blocks, int32_t n_blocks,
                            int32_t unroll_levels, const int32_t* taps,
                            int32_t n_taps, vit_stack_t* out);

/* Bytes of device workspace a stack forward needs (two activation buffers
 * and the largest block workspace; a multiple of 256). */
vit_status vit_stack_workspace_size(vit_stack_t plan, size_t* bytes);

/* Run the stack: weights[i] for block i; features[k] receives tap k (all
 * 16-byte aligned, not overlapping x or the workspace). Asynchronous on
 * `stream`, like vit_block_forward. */
vit_status vit_stack_forward(vit_stack_t plan, const vit_block_weights* weights,
                             const void* x, void* const* features,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

vit_status vit_stack_destroy(vit_stack_t plan);

/* ---- single steps (same kernels the block uses) ---- */

/* Row LayerNorm (SAM3 `layer_norm_rows`): y = (x - mean) / sqrt(var + eps)
 * * gamma + beta, biased variance, float32 statistics. x, y [rows, dim],
 * dim a multiple of 8 and <= 8192; y may equal x. */
vit_status vit_layernorm(const void* x, void* y, const float* gamma,
                         const float* beta, int64_t rows, int32_t dim,
                         float eps, int32_t dtype, void* stream);

/* Hiera Unroll (Hiera plan, "Architecture Summary": permutes the spatial
 * tokens for mask-unit attention). x [batch, grid_h*grid_w, channels] in
 * row-major spatial order -> y in the unrolled order: the token at (i, j)
 * moves to n = (((s_0*4 + s_1)*4 + ...)*4 + s_{L-1}) * (H_L*W_L)
 *            + (i >> L) * W_L + (j >> L),
 * s_k = 2*((i >> k) & 1) + ((j >> k) & 1), H_L = grid_h >> L,
 * W_L = grid_w >> L, L = levels (0..8). grid_h, grid_w divisible by 2^L;
 * channels a multiple of 8. Bit-exact copy. y must not overlap x. */
vit_status vit_unroll(const void* x, void* y, int32_t batch, int32_t grid_h,
                      int32_t grid_w, int32_t levels, int32_t channels,
                      int32_t dtype, void* stream);

/* Hiera Reroll: the inverse of vit_unroll (unrolled order -> row-major
 * spatial order), same arguments. */
vit_status vit_reroll(const void* x, void* y, int32_t batch, int32_t grid_h,
                      int32_t grid_w, int32_t levels, int32_t channels,
                      int32_t dtype, void* stream);

/* 4x max-pool over the q_stride axis of the unrolled order (Hiera
 * MaskUnitAttention's query pooling; a 2x2 spatial max): for every frame,
 * y[m, c] = max_s x[s*tokens/4 + m, c], s = 0..3, m < tokens/4.
 * Row strides in elements (>= channels, multiples of 8); channels a
 * multiple of 8; tokens a multiple of 4. Bit-exact. */
vit_status vit_pool4(const void* x, int64_t x_row_stride, void* y,
                     int64_t y_row_stride, int32_t batch, int32_t tokens,
                     int32_t channels, int32_t dtype, void* stream);

/* ---- patch-embedding stems (the step that makes the token grid) ----
 *
 *   tokens[b, y*out_w + x, o] = bias[o] + pos[row(y, x), o]
 *       + sum_{c,ky,kx} w[o, c, ky, kx] * P[b, c, y*stride + ky - pad, x*stride + kx - pad]
 *
 * with P zero outside the image and out_h = (in_h + 2 pad - kernel) / stride
 * + 1 (likewise out_w). Sources: the Hiera plan ("Architecture Summary":
 * PatchEmbed Conv2d 4->112, 7x7, stride 4, then the learned pos_embed, one
 * row per token); the SigLIP page (`embed_frame`: Conv 3->768, 16x16, stride
 * 16, with bias, then position rows from bucketized patch coordinates); the
 * SAM3 page (trunk: Conv 3->1024, 14x14, stride 14, no bias, then a 24x24
 * position table tiled over the 72x72 grid; its ln_pre is vit_layernorm).
 */
enum { VIT_PIXELS_NCHW = 0, VIT_PIXELS_NHWC = 1 };
enum { VIT_CONV_OIHW = 0, VIT_CONV_OHWI = 1 };
/* Position-table row of output token (y, x):
 *   ROWS    y*out_w + x   (table [out_h*out_w, dim])
 *   BUCKET  max(y-1,0)*pos_side + max(x-1,0)   (table [pos_side^2, dim];
 *           the SigLIP NaViT bucketize at the full-mask geometry, where
 *           coordinates 0 and 1 share bucket 0; needs out_h = out_w = pos_side)
 *   TILE    (y mod pos_side)*pos_side + (x mod pos_side)   (table [pos_side^2, dim]) */
enum { VIT_POS_NONE = 0, VIT_POS_ROWS = 1, VIT_POS_BUCKET = 2, VIT_POS_TILE = 3 };

typedef struct vit_patch_embed_desc {
  int32_t batch;          /* frames >= 1                                    */
  int32_t in_h, in_w;     /* pixel grid                                     */
  int32_t in_ch;          /* channels C, 1..64 (3 RGB; 4 for Hiera)          */
  int32_t pixel_layout;   /* VIT_PIXELS_NCHW [B, C, H, W] or _NHWC [B, H, W, C] */
  int32_t kernel;         /* square kernel k, 1..32                         */
  int32_t stride;         /* >= 1                                           */
  int32_t pad;            /* zero padding on every side, 0 <= pad < kernel  */
  int32_t dim;            /* output channels, a multiple of 8, <= 8192      */
  int32_t weight_layout;  /* VIT_CONV_OIHW [dim, C, k, k] or _OHWI [dim, k, k, C] */
  int32_t pos_mode;       /* VIT_POS_*                                      */
  int32_t pos_side;       /* BUCKET and TILE: side of the square table      */
  int32_t act_dtype;      /* dtype of weight and tokens: VIT_DTYPE_F32 or _BF16 */
} vit_patch_embed_desc;

/* Bytes of device workspace vit_patch_embed needs for `desc` (the gathered
 * [B*out_h*out_w, K] pixel matrix, K = C*k*k padded to a multiple of 64, and
 * the weight padded to the same K when C*k*k is not a multiple of 64; a
 * multiple of 256). Validates desc as vit_patch_embed does. */
vit_status vit_patch_embed_workspace_size(const vit_patch_embed_desc* desc, size_t* bytes);

/* Run a stem. pixels: float32 in pixel_layout (bf16 stems round them to
 * bf16 as matrix operands); weight: act_dtype in weight_layout; bias:
 * float32 [dim] or NULL; pos: float32 table (rows as pos_mode says) or NULL
 * when pos_mode is NONE; tokens: [B, out_h*out_w, dim] act_dtype, raster
 * order. Accumulation in float32; bias and position are added before the one
 * rounding to act_dtype. All pointers device, 16-byte aligned; tokens must
 * not overlap pixels or the workspace. Errors: VIT_ERR_INVALID_ARG for a bad
 * descriptor (also a BUCKET grid that is not pos_side x pos_side) or
 * pointer, VIT_ERR_WORKSPACE, VIT_ERR_UNSUPPORTED when the gathered matrix
 * reaches 2^31 entries. Asynchronous on `stream`. */
vit_status vit_patch_embed(const vit_patch_embed_desc* desc, const float* pixels,
                           const void* weight, const float* bias, const float* pos,
                           void* tokens, void* workspace, size_t workspace_bytes,
                           void* stream);

#ifdef __cplusplus
}
#endif
#endif /* VIT_BLOCK_H */
