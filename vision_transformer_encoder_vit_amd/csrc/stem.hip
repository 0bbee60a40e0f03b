// Patch-embedding stems: the strided convolution that turns pixels into the
// token grid, run as a gather (im2col) into a [tokens, K] matrix followed by
// the MFMA GEMM, whose epilogue adds the bias and the position table row of
// each token. Sources: the Hiera plan ("Phase 4: Hiera Backbone MLX Port",
// "Architecture Summary": PatchEmbed Conv2d 4->112, 7x7, stride 4, then the
// learned pos_embed); the SigLIP page (``embed_frame``: k16 s16 conv with
// bias, position rows from bucketized coordinates); the SAM3 page (trunk
// patch step: k14 s14 conv without bias, a 24x24 table tiled over the grid,
// then ln_pre).
//
// The gather writes row m = (frame, y, x) of A with its K = C*k*k pixels in
// the weight's own flattening order -- (c, ky, kx) for OIHW weights,
// (ky, kx, c) for OHWI -- so the weight is used as the GEMM's [N, K] operand
// without any transpose; K is padded with zeros to a multiple of 64 (the
// MFMA GEMM's K tile), and the weight rows are padded to match, in the same
// launch, when K is not already a multiple of 64.
#include "common.h"
#include "launch.h"

#include <hip/hip_ext.h>

namespace vit {

struct Im2colParams {
  int64_t M;  // frames * out_h * out_w
  int C, H, W, k, s, p, out_h, out_w;
  int K, Kp;  // C*k*k and its padded width
  int nhwc, ohwi;
  // optional weight rows padded from K to Kp by the same launch (workgroups
  // past the gather's): wsrc [wrows, K] -> wdst [wrows, Kp]
  const void* wsrc;
  void* wdst;
  int wrows;
  unsigned gather_blocks;
};

// One thread per 16-byte chunk of an A row (8 bf16 or 4 float entries):
// consecutive threads write consecutive chunks of a row. Entries outside
// the image (the zero padding) and past K are zero. The chunk's first entry
// is located with two divisions, the rest by stepping the (c, ky, kx) or
// (ky, kx, c) indices; runs of 4 pixels that are contiguous in memory and
// 16-byte aligned (4 pixels of an NCHW kernel row, or the 4 channels of one
// NHWC pixel) are read with one 16-byte load.
template <typename T>
__global__ __launch_bounds__(256) void im2col_kernel(const float* __restrict__ px, T* __restrict__ A,
                                                     Im2colParams q) {
  constexpr int VN = Vec<T>::N;
  const int cpr = q.Kp / VN;
  if (blockIdx.x >= q.gather_blocks) {  // weight padding, one chunk per thread
    const int64_t wid = (int64_t)(blockIdx.x - q.gather_blocks) * 256 + threadIdx.x;
    const int64_t r = wid / cpr;
    if (r >= q.wrows) return;
    const int c0 = (int)(wid - r * cpr) * VN;
    const T* ws = static_cast<const T*>(q.wsrc);
    float f[VN];
#pragma unroll
    for (int e = 0; e < VN; ++e) f[e] = c0 + e < q.K ? to_f32(ws[r * q.K + c0 + e]) : 0.f;
    st16(static_cast<T*>(q.wdst) + r * q.Kp + c0, pack16<T>(f));
    return;
  }
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t m = id / cpr;
  if (m >= q.M) return;
  const int chunk = (int)(id - m * cpr);
  const int T_ = q.out_h * q.out_w;
  const int b = (int)(m / T_), t = (int)(m - (int64_t)b * T_);
  const int y = t / q.out_w, x = t - y * q.out_w;
  const int y0 = y * q.s - q.p, x0 = x * q.s - q.p;
  const int kk0 = chunk * VN;
  float v[VN];
  int c, ky, kx;
  if (q.ohwi) {
    const int kc = q.k * q.C;
    ky = kk0 / kc;
    const int r = kk0 - ky * kc;
    kx = r / q.C;
    c = r - kx * q.C;
  } else {
    const int kk2 = q.k * q.k;
    c = kk0 / kk2;
    const int r = kk0 - c * kk2;
    ky = r / q.k;
    kx = r - ky * q.k;
  }
  // groups of 4 entries: one 16-byte load where the run allows it, else
  // four single loads, stepping the indices either way
#pragma unroll
  for (int g = 0; g < VN / 4; ++g) {
    const int kk = kk0 + 4 * g;
    int py = y0 + ky, pxx = x0 + kx;
    if (q.ohwi && q.C == 4 && c == 0) {
      // the 4 channels of one NHWC pixel
      f32x4 pv = {0.f, 0.f, 0.f, 0.f};
      if (kk < q.K && py >= 0 && py < q.H && pxx >= 0 && pxx < q.W)
        pv = *reinterpret_cast<const f32x4*>(px + (((int64_t)b * q.H + py) * q.W + pxx) * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * g + j] = pv[j];
      if (++kx == q.k) { kx = 0; ++ky; }
      continue;
    }
    if (!q.ohwi && (kx & 3) == 0 && kx + 4 <= q.k && kk + 4 <= q.K && ((x0 + kx) & 3) == 0 && (q.W & 3) == 0 &&
        py >= 0 && py < q.H && pxx >= 0 && pxx + 4 <= q.W) {
      // four pixels of one NCHW kernel row, contiguous and aligned
      const f32x4 pv = *reinterpret_cast<const f32x4*>(px + (((int64_t)b * q.C + c) * q.H + py) * q.W + pxx);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * g + j] = pv[j];
      kx += 4;
      if (kx == q.k) { kx = 0; if (++ky == q.k) { ky = 0; ++c; } }
      continue;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      py = y0 + ky;
      pxx = x0 + kx;
      const bool inside = kk + j < q.K && py >= 0 && py < q.H && pxx >= 0 && pxx < q.W;
      if (q.ohwi) {
        v[4 * g + j] = inside ? px[(((int64_t)b * q.H + py) * q.W + pxx) * q.C + c] : 0.f;
        if (++c == q.C) { c = 0; if (++kx == q.k) { kx = 0; ++ky; } }
      } else {
        v[4 * g + j] = inside ? px[(((int64_t)b * q.C + c) * q.H + py) * q.W + pxx] : 0.f;
        if (++kx == q.k) { kx = 0; if (++ky == q.k) { ky = 0; ++c; } }
      }
    }
  }
  st16(A + m * q.Kp + kk0, pack16<T>(v));
}

hipError_t launch_im2col(const float* pixels, bool nhwc, int batch, int C, int H, int W, int k, int s, int p,
                         bool ohwi, void* A, int Kp, DType dt, hipStream_t st, const void* wsrc, void* wdst,
                         int wrows, StageEvents ev) {
  Im2colParams q;
  q.C = C;
  q.H = H;
  q.W = W;
  q.k = k;
  q.s = s;
  q.p = p;
  q.out_h = (H + 2 * p - k) / s + 1;
  q.out_w = (W + 2 * p - k) / s + 1;
  q.M = (int64_t)batch * q.out_h * q.out_w;
  q.K = C * k * k;
  q.Kp = Kp;
  q.nhwc = nhwc;
  q.ohwi = ohwi;
  const int vn = dt == DType::BF16 ? 8 : 4;
  const int64_t threads = q.M * (Kp / vn);
  q.gather_blocks = (unsigned)((threads + 255) / 256);
  q.wsrc = wsrc;
  q.wdst = wdst;
  q.wrows = wsrc ? wrows : 0;
  const int64_t wthreads = (int64_t)q.wrows * (Kp / vn);
  dim3 grid(q.gather_blocks + (unsigned)((wthreads + 255) / 256)), block(256);
  if (dt == DType::BF16)
    hipExtLaunchKernelGGL(im2col_kernel<bf16>, grid, block, 0, st, ev.start, ev.stop, 0, pixels, (bf16*)A, q);
  else
    hipExtLaunchKernelGGL(im2col_kernel<float>, grid, block, 0, st, ev.start, ev.stop, 0, pixels, (float*)A, q);
  return hipGetLastError();
}

}  // namespace vit
