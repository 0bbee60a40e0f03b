// Dense projections of the block on MFMA: C = epilogue(A W^T + bias).
//
// A [M, K] (token rows) and W [N, K] (PyTorch Linear layout) are both
// K-contiguous, so both MFMA operands are 16-byte LDS reads of 8 bf16 (or 4
// float) along K. The MFMA's A operand is the W tile and its B operand the
// token tile, so each lane ends with 4 consecutive output COLUMNS of one
// token row: the bias, a RoPE pair (2j, 2j+1), GELU and the residual all
// work on lane-local registers, and stores are 8-byte (bf16) vectors.
//
// Workgroup: 256 threads = 4 waves (2 x 2), tile BM x BN, K step of 128
// bytes per row; double-buffered LDS (rows padded by 16 bytes so the
// 16-lane column reads of an MFMA fragment hit distinct banks); the next K
// tile is fetched into registers while the current one is multiplied.
#include "common.h"
#include "launch.h"

#include <hip/hip_ext.h>

namespace vit {

template <typename T>
struct GemmParams {
  const T* A;
  int64_t lda;
  const T* W0;
  const T* W1;
  const T* W2;
  const float* b0;
  const float* b1;
  const float* b2;
  int seg_cols;
  T* C;
  int64_t ldc;
  int M, N, K;
  const T* res;
  int64_t ldres;
  T* branch;
  int64_t ldbranch;
  const float* rope;
  int rope_cols, head_dim, rope_mode, tokens_per_frame, grid_w, win_h, win_w;
};

__device__ __forceinline__ float gelu_erf_f(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_tanh_f(float v) {
  return 0.5f * v * (1.0f + tanhf(0.79788456080286536f * (v + 0.044715f * v * v * v)));
}

template <typename T, int BM, int BN, int WTM, int WTN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams<T> p) {
  constexpr int VN = Vec<T>::N;              // elements per 16 bytes
  constexpr int BK = 8 * VN;                 // 128 bytes of K per tile row
  constexpr int BKP = BK + VN;               // padded LDS row (144 bytes)
  constexpr int KSTEPS = BK / Mma<T>::KSTEP;  // MFMA K steps per tile (2)
  constexpr int WAVES_N = BN / (16 * WTN);
  constexpr int WAVES_M = BM / (16 * WTM);
  static_assert(WAVES_N * WAVES_M == 4, "4 waves per workgroup");
  constexpr int XL = BM / 32;  // 16-byte loads per thread per tile (tokens)
  constexpr int WL = BN / 32;  // (weights)

  __shared__ __attribute__((aligned(16))) T Xs[2][BM][BKP];
  __shared__ __attribute__((aligned(16))) T Ws[2][BN][BKP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % WAVES_N, wm = wave / WAVES_N;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x % tiles_n;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  // global -> register staging: thread owns chunk c of rows r, r+32, ...
  const int c = tid & 7, r = tid >> 3;
  const T* xrow[XL];
  const T* wrow[WL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int m = m0 + r + 32 * i;
    xrow[i] = m < p.M ? p.A + (int64_t)m * p.lda : nullptr;
  }
#pragma unroll
  for (int i = 0; i < WL; ++i) {
    const int n = n0 + r + 32 * i;
    if (n < p.N) {
      const int seg = n / p.seg_cols;
      const T* base = seg == 0 ? p.W0 : (seg == 1 ? p.W1 : p.W2);
      wrow[i] = base + (int64_t)(n - seg * p.seg_cols) * p.K;
    } else {
      wrow[i] = nullptr;
    }
  }
  u32x4 xreg[XL], wreg[WL];
  auto fetch = [&](int kt) {
    const int k = kt * BK + c * VN;
    const bool kin = k < p.K;
#pragma unroll
    for (int i = 0; i < XL; ++i) xreg[i] = (xrow[i] && kin) ? ld16(xrow[i] + k) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < WL; ++i) wreg[i] = (wrow[i] && kin) ? ld16(wrow[i] + k) : u32x4{0, 0, 0, 0};
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XL; ++i) st16(&Xs[buf][r + 32 * i][c * VN], xreg[i]);
#pragma unroll
    for (int i = 0; i < WL; ++i) st16(&Ws[buf][r + 32 * i][c * VN], wreg[i]);
  };

  f32x4 acc[WTN][WTM];
#pragma unroll
  for (int i = 0; i < WTN; ++i)
#pragma unroll
    for (int j = 0; j < WTM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ktiles = (p.K + BK - 1) / BK;
  fetch(0);
  stash(0);
  __syncthreads();
  const int fr = lane & 15, g = lane >> 4;
  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) fetch(kt + 1);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int col = (ks * 4 + g) * VN;
      u32x4 af[WTN], bfr[WTM];
#pragma unroll
      for (int i = 0; i < WTN; ++i) af[i] = ld16(&Ws[buf][wn * WTN * 16 + i * 16 + fr][col]);
#pragma unroll
      for (int j = 0; j < WTM; ++j) bfr[j] = ld16(&Xs[buf][wm * WTM * 16 + j * 16 + fr][col]);
#pragma unroll
      for (int i = 0; i < WTN; ++i)
#pragma unroll
        for (int j = 0; j < WTM; ++j) acc[i][j] = Mma<T>::step(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < ktiles) stash(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds columns n..n+3 of token row m for every (i, j)
#pragma unroll
  for (int j = 0; j < WTM; ++j) {
    const int m = m0 + wm * WTM * 16 + j * 16 + fr;
    if (m >= p.M) continue;
    int rope_row = 0;
    if (EPI == EPI_BIAS_ROPE) {
      const int t = m % p.tokens_per_frame;
      if (p.rope_mode == 1) {
        const int yy = t / p.grid_w, xx = t % p.grid_w;
        rope_row = (yy % p.win_h) * p.win_w + (xx % p.win_w);
      } else {
        rope_row = t;
      }
    }
#pragma unroll
    for (int i = 0; i < WTN; ++i) {
      const int n = n0 + wn * WTN * 16 + i * 16 + 4 * g;
      if (n >= p.N) continue;
      const int seg = n / p.seg_cols;
      const float* bb = seg == 0 ? p.b0 : (seg == 1 ? p.b1 : p.b2);
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(bb + (n - seg * p.seg_cols));
      f32x4 v = acc[i][j] + b4;
      if (EPI == EPI_BIAS_ROPE) {
        if (n < p.rope_cols) {
          const int d = (n % (p.rope_cols / 2)) % p.head_dim;  // even, pair d/2 and d/2+1
          const f32x4 cs = *reinterpret_cast<const f32x4*>(p.rope + ((int64_t)rope_row * (p.head_dim / 2) + d / 2) * 2);
          const float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
          v[0] = a0 * cs[0] - a1 * cs[1];
          v[1] = a1 * cs[0] + a0 * cs[1];
          v[2] = a2 * cs[2] - a3 * cs[3];
          v[3] = a3 * cs[2] + a2 * cs[3];
        }
      } else if (EPI == EPI_GELU_ERF) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = gelu_erf_f(v[e]);
      } else if (EPI == EPI_GELU_TANH) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = gelu_tanh_f(v[e]);
      } else if (EPI == EPI_BIAS_RES) {
        if (p.branch) store4<T>(p.branch + (int64_t)m * p.ldbranch + n, v);
        v = v + load4<T>(p.res + (int64_t)m * p.ldres + n);
      }
      store4<T>(p.C + (int64_t)m * p.ldc + n, v);
    }
  }
}

template <typename T, int BM, int BN, int WTM, int WTN>
static hipError_t gemm_go(const GemmArgs& a, hipStream_t s, StageEvents ev) {
  GemmParams<T> p;
  p.A = (const T*)a.A;
  p.lda = a.lda;
  p.W0 = (const T*)a.W[0];
  p.W1 = (const T*)(a.W[1] ? a.W[1] : a.W[0]);
  p.W2 = (const T*)(a.W[2] ? a.W[2] : a.W[0]);
  p.b0 = a.bias[0];
  p.b1 = a.bias[1] ? a.bias[1] : a.bias[0];
  p.b2 = a.bias[2] ? a.bias[2] : a.bias[0];
  p.seg_cols = a.seg_cols > 0 ? a.seg_cols : a.N;
  p.C = (T*)a.C;
  p.ldc = a.ldc;
  p.M = a.M;
  p.N = a.N;
  p.K = a.K;
  p.res = (const T*)a.res;
  p.ldres = a.ldres;
  p.branch = (T*)a.branch;
  p.ldbranch = a.ldbranch;
  p.rope = a.rope;
  p.rope_cols = a.rope_cols;
  p.head_dim = a.head_dim;
  p.rope_mode = a.rope_mode;
  p.tokens_per_frame = a.tokens_per_frame;
  p.grid_w = a.grid_w;
  p.win_h = a.win_h;
  p.win_w = a.win_w;
  const int64_t tiles = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  dim3 grid((unsigned)tiles), block(256);
  switch (a.epi) {
    case EPI_BIAS: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_BIAS>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_BIAS_ROPE: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_BIAS_ROPE>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_GELU_ERF: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_GELU_ERF>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_GELU_TANH: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_GELU_TANH>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    default: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_BIAS_RES>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, DType dt, hipStream_t s, StageEvents ev) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (dt == DType::F32) return gemm_go<float, 64, 64, 2, 2>(a, s, ev);
  const int64_t big_tiles = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
  if (big_tiles >= 512) return gemm_go<bf16, 128, 128, 4, 4>(a, s, ev);
  return gemm_go<bf16, 64, 64, 2, 2>(a, s, ev);
}

}  // namespace vit
