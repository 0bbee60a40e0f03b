// Bandwidth-bound row kernels: LayerNorm, Hiera unroll/reroll permutes and
// the 4x max-pool. Each row is handled by a group of G lanes that move it in
// 16-byte vectors, so every global access is a coalesced 16-byte load/store.
#include "common.h"
#include "launch.h"

#include <hip/hip_ext.h>

#include <type_traits>

namespace vit {

// the permutes are stage-boundary copies whose output is not read back at
// once: non-temporal stores (measured +7 % on HBM-resident working sets; the
// same stores slow down a consumer kernel that reads the data right away)
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }
// pool4 reads each source row once: non-temporal loads (measured 0.663 ->
// 0.771 of the HBM peak on HBM-resident rows; the same hint on LayerNorm's
// loads or on pool4's stores was slower)
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Sum over each aligned group of G lanes: DPP within 16-lane rows, then the
// row-pair and wave-half swaps; narrower groups use LDS shuffles.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 16) {
    v = row16_sum(v);
    if constexpr (G >= 32) v = pair16_sum(v);
    if constexpr (G >= 64) v = pair32_sum(v);
  } else {
#pragma unroll
    for (int m = G / 2; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  }
  return v;
}

// Row LayerNorm (SAM3 layer_norm_rows): mean, biased variance over the row,
// (x - mean) / sqrt(var + eps) * gamma + beta. Statistics in float32, two
// passes over the values held in registers; gamma and beta are read with x,
// so their latency hides behind the reductions (inv_dim = 1 / dim, and the
// hardware reciprocal square root, ~1 ulp, instead of divisions).
template <typename T, int G, int V>
__global__ __launch_bounds__(256) void layernorm_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ beta,
                                                        int64_t rows, int dim, float inv_dim, float eps) {
  constexpr int VN = Vec<T>::N;
  const int lane = threadIdx.x % G;
  const int64_t row = (int64_t)blockIdx.x * (256 / G) + threadIdx.x / G;
  if (row >= rows) return;  // whole group exits together (G divides 64)
  const int nvec = dim / VN;
  const T* xr = x + row * dim;
  float v[V][VN];
  // (rows of more than 2 vectors per lane read gamma and beta at use: held
  // early they would cost 2 VN registers per vector and, on the wide rows of
  // the bandwidth-bound launches, occupancy)
  constexpr bool GB_EARLY = V <= 2;
  constexpr int VG = GB_EARLY ? V : 1;
  f32x4 g4[VG][VN / 4], b4[VG][VN / 4];
#pragma unroll
  for (int i = 0; i < VG; ++i) {
    const int vi = lane + i * G;
    if (GB_EARLY && vi < nvec) {
#pragma unroll
      for (int e = 0; e < VN; e += 4) {
        g4[i][e / 4] = *reinterpret_cast<const f32x4*>(gamma + vi * VN + e);
        b4[i][e / 4] = *reinterpret_cast<const f32x4*>(beta + vi * VN + e);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int vi = lane + i * G;
    if (vi < nvec) {
      unpack16<T>(ld16(xr + vi * VN), v[i]);
#pragma unroll
      for (int e = 0; e < VN; ++e) s += v[i][e];
    } else {
#pragma unroll
      for (int e = 0; e < VN; ++e) v[i][e] = 0.f;
    }
  }
  s = group_sum<G>(s);
  const float mean = s * inv_dim;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (lane + i * G < nvec) {
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        const float d = v[i][e] - mean;
        q += d * d;
      }
    }
  }
  q = group_sum<G>(q);
  const float inv = __builtin_amdgcn_rsqf(q * inv_dim + eps);
  T* yr = y + row * dim;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int vi = lane + i * G;
    if (vi < nvec) {
      float o[VN];
#pragma unroll
      for (int e = 0; e < VN; e += 4) {
        f32x4 gg, bb;
        if constexpr (GB_EARLY) {
          gg = g4[i][e / 4];
          bb = b4[i][e / 4];
        } else {
          gg = *reinterpret_cast<const f32x4*>(gamma + vi * VN + e);
          bb = *reinterpret_cast<const f32x4*>(beta + vi * VN + e);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) o[e + j] = (v[i][e + j] - mean) * inv * gg[j] + bb[j];
      }
      st16(yr + vi * VN, pack16<T>(o));
    }
  }
}

template <typename T, int G, int V>
static hipError_t ln_launch(const void* x, void* y, const float* g, const float* b, int64_t rows,
                            int dim, float eps, hipStream_t s, StageEvents ev) {
  const int rpb = 256 / G;
  const int64_t blocks = (rows + rpb - 1) / rpb;
  hipExtLaunchKernelGGL((layernorm_kernel<T, G, V>), dim3((unsigned)blocks), dim3(256), 0, s, ev.start,
                        ev.stop, 0, (const T*)x, (T*)y, g, b, rows, dim, 1.0f / (float)dim, eps);
  return hipGetLastError();
}

template <typename T>
static hipError_t ln_dispatch(const void* x, void* y, const float* g, const float* b, int64_t rows,
                              int dim, float eps, hipStream_t s, StageEvents ev) {
  const int nvec = dim / Vec<T>::N;
  // rows of 96 vectors (768 bf16): 32 lanes x 3 loads leave no lane idle
  // (64 x 2 would idle half the wave on the second load); measured faster
  if (nvec == 96) return ln_launch<T, 32, 3>(x, y, g, b, rows, dim, eps, s, ev);
  if (nvec <= 4) return ln_launch<T, 4, 1>(x, y, g, b, rows, dim, eps, s, ev);
  if (nvec <= 8) return ln_launch<T, 8, 1>(x, y, g, b, rows, dim, eps, s, ev);
  if (nvec <= 16) return ln_launch<T, 16, 1>(x, y, g, b, rows, dim, eps, s, ev);
  if (nvec <= 32) return ln_launch<T, 32, 1>(x, y, g, b, rows, dim, eps, s, ev);
  if (nvec <= 64) return ln_launch<T, 64, 1>(x, y, g, b, rows, dim, eps, s, ev);
  if (nvec <= 128) return ln_launch<T, 64, 2>(x, y, g, b, rows, dim, eps, s, ev);
  if (nvec <= 256) return ln_launch<T, 64, 4>(x, y, g, b, rows, dim, eps, s, ev);
  if (nvec <= 512) return ln_launch<T, 64, 8>(x, y, g, b, rows, dim, eps, s, ev);
  if (nvec <= 1024) return ln_launch<T, 64, 16>(x, y, g, b, rows, dim, eps, s, ev);
  return ln_launch<T, 64, 32>(x, y, g, b, rows, dim, eps, s, ev);  // float rows up to 8192
}

hipError_t launch_layernorm(const void* x, void* y, const float* g, const float* b, int64_t rows,
                            int dim, float eps, DType dt, hipStream_t s, StageEvents ev) {
  if (rows == 0) return hipSuccess;
  return dt == DType::BF16 ? ln_dispatch<bf16>(x, y, g, b, rows, dim, eps, s, ev)
                           : ln_dispatch<float>(x, y, g, b, rows, dim, eps, s, ev);
}

// Unrolled position of the spatial token (i, j) on an H x W grid with L
// levels: each level appends the token's 2x2 offset 2*(i&1) + (j&1) to an
// outer index and halves the coordinates; the position is the outer index
// times the size of the coarse grid plus the token's coarse raster index.
__device__ __forceinline__ int64_t unrolled_pos(int i, int j, int H, int W, int L) {
  int64_t outer = 0;
  for (int k = 0; k < L; ++k) {
    outer = outer * 4 + 2 * (i & 1) + (j & 1);
    i >>= 1;
    j >>= 1;
  }
  const int64_t HL = H >> L, WL = W >> L;
  return outer * (HL * WL) + (int64_t)i * WL + j;
}

// Row permutation between the spatial order and Hiera's unrolled order. A
// group of G lanes copies one token row; the group is indexed by the spatial
// token, so unroll scatters rows and reroll gathers them. Bit-exact copy.
template <int G>
__global__ __launch_bounds__(256) void permute_kernel(const uint8_t* __restrict__ x, uint8_t* __restrict__ y,
                                                      int batch, int H, int W, int L,
                                                      int row_bytes, int inverse) {
  const int lane = threadIdx.x % G;
  const int64_t t = (int64_t)blockIdx.x * (256 / G) + threadIdx.x / G;
  const int64_t ntok = (int64_t)H * W;
  if (t >= (int64_t)batch * ntok) return;
  const int64_t b = t / ntok;
  const int sp = (int)(t - b * ntok);
  const int64_t un = unrolled_pos(sp / W, sp % W, H, W, L);
  const int64_t src = b * ntok + (inverse ? un : sp);
  const int64_t dst = b * ntok + (inverse ? sp : un);
  const uint8_t* xs = x + src * row_bytes;
  uint8_t* yd = y + dst * row_bytes;
  for (int o = lane * 16; o < row_bytes; o += G * 16) st16_nt(yd + o, ld16(xs + o));
}

hipError_t launch_permute(const void* x, void* y, int batch, int H, int W, int L, int channels,
                          bool inverse, DType dt, hipStream_t s) {
  const int row_bytes = channels * (dt == DType::BF16 ? 2 : 4);
  const int64_t rows = (int64_t)batch * H * W;
  if (rows == 0) return hipSuccess;
  const int nvec = row_bytes / 16;
  auto go = [&](auto gtag) {
    constexpr int G = decltype(gtag)::value;
    const int64_t blocks = (rows + (256 / G) - 1) / (256 / G);
    hipLaunchKernelGGL((permute_kernel<G>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const uint8_t*)x, (uint8_t*)y, batch, H, W, L, row_bytes, (int)inverse);
    return hipGetLastError();
  };
  if (nvec <= 8) return go(std::integral_constant<int, 8>());
  if (nvec <= 16) return go(std::integral_constant<int, 16>());
  if (nvec <= 32) return go(std::integral_constant<int, 32>());
  return go(std::integral_constant<int, 64>());
}

// 4x max-pool over the q_stride axis of the unrolled order: output token m
// of a frame is the elementwise max of tokens m + s * tokens/4, s = 0..3
// (a 2x2 spatial max). max() of values that are all representable in T
// returns one of them, so the result is bit-exact.
template <typename T, int G>
__global__ __launch_bounds__(256) void pool4_kernel(const T* __restrict__ x, int64_t xs, T* __restrict__ y,
                                                    int64_t ys, int batch, int tokens, int channels) {
  constexpr int VN = Vec<T>::N;
  const int lane = threadIdx.x % G;
  const int q = tokens / 4;
  const int64_t t = (int64_t)blockIdx.x * (256 / G) + threadIdx.x / G;
  if (t >= (int64_t)batch * q) return;
  const int64_t b = t / q;
  const int64_t m = t - b * q;
  const T* x0 = x + (b * tokens + m) * xs;
  T* yr = y + t * ys;
  for (int c = lane * VN; c < channels; c += G * VN) {
    float acc[VN], v[VN];
    unpack16<T>(ld16_nt(x0 + c), acc);
#pragma unroll
    for (int s = 1; s < 4; ++s) {
      unpack16<T>(ld16_nt(x0 + (int64_t)s * q * xs + c), v);
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[e] = fmaxf(acc[e], v[e]);
    }
    st16(yr + c, pack16<T>(acc));
  }
}

hipError_t launch_pool4(const void* x, int64_t xs, void* y, int64_t ys, int batch, int tokens,
                        int channels, DType dt, hipStream_t s, StageEvents ev) {
  const int64_t rows = (int64_t)batch * (tokens / 4);
  if (rows == 0) return hipSuccess;
  // G lanes per output row: the smallest group that covers the row in one
  // pass of 16-byte vectors (all four source loads of a lane in flight at once)
  auto launch = [&](auto ttag, auto gtag) {
    using T = decltype(ttag);
    constexpr int G = decltype(gtag)::value;
    const int64_t blocks = (rows + (256 / G) - 1) / (256 / G);
    hipExtLaunchKernelGGL((pool4_kernel<T, G>), dim3((unsigned)blocks), dim3(256), 0, s, ev.start, ev.stop, 0,
                          (const T*)x, xs, (T*)y, ys, batch, tokens, channels);
    return hipGetLastError();
  };
  auto go = [&](auto ttag) {
    using T = decltype(ttag);
    const int nvec = channels / Vec<T>::N;
    if (nvec <= 8) return launch(ttag, std::integral_constant<int, 8>());
    if (nvec <= 16) return launch(ttag, std::integral_constant<int, 16>());
    if (nvec <= 32) return launch(ttag, std::integral_constant<int, 32>());
    return launch(ttag, std::integral_constant<int, 64>());
  };
  return dt == DType::BF16 ? go(bf16()) : go(float());
}

// V^T for the large-window attention when the qkv projection cannot write it
// from its epilogue: vt[b][h][d][t] = qkv[b*T + t][col0 + h*hd + d]. One
// workgroup per (64 tokens, head, frame): the tile goes through LDS so both
// the reads (16-byte runs of d) and the writes (16-byte runs of tokens) are
// full vectors. T % 8 == 0 and hd % 8 == 0, hd <= 64.
__global__ __launch_bounds__(256) void v_transpose_kernel(const bf16* __restrict__ qkv, int64_t ld, int col0,
                                                          bf16* __restrict__ vt, int T, int heads, int hd) {
  constexpr int TT = 64, ROW = 64 + 8;  // tile tokens; LDS row (elements)
  __shared__ __attribute__((aligned(16))) bf16 tile[TT * ROW];
  const int t0 = blockIdx.x * TT, h = blockIdx.y, b = blockIdx.z;
  const int nch = hd / 8;
  for (int e = threadIdx.x; e < TT * nch; e += 256) {
    const int t = e / nch, c = e - t * nch;
    if (t0 + t < T)
      st16(tile + t * ROW + c * 8, ld16(qkv + ((int64_t)b * T + t0 + t) * ld + col0 + h * hd + c * 8));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < hd * (TT / 8); e += 256) {
    const int d = e / (TT / 8), tc = e - d * (TT / 8);
    if (t0 + tc * 8 >= T) continue;
    bf16 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = tile[(tc * 8 + k) * ROW + d];
    st16(vt + (((int64_t)b * heads + h) * hd + d) * T + t0 + tc * 8, *reinterpret_cast<const u32x4*>(v));
  }
}

hipError_t launch_v_transpose(const void* qkv, int64_t ld, int col0, void* vt, int batch, int tokens, int heads,
                              int head_dim, hipStream_t s, StageEvents ev) {
  if (batch == 0 || tokens == 0) return hipSuccess;
  dim3 grid((unsigned)((tokens + 63) / 64), (unsigned)heads, (unsigned)batch);
  hipExtLaunchKernelGGL(v_transpose_kernel, grid, dim3(256), 0, s, ev.start, ev.stop, 0, (const bf16*)qkv, ld, col0,
                        (bf16*)vt, tokens, heads, head_dim);
  return hipGetLastError();
}


// int8 -> activation type, exact (|q| <= 128 fits in bf16's 8 significant
// bits). Work unit: the int8 values of one 16-byte output chunk (8 for bf16,
// 4 for float), so that a wave's loads and stores are both contiguous; the
// segments are laid end to end, and each thread takes I8U units spaced a
// grid apart, all loads issued before the stores.
constexpr int I8U = 4;

struct I8Params {
  const int8_t* src[6];
  void* dst[6];
  int64_t start[7];  // unit offsets of the segments
  int count;
};

template <typename T>
__global__ __launch_bounds__(256) void i8_convert_kernel(I8Params q) {
  constexpr int VN = Vec<T>::N;
  const int64_t total = q.start[q.count], stride = (int64_t)gridDim.x * 256;
  uint32_t raw[I8U][VN / 4];
  T* out[I8U];
#pragma unroll
  for (int u = 0; u < I8U; ++u) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x + u * stride;
    out[u] = nullptr;
    if (c >= total) continue;
    // segment of unit c (constant indices only: no indexed copy of the
    // parameter arrays)
    const int8_t* src = q.src[0];
    void* dst = q.dst[0];
    int64_t first = 0;
#pragma unroll
    for (int i = 1; i < 6; ++i)
      if (i < q.count && c >= q.start[i]) {
        src = q.src[i];
        dst = q.dst[i];
        first = q.start[i];
      }
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(src + (c - first) * VN);
    if constexpr (VN == 8) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(sp);
      raw[u][0] = v[0];
      raw[u][VN / 4 - 1] = v[1];
    } else {
      raw[u][0] = sp[0];
    }
    out[u] = static_cast<T*>(dst) + (c - first) * VN;
  }
#pragma unroll
  for (int u = 0; u < I8U; ++u) {
    if (out[u] == nullptr) continue;
    float f[VN];
#pragma unroll
    for (int e = 0; e < VN; ++e) f[e] = (float)(int8_t)(raw[u][e / 4] >> (8 * (e % 4)));
    st16(out[u], pack16<T>(f));
  }
}

hipError_t launch_i8_convert(const I8Segments& sg, DType dt, hipStream_t s, StageEvents ev) {
  I8Params q{};
  q.count = sg.count;
  q.start[0] = 0;
  const int vn = dt == DType::BF16 ? 8 : 4;
  for (int i = 0; i < sg.count; ++i) {
    if (sg.n[i] % 16) return hipErrorInvalidValue;
    q.src[i] = sg.src[i];
    q.dst[i] = sg.dst[i];
    q.start[i + 1] = q.start[i] + sg.n[i] / vn;
  }
  for (int i = sg.count; i < 6; ++i) q.start[i + 1] = q.start[sg.count];
  const int64_t units = q.start[sg.count];
  if (units == 0) return hipSuccess;
  dim3 grid((unsigned)((units + 256 * I8U - 1) / (256 * I8U))), block(256);
  if (dt == DType::BF16)
    hipExtLaunchKernelGGL(i8_convert_kernel<bf16>, grid, block, 0, s, ev.start, ev.stop, 0, q);
  else
    hipExtLaunchKernelGGL(i8_convert_kernel<float>, grid, block, 0, s, ev.start, ev.stop, 0, q);
  return hipGetLastError();
}

}  // namespace vit
