// Non-causal multi-head attention over windows, flash style, on MFMA.
//
// One workgroup (4 waves) takes one (frame, window, query tile) and HPW
// heads; each wave owns 16*QB query rows of one head. Per 64-key tile the
// workgroup stages K (row-major, [key][d]) and V transposed ([d][key]) of
// its heads in LDS; each wave then computes S^T = K Q^T with MFMA (keys on
// the MFMA rows, so every lane holds 4 keys of ONE query row), updates the
// running row max and sum (online softmax, base-2 exponentials with the
// scale folded into log2 e), and accumulates O^T = V^T P^T with MFMA. The
// query's row statistics and its output column are per-lane values, so the
// softmax correction is a per-lane scalar and the only cross-lane traffic
// is two xor-shuffles per row max (lanes l, l^16, l^32, l^48).
//
// Windows are address maps, not copies: the kernel computes each query and
// key token's row in the [tokens, 3*dim] qkv buffer from the window index:
//   GLOBAL     token = i                                (one window/frame)
//   MASK_UNIT  token = w + i * n_windows                (Hiera mask units)
//   SPATIAL    token = (wy*win_h + i/win_w)*grid_w + wx*win_w + i%win_w
// With q_stride 4 the query of pooled token m is the elementwise max of the
// q rows m + s*N/4 (s = 0..3), taken while loading Q.
// head_dim up to 64 (multiple of 8); columns past head_dim are zero-padded
// in registers and LDS, which leaves every dot product unchanged.
#include "common.h"
#include "launch.h"

#include <hip/hip_ext.h>

#include <type_traits>

namespace vit {

constexpr int KT = 64;   // keys per tile
constexpr int HDP = 64;  // padded head dim

template <typename T>
struct AttnParams {
  const T* qkv;
  int64_t ld_qkv;
  T* ctx;
  int64_t ld_ctx;
  int tokens_in, tokens_out, dim, heads, head_dim;
  int mode, n_windows, grid_w, win_h, win_w;
  int n_q, n_kv, q_tiles, head_groups, windows;
  float scale_log2;
};

__device__ __forceinline__ int window_token(int mode, int w, int i, int n_windows, int grid_w, int win_h,
                                            int win_w) {
  if (mode == ATTN_MASK_UNIT) return w + i * n_windows;
  if (mode == ATTN_SPATIAL) {
    const int nwx = grid_w / win_w;
    const int wy = w / nwx, wx = w - wy * nwx;
    const int iy = i / win_w, ix = i - iy * win_w;
    return (wy * win_h + iy) * grid_w + wx * win_w + ix;
  }
  return i;
}

template <typename T, int QB, int HPW, bool POOL>
__global__ __launch_bounds__(256) void attention_kernel(AttnParams<T> p) {
  constexpr int VN = Vec<T>::N;
  constexpr int CH = HDP / VN;  // 16-byte chunks per padded head row
  constexpr int WPH = 4 / HPW;  // waves per head
  constexpr int QSTEPS = HDP / Mma<T>::KSTEP;
  constexpr int PAD = VN;
  constexpr int KROW = HDP + PAD;
  constexpr int VROW = KT + PAD;
  constexpr int LOADS = KT * HPW * CH / 256;  // 16-byte K (and V) loads per thread per tile

  __shared__ __attribute__((aligned(16))) T Ks[HPW][KT][KROW];
  __shared__ __attribute__((aligned(16))) T Vt[HPW][HDP][VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;

  int bid = blockIdx.x;
  const int hg = bid % p.head_groups;
  bid /= p.head_groups;
  const int qt = bid % p.q_tiles;
  bid /= p.q_tiles;
  const int win = bid % p.windows;
  const int b = bid / p.windows;

  const int hl = wave / WPH;
  const int head = hg * HPW + hl;
  const int hd = p.head_dim;
  const int D = p.dim;
  const int64_t frame_in = (int64_t)b * p.tokens_in;

  // ---- Q fragments (B operand of S^T = K Q^T), scaled later in fp32
  u32x4 qf[QB][QSTEPS];
  int qrow_out[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int i = (qt * WPH + wave % WPH) * 16 * QB + qb * 16 + fr;
    const bool valid = i < p.n_q;
    const int tq = valid ? window_token(p.mode, win, i, p.n_windows, p.grid_w, p.win_h, p.win_w) : 0;
    qrow_out[qb] = valid ? tq : -1;
#pragma unroll
    for (int ks = 0; ks < QSTEPS; ++ks) {
      const int off = (ks * 4 + g) * VN;
      if (!valid || off >= hd) {
        qf[qb][ks] = u32x4{0, 0, 0, 0};
        continue;
      }
      if (!POOL) {
        qf[qb][ks] = ld16(p.qkv + (frame_in + tq) * p.ld_qkv + head * hd + off);
      } else {
        const int quarter = p.tokens_in / 4;
        float mx[VN], v[VN];
        unpack16<T>(ld16(p.qkv + (frame_in + tq) * p.ld_qkv + head * hd + off), mx);
#pragma unroll
        for (int s = 1; s < 4; ++s) {
          unpack16<T>(ld16(p.qkv + (frame_in + tq + (int64_t)s * quarter) * p.ld_qkv + head * hd + off), v);
#pragma unroll
          for (int e = 0; e < VN; ++e) mx[e] = fmaxf(mx[e], v[e]);
        }
        qf[qb][ks] = pack16<T>(mx);
      }
    }
  }

  // ---- K / V tile staging: thread -> (key row, head, chunk), chunk fastest
  u32x4 kreg[LOADS], vreg[LOADS];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int v = tid + 256 * it;
      const int c = v % CH, rest = v / CH;
      const int h = rest % HPW, j = rest / HPW;
      const int kv = kt * KT + j;
      if (kv < p.n_kv && c * VN < hd) {
        const int tk = window_token(p.mode, win, kv, p.n_windows, p.grid_w, p.win_h, p.win_w);
        const T* rowp = p.qkv + (frame_in + tk) * p.ld_qkv + (hg * HPW + h) * hd + c * VN;
        kreg[it] = ld16(rowp + D);
        vreg[it] = ld16(rowp + 2 * D);
      } else {
        kreg[it] = u32x4{0, 0, 0, 0};
        vreg[it] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int v = tid + 256 * it;
      const int c = v % CH, rest = v / CH;
      const int h = rest % HPW, j = rest / HPW;
      st16(&Ks[h][j][c * VN], kreg[it]);
      T e[VN];
      *reinterpret_cast<u32x4*>(e) = vreg[it];
#pragma unroll
      for (int k = 0; k < VN; ++k) Vt[h][c * VN + k][j] = e[k];
    }
  };

  f32x4 acc_o[HDP / 16][QB];
#pragma unroll
  for (int db = 0; db < HDP / 16; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc_o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[QB], l_part[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -1e30f;
    l_part[qb] = 0.f;
  }

  const int ntiles = (p.n_kv + KT - 1) / KT;
  fetch(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    stash();
    __syncthreads();
    if (kt + 1 < ntiles) fetch(kt + 1);

    // S^T = K Q^T for this wave's head: s[kb][qb][r] = S[q][key = kb*16 + 4g + r]
    f32x4 s[KT / 16][QB];
#pragma unroll
    for (int kb = 0; kb < KT / 16; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < QSTEPS; ++ks) {
        const u32x4 kf = ld16(&Ks[hl][kb * 16 + fr][(ks * 4 + g) * VN]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = Mma<T>::step(kf, qf[qb][ks], s[kb][qb]);
      }
    }
    const int kv_left = p.n_kv - kt * KT;  // keys valid in this tile (may exceed KT)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -1e30f;
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = s[kb][qb][r] * p.scale_log2;
          if (kb * 16 + 4 * g + r >= kv_left) v = -1e30f;
          s[kb][qb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m_run[qb], mx);
      const float alpha = exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = exp2f(s[kb][qb][r] - m_new);
          s[kb][qb][r] = e;
          ls += e;
        }
      l_part[qb] = l_part[qb] * alpha + ls;
#pragma unroll
      for (int db = 0; db < HDP / 16; ++db) acc_o[db][qb] = acc_o[db][qb] * alpha;
    }

    // O^T += V^T P^T
    if constexpr (std::is_same<T, bf16>::value) {
#pragma unroll
      for (int c2 = 0; c2 < KT / 32; ++c2) {
        u32x4 pf[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          bf16x8 pv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pv[r] = (bf16)s[2 * c2][qb][r];
            pv[4 + r] = (bf16)s[2 * c2 + 1][qb][r];
          }
          pf[qb] = __builtin_bit_cast(u32x4, pv);
        }
#pragma unroll
        for (int db = 0; db < HDP / 16; ++db) {
          const T* vrow = &Vt[hl][db * 16 + fr][0];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 32 * c2 + 4 * g);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 32 * c2 + 16 + 4 * g);
          const u32x4 vf = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc_o[db][qb] = Mma<T>::step(vf, pf[qb], acc_o[db][qb]);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb) {
#pragma unroll
        for (int db = 0; db < HDP / 16; ++db) {
          const u32x4 vf = ld16(&Vt[hl][db * 16 + fr][kb * 16 + 4 * g]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc_o[db][qb] = Mma<T>::step(vf, __builtin_bit_cast(u32x4, s[kb][qb]), acc_o[db][qb]);
        }
      }
    }
  }

  // ---- normalise and store: lane holds ctx[q][16*db + 4g .. +3]
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l = l_part[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (qrow_out[qb] < 0) continue;
    const float inv = 1.0f / l;
    T* out = p.ctx + ((int64_t)b * p.tokens_out + qrow_out[qb]) * p.ld_ctx + head * hd;
#pragma unroll
    for (int db = 0; db < HDP / 16; ++db) {
      const int d = db * 16 + 4 * g;
      if (d < hd) store4<T>(out + d, acc_o[db][qb] * inv);
    }
  }
}

template <typename T, int QB, int HPW, bool POOL>
static hipError_t attn_go(const AttnArgs& a, AttnParams<T> p, hipStream_t s, StageEvents ev) {
  constexpr int rows = (4 / HPW) * 16 * QB;
  p.q_tiles = (p.n_q + rows - 1) / rows;
  p.head_groups = a.heads / HPW;
  const int64_t blocks = (int64_t)a.batch * p.windows * p.q_tiles * p.head_groups;
  if (blocks == 0) return hipSuccess;
  hipExtLaunchKernelGGL((attention_kernel<T, QB, HPW, POOL>), dim3((unsigned)blocks), dim3(256), 0, s, ev.start,
                        ev.stop, 0, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t attn_dispatch(const AttnArgs& a, hipStream_t s, StageEvents ev) {
  AttnParams<T> p;
  p.qkv = (const T*)a.qkv;
  p.ld_qkv = a.ld_qkv;
  p.ctx = (T*)a.ctx;
  p.ld_ctx = a.ld_ctx;
  p.tokens_in = a.tokens_in;
  p.tokens_out = a.tokens_out;
  p.dim = a.dim;
  p.heads = a.heads;
  p.head_dim = a.head_dim;
  p.mode = a.mode;
  p.n_windows = a.n_windows;
  p.grid_w = a.grid_w;
  p.win_h = a.win_h;
  p.win_w = a.win_w;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  if (a.mode == ATTN_MASK_UNIT) {
    p.windows = a.n_windows;
    p.n_q = a.tokens_out / a.n_windows;
    p.n_kv = a.tokens_in / a.n_windows;
  } else if (a.mode == ATTN_SPATIAL) {
    p.windows = (a.tokens_in / a.grid_w / a.win_h) * (a.grid_w / a.win_w);
    p.n_q = p.n_kv = a.win_h * a.win_w;
  } else {
    p.windows = 1;
    p.n_q = a.tokens_out;
    p.n_kv = a.tokens_in;
  }
  const bool pool = a.q_stride == 4;
  // small query sets: several heads per workgroup, one wave each
  if (p.n_q <= 16 && a.heads % 4 == 0) {
    return pool ? attn_go<T, 1, 4, true>(a, p, s, ev) : attn_go<T, 1, 4, false>(a, p, s, ev);
  }
  if (p.n_q <= 32 && a.heads % 2 == 0) {
    return pool ? attn_go<T, 1, 2, true>(a, p, s, ev) : attn_go<T, 1, 2, false>(a, p, s, ev);
  }
  if (p.n_q <= 64) return pool ? attn_go<T, 1, 1, true>(a, p, s, ev) : attn_go<T, 1, 1, false>(a, p, s, ev);
  return pool ? attn_go<T, 2, 1, true>(a, p, s, ev) : attn_go<T, 2, 1, false>(a, p, s, ev);
}

hipError_t launch_attention(const AttnArgs& a, DType dt, hipStream_t s, StageEvents ev) {
  return dt == DType::BF16 ? attn_dispatch<bf16>(a, s, ev) : attn_dispatch<float>(a, s, ev);
}

}  // namespace vit
