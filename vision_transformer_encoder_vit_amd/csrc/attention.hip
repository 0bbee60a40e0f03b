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

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <type_traits>

namespace vit {

constexpr int KT = 64;   // keys per tile
#ifndef ATTN_NW
#define ATTN_NW 4
#endif
#ifndef ATTN_QB
#define ATTN_QB 1
#endif
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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
  const T* vt;  // V transposed [B, heads, head_dim, tokens_in] (large-window kernel)
  // key-split partials (splits > 1): unnormalised O [split][B*tokens_out][dim]
  // and (row max, row sum) [split][B*tokens_out][heads][2], fp32
  int splits;
  int64_t batch_rows;  // B * tokens_out
  float* part_o;
  float* part_ml;
  float l_lo, l_hi;  // large-window kernel: the band a row sum must fall in (2^-64, 2^64)
  float m_band;      // large-window kernel with the keys split among the waves: first tile's row maxima band
};

// Work-item and workgroup ids and votes from compiler builtins: this file is
// compiled without IEEE mode, so the device-library versions behind
// threadIdx, blockIdx, __any and __syncthreads_or (compiled with it) are not
// inlined; each was a real call, with the registers it may clobber spilled
// around it.
__device__ __forceinline__ int wi_id() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int wg_id() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }
// true in every thread when p holds in some thread of the workgroup of NW
// waves: one vote per wave through LDS and a barrier (the votes may be
// written again only after a later barrier)
template <int NW>
__device__ __forceinline__ bool wg_any(bool p) {
  __shared__ int votes[NW];
  const bool w = wave_any(p);
  if ((wi_id() & 63) == 0) votes[wi_id() >> 6] = w;
  __syncthreads();
  bool any = false;
#pragma unroll
  for (int i = 0; i < NW; ++i) any |= votes[i] != 0;
  return any;
}

// The row-sum band of the softmax passes without a running maximum.
// VIT_ATTN_RANGE_LOG2 (test hook, default 64) narrows it; 0 sends every
// window through the pass with the running maximum.
static void attn_band(float& lo, float& hi) {
  int range = 64;
  if (const char* env = std::getenv("VIT_ATTN_RANGE_LOG2")) range = std::max(0, std::min(64, std::atoi(env)));
  lo = std::ldexp(1.0f, -range);
  hi = range == 0 ? 0.f : std::ldexp(1.0f, range);
}

// The band of the first key tile's row maxima (c*s units) inside which the
// large-window kernels keep the pass without a running maximum: 16, or
// VIT_ATTN_TILE0_BAND (test hook; a negative value sends every wave to the
// running-maximum pass).
static float attn_tile0_band() {
  const char* env = std::getenv("VIT_ATTN_TILE0_BAND");
  return env ? (float)std::atof(env) : 16.f;
}

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

  const int tid = wi_id(), lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;

  int bid = wg_id();
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

  // ---- K / V tile staging. K: thread -> (key row, head, chunk), chunk
  // fastest (a row's chunks are contiguous in memory). V: key fastest, so
  // that each of the transposing 2-byte LDS writes of a wave covers 64
  // consecutive keys of one V^T row (chunk fastest put 8 chunks x 4 heads
  // of a write on two banks: 16-way conflicts)
  static_assert(256 % KT == 0, "a wave's V loads share one (head, chunk)");
  u32x4 kreg[LOADS], vreg[LOADS];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int v = tid + 256 * it;
      {
        const int c = v % CH, rest = v / CH;
        const int h = rest % HPW, j = rest / HPW;
        const int kv = kt * KT + j;
        if (kv < p.n_kv && c * VN < hd) {
          const int tk = window_token(p.mode, win, kv, p.n_windows, p.grid_w, p.win_h, p.win_w);
          kreg[it] = ld16(p.qkv + (frame_in + tk) * p.ld_qkv + D + (hg * HPW + h) * hd + c * VN);
        } else {
          kreg[it] = u32x4{0, 0, 0, 0};
        }
      }
      {
        const int j = v % KT, rest = v / KT;
        const int c = rest % CH, h = rest / CH;
        const int kv = kt * KT + j;
        if (kv < p.n_kv && c * VN < hd) {
          const int tk = window_token(p.mode, win, kv, p.n_windows, p.grid_w, p.win_h, p.win_w);
          vreg[it] = ld16(p.qkv + (frame_in + tk) * p.ld_qkv + 2 * D + (hg * HPW + h) * hd + c * VN);
        } else {
          vreg[it] = u32x4{0, 0, 0, 0};
        }
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int v = tid + 256 * it;
      {
        const int c = v % CH, rest = v / CH;
        const int h = rest % HPW, j = rest / HPW;
        st16(&Ks[h][j][c * VN], kreg[it]);
      }
      {
        const int j = v % KT, rest = v / KT;
        const int c = rest % CH, h = rest / CH;
        T e[VN];
        *reinterpret_cast<u32x4*>(e) = vreg[it];
#pragma unroll
        for (int k = 0; k < VN; ++k) Vt[h][c * VN + k][j] = e[k];
      }
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

// ---------------------------------------------------------------------------
// bf16 kernel for large windows (>= 128 queries): 32x32x16 MFMA.
//
// A workgroup of NW waves takes 32*QB*NW queries of one (frame, window,
// head); each wave owns QB blocks of 32 queries, and every K and V fragment
// read from LDS feeds QB MFMAs. Per 64-key tile, K rows ([key][d]) and V^T
// rows ([d][key], written transposed by the qkv projection) go global ->
// LDS directly (global_load_lds, XOR-swizzled 16-byte chunks), double
// buffered: the next tile is in flight while this one is multiplied.
//   S^T = K Q^T    lane (q = l%32, h = l/32) receives S^T rows
//                  R = 32kb + 8(r/4) + 4h + r%4 (r = register)
//   key order      LDS row R of the K tile holds key pi(R), pi swapping bits
//                  2 and 3 of R; then registers 8s..8s+7 of lane half h are
//                  keys 32kb + 16s + 8h + 0..7, i.e. 8 consecutive keys
//   softmax        row max = in-lane max + one swap of the wave halves
//                  (permlane32); exponentials exp2(s*c - m*c) with
//                  c = scale*log2(e); the output is rescaled every tile
//                  (a branch around it costs more in register copies)
//   O^T += V^T P^T P goes to the MFMA as the B operand straight from the
//                  softmax registers; its k-slots 8h..8h+7 are the 8
//                  consecutive keys above, so the V^T operand is one
//                  16-byte LDS chunk of row d
// ---------------------------------------------------------------------------

// max of x over lanes l and l ^ 32 (the two halves of the wave)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__host__ __device__ constexpr int attn_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
__device__ __forceinline__ int kswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// key held by LDS row R of a K tile: R with bits 2 and 3 swapped (an involution)
__device__ __forceinline__ int key_of_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
typedef __attribute__((address_space(3))) void* attn_lds_ptr;

// Token index of in-window position i, kept as (x, y) in the window and
// advanced by a fixed step without divisions: GLOBAL windows are the frame
// (token = i), SPATIAL windows are win_h x win_w blocks of the grid.
struct WinCursor {
  int x, y;
  __device__ __forceinline__ void init(int i, int ww) {
    y = i / ww;
    x = i - y * ww;
  }
  __device__ __forceinline__ void step(int dx, int dy, int ww) {
    x += dx;
    y += dy;
    if (x >= ww) {
      x -= ww;
      y += 1;
    }
  }
};

// KSW: the workgroup's waves share one block of QW queries and split the
// window's key tiles among them, each with its own K / V^T buffers; at the
// end the waves' (max, sum, O) merge through LDS (weights 2^((m_w - m) c)).
// For grids too small to fill the chip without splitting the keys, and no
// partials leave the workgroup.
template <int NW, int QB, int MODE, bool POOL, bool KSW = false>
__global__ __launch_bounds__(64 * NW) void attention_mfma32_kernel(AttnParams<bf16> p) {
  constexpr int QW = 32 * QB;  // queries per wave
  static_assert(MODE == ATTN_GLOBAL || MODE == ATTN_SPATIAL, "large-window kernel");
  constexpr int NB = KSW ? NW : 1;  // K / V^T double buffers: one per wave (KSW) or shared
  __shared__ __attribute__((aligned(1024))) bf16 Ks[NB][2][KT * 64];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[NB][2][64 * KT];

  const int tid = wi_id(), lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, h = lane >> 5;
  const int wb = KSW ? wave : 0;
  int bid = wg_id();
  const int split = KSW ? 0 : bid % p.splits;  // key split: tiles [t0, t1) of the window
  bid /= KSW ? 1 : p.splits;
  const int head = bid % p.heads;
  bid /= p.heads;
  const int qt = bid % p.q_tiles;
  bid /= p.q_tiles;
  const int win = bid % p.windows;
  const int b = bid / p.windows;
  const int hd = p.head_dim, D = p.dim;
  const int ld = (int)p.ld_qkv;
  const int ntiles = (p.n_kv + KT - 1) / KT;
  const int nsplit = KSW ? NW : p.splits, part = KSW ? wave : split;
  const int per = (ntiles + nsplit - 1) / nsplit;
  const int t0 = part * per, t1 = min(ntiles, t0 + per);
  // element offset of this frame + window origin in qkv (fits 32 bits: the
  // host checks the buffer size); token (x, y) of the window is at
  // base + (y * grid_w + x) * ld
  int origin = 0, ww = p.n_kv, gw = 0;
  if (MODE == ATTN_SPATIAL) {
    const int nwx = p.grid_w / p.win_w;
    const int wy = win / nwx, wx = win - wy * nwx;
    origin = (wy * p.win_h) * p.grid_w + wx * p.win_w;
    ww = p.win_w;
    gw = p.grid_w;
  }
  const bf16* base = p.qkv + (int64_t)b * p.tokens_in * ld;
  // V^T rows of this (frame, head): row d holds V[token][d] over the frame's tokens
  const bf16* vt_base = p.vt + ((int64_t)b * p.heads + head) * hd * p.tokens_in;
  auto tok = [&](const WinCursor& cur) { return MODE == ATTN_SPATIAL ? origin + cur.y * gw + cur.x : cur.x; };
  // per-tile cursor step: KT positions = dy rows + dx columns of the window
  const int step_dy = MODE == ATTN_SPATIAL ? KT / ww : 0;
  const int step_dx = MODE == ATTN_SPATIAL ? KT - step_dy * ww : KT;
  const int wwx = MODE == ATTN_SPATIAL ? ww : 0x7fffffff;

  // ---- Q fragments: B operand of S^T; lane holds Q[q][16ks + 8h .. +7]
  u32x4 qf[QB][4];
  int qrow_out[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int i = KSW ? qt * QW + qb * 32 + fr : qt * NW * QW + wave * QW + qb * 32 + fr;
    const bool valid = i < p.n_q;
    WinCursor cur;
    cur.init(valid ? i : 0, wwx);
    const int tq = tok(cur);
    qrow_out[qb] = valid ? tq : -1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int off = ks * 16 + h * 8;
      if (!valid || off >= hd) {
        qf[qb][ks] = u32x4{0, 0, 0, 0};
      } else if (!POOL) {
        qf[qb][ks] = ld16(base + tq * ld + head * hd + off);
      } else {
        const int quarter = p.tokens_in / 4;
        float mx[8], v[8];
        unpack16<bf16>(ld16(base + tq * ld + head * hd + off), mx);
#pragma unroll
        for (int s = 1; s < 4; ++s) {
          unpack16<bf16>(ld16(base + (tq + s * quarter) * ld + head * hd + off), v);
#pragma unroll
          for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], v[e]);
        }
        qf[qb][ks] = pack16<bf16>(mx);
      }
    }
  }

  // ---- K tile: wave instruction j fills LDS rows 8j .. 8j+7 (16 bytes per
  // lane); LDS row R holds key pi(R) of the tile.
  constexpr int LOADS = KSW ? KT / 8 : KT / 8 / NW;
  static_assert(KT % (8 * NW) == 0, "tile rows must split over the waves");
  const int grp0 = KSW ? 0 : wave * LOADS;  // this wave's first 8-row group of a tile
  const int last_kv = p.n_kv - 1;
  WinCursor last_cur;
  last_cur.init(last_kv, wwx);
  WinCursor kcur[LOADS];
  int kchunk[LOADS], kkey[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int row = (grp0 + j) * 8 + lane / 8;
    kkey[j] = key_of_row(row);
    // chunks past head_dim read neighbouring finite values (Q is zero there)
    kchunk[j] = min(((lane & 7) ^ kswz(row)) * 8, 2 * D - head * hd - 8) + D + head * hd;
  }
  // ---- V^T tile: LDS row d = V^T row min(d, hd - 1) (rows past head_dim
  // only feed output rows that are never stored); 16-byte chunk c of a row
  // is keys 8c .. 8c+7 of the tile, which are consecutive tokens (the window
  // width is a multiple of 8). Chunks past the window repeat its last chunk
  // (finite values under P = 0).
  WinCursor vcur[LOADS];
  int vrow_off[LOADS], vpos[LOADS];
  WinCursor vlast;
  vlast.init(p.n_kv - 8, wwx);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int row = (grp0 + j) * 8 + lane / 8;
    vpos[j] = ((lane & 7) ^ kswz(row)) * 8;
    vrow_off[j] = min(row, hd - 1) * p.tokens_in;
  }
  // the cursors at tile t0 (again for the fallback pass)
  auto cursors_at_start = [&]() {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      kcur[j].init(t0 * KT + kkey[j], wwx);
      vcur[j].init(t0 * KT + vpos[j], wwx);
    }
  };
  auto issue = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      // keys past the window read the last key (masked out of the softmax)
      const int t = kt * KT + kkey[j] <= last_kv ? tok(kcur[j]) : tok(last_cur);
      __builtin_amdgcn_global_load_lds((const void*)(base + t * ld + kchunk[j]),
                                       (attn_lds_ptr)(&Ks[wb][kt & 1][(grp0 + j) * 512]), 16, 0, 0);
      kcur[j].step(step_dx, step_dy, wwx);
    }
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int t = kt * KT + vpos[j] <= p.n_kv - 8 ? tok(vcur[j]) : tok(vlast);
      __builtin_amdgcn_global_load_lds((const void*)(vt_base + vrow_off[j] + t),
                                       (attn_lds_ptr)(&Vs[wb][kt & 1][(grp0 + j) * 512]), 16, 0, 0);
      vcur[j].step(step_dx, step_dy, wwx);
    }
  };

  f32x16 acc_o[QB][2];  // [qb][db]: O^T[d = 32db + 8(r/4) + 4h + r%4][q]
  float m_run[QB], l_part[QB];
  const float c = p.scale_log2;
  const bf16x2_t ones = {(bf16)1.f, (bf16)1.f};

  // One pass over tiles t0 .. t1-1. MF (first pass): softmax without a
  // running maximum, P = 2^(c s) straight from the scores, the row sums
  // from the bf16 P (m = 0 for the partials and the merge); a row whose sum
  // leaves the band [2^-64, 2^64] (scores too large or too small for that)
  // sends its wave, or with shared tiles its workgroup, through the pass
  // again with the online maximum (m_run subtracted, O and l rescaled as it
  // grows).
  bool stopped = false;  // KSW: this wave left the first pass at its first tile
  auto tile_pass = [&](auto mf_tag) {
    constexpr bool MF = decltype(mf_tag)::value;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int db = 0; db < 2; ++db) acc_o[qb][db] = f32x16{};
      m_run[qb] = MF ? 0.f : -1e30f;
      l_part[qb] = 0.f;
    }
    cursors_at_start();
    if (t0 < t1) issue(t0);
    for (int kt = t0; kt < t1; ++kt) {
      const int buf = kt & 1;
      // this wave's loads of tile kt have landed; after the barrier every
      // wave's have, and every wave is done with the buffer refilled next
      // (KSW: the buffers are the wave's own, and the waves' tile counts
      // differ, so no barrier)
      __builtin_amdgcn_s_waitcnt(attn_vmcnt(0));
      if (!KSW) __syncthreads();
      if (kt + 1 < t1) issue(kt + 1);
      f32x16 sacc[QB][2];  // [qb][kb]
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sacc[qb][kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = kb * 32 + fr;
          const u32x4 kfr = ld16(&Ks[wb][buf][row * 64 + ((ks * 2 + h) ^ kswz(row)) * 8]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kfr),
                                                                  __builtin_bit_cast(bf16x8, qf[qb][ks]), sacc[qb][kb], 0, 0, 0);
        }
      }
      const int kv_left = p.n_kv - kt * KT;
      if (kv_left < KT) {  // uniform: only the last tile of a ragged window
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (key_of_row(kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) >= kv_left) sacc[qb][kb][r] = -1e30f;
      }
      if constexpr (MF && KSW) {
        // the wave's own keys and no barriers: a wave some of whose rows
        // have their maximum c s over its first tile outside [-m_band,
        // m_band] (trained weights) stops here and takes the online pass
        if (kt == t0) {
          bool wide = false;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            float mx = -1e30f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
            const float mc = halves_max(mx) * c;
            wide |= qrow_out[qb] >= 0 && !(mc >= -p.m_band && mc <= p.m_band);
          }
          if (wave_any(wide)) {
            stopped = true;
            break;
          }
        }
      }
      u32x4 pf[QB][2][2];  // [qb][kb][s]: bf16 P for MFMA k-step s of key block kb
      if constexpr (MF) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              bf16x8 pv;
#pragma unroll
              for (int e = 0; e < 8; ++e) pv[e] = (bf16)__builtin_amdgcn_exp2f(sacc[qb][kb][8 * s + e] * c);
              pf[qb][kb][s] = __builtin_bit_cast(u32x4, pv);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bf16x2_t pr = {pv[2 * e], pv[2 * e + 1]};
                l_part[qb] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_part[qb], false);
              }
            }
      } else {
        float alpha[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float mx = fmaxf(sacc[qb][0][0], sacc[qb][0][1]);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = (kb == 0 ? 2 : 0); r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[qb][kb][r], sacc[qb][kb][r + 1]));
          const float m_new = fmaxf(m_run[qb], halves_max(mx));
          alpha[qb] = __builtin_amdgcn_exp2f((m_run[qb] - m_new) * c);
          m_run[qb] = m_new;
          const float mc = m_new * c;
          float ls = 0.f;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              bf16x8 pv;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][8 * s + e], c, -mc));
                ls += pe;
                pv[e] = (bf16)pe;
              }
              pf[qb][kb][s] = __builtin_bit_cast(u32x4, pv);
            }
          }
          l_part[qb] = l_part[qb] * alpha[qb] + ls;
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int db = 0; db < 2; ++db) acc_o[qb][db] = acc_o[qb][db] * alpha[qb];
      }
      // O^T += V^T P^T: k-step s of key block kb covers keys 32kb + 16s + 8h + 0..7
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const int row = db * 32 + fr;
            const u32x4 vf = ld16(&Vs[wb][buf][row * 64 + ((4 * kb + 2 * s + h) ^ kswz(row)) * 8]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              acc_o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf),
                                                                     __builtin_bit_cast(bf16x8, pf[qb][kb][s]), acc_o[qb][db], 0, 0, 0);
          }
    }
  };
  tile_pass(std::integral_constant<bool, true>{});
  {
    bool out = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = l_part[qb] + __shfl_xor(l_part[qb], 32, 64);
      out |= qrow_out[qb] >= 0 && !(l >= p.l_lo && l <= p.l_hi);
    }
    // KSW: the wave's own keys, so its own decision; shared tiles: the
    // workgroup's (uniform, and a barrier before the tiles are refilled)
    const bool again = KSW ? stopped || wave_any(out) : wg_any<NW>(out);
    if (again) tile_pass(std::integral_constant<bool, false>{});
  }

  if constexpr (KSW) {
    // ---- merge the waves: (m, l) per query -> LDS; each wave's O^T times
    // 2^((m_w - m) c) / l -> LDS as [wave][query][d]; thread (query, 8 d)
    // sums the waves' values and stores 16 bytes of ctx
    float* mls = reinterpret_cast<float*>(&Vs[0][0][0]);  // [NW][QW][2]
    float* ops = reinterpret_cast<float*>(&Ks[0][0][0]);  // [NW][QW][64]
    static_assert(NW * QW * 64 * 4 <= (int)sizeof(Ks) && NW * QW * 2 * 4 <= (int)sizeof(Vs), "merge space");
    __syncthreads();  // every wave is done with its K / V^T buffers
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = l_part[qb] + __shfl_xor(l_part[qb], 32, 64);
      if (h == 0) {
        mls[(wave * QW + qb * 32 + fr) * 2] = m_run[qb];
        mls[(wave * QW + qb * 32 + fr) * 2 + 1] = l;
      }
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int q = qb * 32 + fr;
      float m = mls[q * 2];
#pragma unroll
      for (int w = 1; w < NW; ++w) m = fmaxf(m, mls[(w * QW + q) * 2]);
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) l += __builtin_amdgcn_exp2f((mls[(w * QW + q) * 2] - m) * c) * mls[(w * QW + q) * 2 + 1];
      const float sc = __builtin_amdgcn_exp2f((m_run[qb] - m) * c) / l;
      float* op = ops + (wave * QW + q) * 64;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          *reinterpret_cast<f32x4*>(op + db * 32 + 8 * gq + 4 * h) =
              f32x4{acc_o[qb][db][4 * gq], acc_o[qb][db][4 * gq + 1], acc_o[qb][db][4 * gq + 2],
                    acc_o[qb][db][4 * gq + 3]} * sc;
    }
    __syncthreads();
    for (int e = tid; e < QW * 8; e += 64 * NW) {
      const int q = e / 8, d0 = (e % 8) * 8;
      const int i = qt * QW + q;
      if (i >= p.n_q || d0 >= hd) continue;
      f32x4 o0 = *reinterpret_cast<const f32x4*>(ops + q * 64 + d0);
      f32x4 o1 = *reinterpret_cast<const f32x4*>(ops + q * 64 + d0 + 4);
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        o0 += *reinterpret_cast<const f32x4*>(ops + (w * QW + q) * 64 + d0);
        o1 += *reinterpret_cast<const f32x4*>(ops + (w * QW + q) * 64 + d0 + 4);
      }
      WinCursor cur;
      cur.init(i, wwx);
      bf16* out = p.ctx + ((int64_t)b * p.tokens_out + tok(cur)) * p.ld_ctx + head * hd + d0;
      store4<bf16>(out, o0);
      if (d0 + 4 < hd) store4<bf16>(out + 4, o1);
    }
    return;
  }

  // ---- normalise and store: lane holds ctx[q][32db + 8g + 4h .. +3], g = r/4
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l = l_part[qb] + __shfl_xor(l_part[qb], 32, 64);
    if (qrow_out[qb] < 0) continue;
    if (p.splits > 1) {
      // partial over this split's keys: unnormalised O, row max and row sum
      const int64_t prow = (int64_t)split * p.batch_rows + (int64_t)b * p.tokens_out + qrow_out[qb];
      float* po = p.part_o + prow * D + head * hd;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = db * 32 + 8 * gq + 4 * h;
          if (d < hd)
            *reinterpret_cast<f32x4*>(po + d) = f32x4{acc_o[qb][db][4 * gq], acc_o[qb][db][4 * gq + 1],
                                                      acc_o[qb][db][4 * gq + 2], acc_o[qb][db][4 * gq + 3]};
        }
      if (h == 0) *reinterpret_cast<f32x2*>(p.part_ml + (prow * p.heads + head) * 2) = f32x2{m_run[qb], l};
      continue;
    }
    const float inv = 1.0f / l;
    bf16* out = p.ctx + ((int64_t)b * p.tokens_out + qrow_out[qb]) * p.ld_ctx + head * hd;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * h;
        if (d < hd)
          store4<bf16>(out + d, f32x4{acc_o[qb][db][4 * gq], acc_o[qb][db][4 * gq + 1], acc_o[qb][db][4 * gq + 2],
                                      acc_o[qb][db][4 * gq + 3]} * inv);
      }
  }
}
// Key-split partials -> ctx: for each (row, head), weights 2^((m_s - m) c)
// with m the largest split max; ctx = sum_s w_s O_s / sum_s w_s l_s.
// One thread per 4 consecutive d of one (row, head).
constexpr int SPLITS_MAX = 8;  // attention_splits() never returns more
template <int S>
__global__ __launch_bounds__(256) void attention_combine_kernel(const float* __restrict__ part_o,
                                                                const float* __restrict__ part_ml, bf16* ctx,
                                                                int64_t ld_ctx, int64_t rows, int heads, int hd,
                                                                int dim, float c) {
  const int q4 = hd / 4;
  const int64_t idx = (int64_t)wg_id() * 256 + wi_id();
  const int64_t r = idx / (heads * q4);
  if (r >= rows) return;
  const int rem = (int)(idx - r * heads * q4), head = rem / q4, d = (rem - head * q4) * 4;
  // every split's (m, l) and O are requested before the first is used: one
  // memory round trip instead of two per split
  f32x2 ml[S];
  f32x4 po[S];
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    ml[sp] = *reinterpret_cast<const f32x2*>(part_ml + ((sp * rows + r) * heads + head) * 2);
    po[sp] = *reinterpret_cast<const f32x4*>(part_o + (sp * rows + r) * dim + head * hd + d);
  }
  float m = ml[0][0];
#pragma unroll
  for (int sp = 1; sp < S; ++sp) m = fmaxf(m, ml[sp][0]);
  float l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    const float w = __builtin_amdgcn_exp2f((ml[sp][0] - m) * c);
    l += w * ml[sp][1];
    o += w * po[sp];
  }
  store4<bf16>(ctx + r * ld_ctx + head * hd + d, o * (1.0f / l));
}

template <int S>
static void combine_go(const AttnParams<bf16>& p, hipStream_t s, hipEvent_t stop) {
  const int64_t threads = p.batch_rows * p.heads * (p.head_dim / 4);
  hipExtLaunchKernelGGL(attention_combine_kernel<S>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                        nullptr, stop, 0, (const float*)p.part_o, (const float*)p.part_ml, p.ctx, p.ld_ctx,
                        p.batch_rows, p.heads, p.head_dim, p.dim, p.scale_log2);
}

template <int NW, int QB, int MODE, bool POOL, bool KSW = false>
static hipError_t attn32_go(AttnParams<bf16> p, int batch, hipStream_t s, StageEvents ev) {
  if (KSW) p.splits = 1;
  p.q_tiles = KSW ? (p.n_q + 32 * QB - 1) / (32 * QB) : (p.n_q + 32 * QB * NW - 1) / (32 * QB * NW);
  const int64_t blocks = (int64_t)batch * p.windows * p.q_tiles * p.heads;
  if (blocks == 0) return hipSuccess;
  p.batch_rows = (int64_t)batch * p.tokens_out;
  const hipEvent_t stop = p.splits > 1 ? nullptr : ev.stop;
  hipExtLaunchKernelGGL((attention_mfma32_kernel<NW, QB, MODE, POOL, KSW>), dim3((unsigned)(blocks * p.splits)),
                        dim3(64 * NW), 0, s, ev.start, stop, 0, p);
  switch (p.splits) {
    case 1: break;
    case 2: combine_go<2>(p, s, ev.stop); break;
    case 3: combine_go<3>(p, s, ev.stop); break;
    case 4: combine_go<4>(p, s, ev.stop); break;
    case 5: combine_go<5>(p, s, ev.stop); break;
    case 6: combine_go<6>(p, s, ev.stop); break;
    case 7: combine_go<7>(p, s, ev.stop); break;
    case 8: combine_go<8>(p, s, ev.stop); break;
    default: return hipErrorInvalidValue;  // more than SPLITS_MAX
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Large windows, head_dim 64, on head-major operands (written in window
// order by the qkv projection): q [B, windows, heads, n, 64] already
// multiplied by scale * log2 e, k likewise, V^T [B, windows, heads, 64, n].
// One workgroup = NW waves of 32 queries of one (frame, window, head); a
// wave computes S^T = K Q^T (keys on the MFMA rows, so a lane holds 16 keys
// of ONE query) and O^T += V^T P^T, K and V^T tiles of 64 keys streamed
// into LDS by buffer loads (the tile offset is a scalar: no per-lane
// address arithmetic).
//
// Softmax without a running maximum: q arrives multiplied by scale * log2 e,
// so the MFMA returns c*s and P = exp2(c*s) directly -- one exponential per
// score, no per-tile maximum, no rescaling of O. Subtracting the row maximum
// (the stable form) changes every P and the row sum l by the same factor,
// which cancels in O / l; it only serves to keep exp2 in range. So the pass
// checks the range instead: if some row ends with l outside [2^-64, 2^64]
// (some c*s above 64, or every c*s of the row far below zero, or an
// overflow), the workgroup runs the window again with the running maximum
// subtracted (the classic online softmax). Within the range every P is at
// most 2^64 and the largest P of a row at least 2^-64 / n, so nothing
// overflows and the terms that matter stay normal floats. The row sums come
// from the bf16 P that multiply V (dot products with (1, 1) over packed
// pairs).
// Trained weights give rows whose largest c*s is in the hundreds, far out
// of that band, so each wave first takes tile 0's scores: if some row's
// maximum over them lies outside [-m_band, m_band], the wave runs the
// running-maximum pass at once (from those scores) instead of a pass that
// would be discarded. (Decided per wave, with a ballot: a decision shared
// by the workgroup, through a barrier, cost 3 % on the small-score path.)
// ---------------------------------------------------------------------------
struct AttnHmParams {
  const bf16* q;
  const bf16* k;
  const bf16* vt;
  bf16* ctx;
  int64_t ld_ctx;
  int n;                 // tokens per window (queries = keys)
  int groups, heads;     // groups = B * windows * heads
  int windows;           // per frame
  int spatial, grid_w, win_h, win_w, tokens_per_frame;
  float l_lo, l_hi;      // the band a row sum must fall in (2^-64, 2^64)
  float m_band;          // tile 0's row maxima of c*s outside [-m_band, m_band]: running-maximum pass at once
};

constexpr uint32_t BUF_WORD3 = 0x00020000;  // raw buffer, 32-bit data, range-checked

// (the operands are wave-uniform; readfirstlane lets the compiler keep the
// descriptor in SGPRs instead of looping over lanes)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ptr = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ptr, (short)0, __builtin_amdgcn_readfirstlane(bytes), BUF_WORD3);
}

// 16 bytes per lane from a buffer into LDS (lane l's at lds + 16 l bytes)
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, bf16* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (attn_lds_ptr)lds, 16, voff, 0, 0, 0);
}

template <int NW>
__global__ __launch_bounds__(64 * NW, 3) void attention_hm_kernel(AttnHmParams p) {
  static_assert(KT == 64 && (KT / 8) % NW == 0, "64-key tiles split over the waves");
  constexpr int LPW = KT / 8 / NW;  // 1 KB buffer loads per wave per tile, for K and for V^T each
  // one array per stage: the compiler can then tell that a tile's buffer
  // loads into one stage never alias the LDS reads of the other (with one
  // array it waits for the prefetch before every read)
  __shared__ __attribute__((aligned(1024))) bf16 Ks0[KT * 64];
  __shared__ __attribute__((aligned(1024))) bf16 Vs0[64 * KT];
  __shared__ __attribute__((aligned(1024))) bf16 Ks1[KT * 64];
  __shared__ __attribute__((aligned(1024))) bf16 Vs1[64 * KT];

  const int tid = wi_id(), lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, h = lane >> 5;
  // consecutive workgroups share (frame, window, head): with groups a
  // multiple of 8 all query tiles of a group land on one XCD (its L2)
  const int g = wg_id() % p.groups, qt = wg_id() / p.groups;
  const int n = p.n;
  const int64_t gbase = (int64_t)g * n * 64;
  const bf16* kg = p.k + gbase;
  const bf16* vg = p.vt + gbase;

  // Q fragments (B operand): lane holds q[qi][16ks + 8h .. +7]
  const int qi = (qt * NW + wave) * 32 + fr;
  const bool qvalid = qi < n;
  u32x4 qf[4];
  {
    const bf16* qr = p.q + gbase + (int64_t)(qvalid ? qi : 0) * 64 + h * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = qvalid ? ld16(qr + ks * 16) : u32x4{0, 0, 0, 0};
  }

  // per-lane byte offsets of the K and V^T tile loads (fixed over tiles).
  // K: LDS row R holds key key_of_row(R), its 16-byte chunks XOR-swizzled;
  // V^T: LDS row R = d, chunk c = keys 8c .. 8c+7 of the tile, swizzled.
  int koff[LPW], voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int row = (wave * LPW + j) * 8 + lane / 8;
    const int ch = (lane & 7) ^ kswz(row);
    koff[j] = (key_of_row(row) * 64 + ch * 8) * 2;
    voff[j] = (row * n + ch * 8) * 2;
  }
  const int ntiles = (n + KT - 1) / KT;
  // the wave index as a scalar: the LDS destinations of the tile loads are
  // then scalar arithmetic, not vector registers
  const int waveu = __builtin_amdgcn_readfirstlane(wave);
  // tile kt's K and V^T into one stage's LDS arrays
  auto issue = [&](bf16* kd, bf16* vd, int kt) {
    // bytes from the tile's start to the end of the (frame, window, head)
    // block: loads past it return zeros
    const __amdgpu_buffer_rsrc_t kr = buf_rsrc(kg + (int64_t)kt * KT * 64, (n - kt * KT) * 128);
    const __amdgpu_buffer_rsrc_t vr = buf_rsrc(vg + (int64_t)kt * KT, (n * 64 - kt * KT) * 2);
#pragma unroll
    for (int j = 0; j < LPW; ++j) buf_load_lds16(kr, kd + (waveu * LPW + j) * 512, koff[j]);
#pragma unroll
    for (int j = 0; j < LPW; ++j) buf_load_lds16(vr, vd + (waveu * LPW + j) * 512, voff[j]);
  };

  f32x16 acc_o[2] = {f32x16{}, f32x16{}};  // O^T[d = 32db + 8(r/4) + 4h + r%4][query]
  float l = 0.f;                            // this lane's share of the row sum
  const bf16x2_t ones = {(bf16)1.f, (bf16)1.f};
  f32x16 sacc[2];

  // S^T (c*s) of the tile in LDS at ks, ragged keys at -1e30
  auto scores = [&](const bf16* ks, int kt) {
    // the two key blocks' MFMA chains interleaved
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = kb * 32 + fr;
        const u32x4 kfr = ld16(ks + row * 64 + ((q * 2 + h) ^ kswz(row)) * 8);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kfr),
                                                           __builtin_bit_cast(bf16x8, qf[q]),
                                                           q == 0 ? f32x16{} : sacc[kb], 0, 0, 0);
      }
    const int kv_left = n - kt * KT;
    if (kv_left < KT) {  // uniform: only the last tile of a ragged window
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key_of_row(kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) >= kv_left) sacc[kb][r] = -1e30f;
    }
  };
  // P = exp2(sacc) in bf16, its row sums, and O^T += V^T P^T for one tile
  // whose V^T is in LDS at vs
  auto pv_step = [&](const bf16* vs) {
    u32x4 pf[2][2];  // [kb][s]: keys 32kb + 16s + 8h + 0..7
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = (bf16)__builtin_amdgcn_exp2f(sacc[kb][8 * s + e]);
        pf[kb][s] = __builtin_bit_cast(u32x4, pv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2_t pr = {pv[2 * e], pv[2 * e + 1]};
          l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
        }
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int row = db * 32 + fr;
          const u32x4 vf = ld16(vs + row * 64 + ((4 * kb + 2 * s + h) ^ kswz(row)) * 8);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf),
                                                             __builtin_bit_cast(bf16x8, pf[kb][s]), acc_o[db], 0, 0, 0);
        }
  };
  // one tile kt in LDS at (ks, vs): wait for its loads, start tile kt + 1's
  // into the other stage (kn, vn), then S and P V. Every call site passes
  // the stage arrays themselves, so the compiler sees which LDS each access
  // touches.
  auto step = [&](const bf16* ks, const bf16* vs, bf16* kn, bf16* vn, int kt) {
    __builtin_amdgcn_s_waitcnt(attn_vmcnt(0));
    __syncthreads();
    if (kt + 1 < ntiles) issue(kn, vn, kt + 1);
    scores(ks, kt);
    // the exponentials and P V at a higher wave priority: a wave that has
    // its scores moves on to its PV MFMAs ahead of the other waves' S MFMAs
    // on the same SIMD (measured 3-4 % on the 5184-token global window)
    __builtin_amdgcn_s_setprio(2);
    pv_step(vs);
    __builtin_amdgcn_s_setprio(0);
  };

  // Tile 0's scores choose each wave's pass: where some row of the wave has
  // its maximum over them outside [-m_band, m_band], the running-maximum
  // pass from these scores, otherwise the pass without a running maximum.
  // Both run one barrier per tile, so the waves of a workgroup may differ.
  issue(Ks0, Vs0, 0);
  __builtin_amdgcn_s_waitcnt(attn_vmcnt(0));
  __syncthreads();
  if (1 < ntiles) issue(Ks1, Vs1, 1);
  scores(Ks0, 0);
  float mt0 = -1e30f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mt0 = fmaxf(mt0, sacc[kb][r]);
  mt0 = halves_max(mt0);
  const bool wide = wave_any(!(mt0 >= -p.m_band && mt0 <= p.m_band));
  float m = -1e30f;
  // the running row maximum m subtracted and O, l rescaled as it grows
  auto rm_softmax_pv = [&](const bf16* vs) {
    float mt = -1e30f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
    const float m_new = fmaxf(m, halves_max(mt));
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
#pragma unroll
    for (int db = 0; db < 2; ++db) acc_o[db] *= alpha;
    l *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sacc[kb] -= m;
    pv_step(vs);
  };
  auto step_rm = [&](const bf16* ks, const bf16* vs, bf16* kn, bf16* vn, int kt) {
    __builtin_amdgcn_s_waitcnt(attn_vmcnt(0));
    __syncthreads();
    if (kt + 1 < ntiles) issue(kn, vn, kt + 1);
    scores(ks, kt);
    rm_softmax_pv(vs);
  };
  // tile kt in stage kt & 1, tiles after the first taken in pairs so that
  // the stage of each is known at compile time
  if (wide) {
    rm_softmax_pv(Vs0);
    for (int kt = 1; kt < ntiles; kt += 2) {
      step_rm(Ks1, Vs1, Ks0, Vs0, kt);
      if (kt + 1 < ntiles) step_rm(Ks0, Vs0, Ks1, Vs1, kt + 1);
    }
  } else {
    __builtin_amdgcn_s_setprio(2);
    pv_step(Vs0);
    __builtin_amdgcn_s_setprio(0);
    for (int kt = 1; kt < ntiles; kt += 2) {
      step(Ks1, Vs1, Ks0, Vs0, kt);
      if (kt + 1 < ntiles) step(Ks0, Vs0, Ks1, Vs1, kt + 1);
    }
  }
  l += __shfl_xor(l, 32, 64);
  const bool running_max = wg_any<NW>(!wide && !(l >= p.l_lo && l <= p.l_hi));

  if (running_max) {
    // a row of a wave without the running maximum left the band: the whole
    // workgroup runs the window again from the start, every wave with the
    // running maximum
    acc_o[0] = f32x16{};
    acc_o[1] = f32x16{};
    l = 0.f;
    m = -1e30f;
    issue(Ks0, Vs0, 0);
    for (int kt = 0; kt < ntiles; ++kt) {
      const int stage = kt & 1;
      __builtin_amdgcn_s_waitcnt(attn_vmcnt(0));
      __syncthreads();
      if (kt + 1 < ntiles) {
        if (stage) issue(Ks0, Vs0, kt + 1);
        else issue(Ks1, Vs1, kt + 1);
      }
      scores(stage ? Ks1 : Ks0, kt);
      rm_softmax_pv(stage ? Vs1 : Vs0);
    }
    l += __shfl_xor(l, 32, 64);
  }

  // the query row again, from scalars and the lane's index: recomputed so
  // that no register carries it across the passes (with 168 VGPRs in use
  // it was spilled to scratch, and a kernel with scratch costs more to
  // dispatch)
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int qo = (qt * NW + waveu) * 32 + (lane_e & 31);
  if (qo >= n) return;
  // output row of query qo: its token in the frame
  const int bw = g / p.heads, head = g - bw * p.heads;
  const int b = bw / p.windows, win = bw - b * p.windows;
  int t = qo;
  if (p.spatial) {
    const int nwx = p.grid_w / p.win_w, wy = win / nwx, wx = win - wy * nwx;
    const int iy = qo / p.win_w, ix = qo - iy * p.win_w;
    t = (wy * p.win_h + iy) * p.grid_w + wx * p.win_w + ix;
  }
  const float inv = 1.0f / l;
  bf16* out = p.ctx + ((int64_t)b * p.tokens_per_frame + t) * p.ld_ctx + head * 64;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
      store4<bf16>(out + db * 32 + 8 * gq + 4 * h,
                   f32x4{acc_o[db][4 * gq], acc_o[db][4 * gq + 1], acc_o[db][4 * gq + 2], acc_o[db][4 * gq + 3]} * inv);
}


static hipError_t attn_hm_go(const AttnArgs& a, hipStream_t s, StageEvents ev) {
  AttnHmParams p;
  p.q = (const bf16*)a.qh;
  p.k = (const bf16*)a.kh;
  p.vt = (const bf16*)a.vt;
  p.ctx = (bf16*)a.ctx;
  p.ld_ctx = a.ld_ctx;
  p.spatial = a.mode == ATTN_SPATIAL;
  p.n = p.spatial ? a.win_h * a.win_w : a.tokens_in;
  p.windows = a.tokens_in / p.n;
  p.heads = a.heads;
  p.groups = a.batch * p.windows * a.heads;
  p.grid_w = a.grid_w;
  p.win_h = a.win_h;
  p.win_w = a.win_w;
  p.tokens_per_frame = a.tokens_in;
  attn_band(p.l_lo, p.l_hi);
  p.m_band = attn_tile0_band();
  constexpr int NW = 4;
  const int q_tiles = (p.n + 32 * NW - 1) / (32 * NW);
  const int64_t blocks = (int64_t)p.groups * q_tiles;
  if (blocks == 0) return hipSuccess;
  hipExtLaunchKernelGGL(attention_hm_kernel<NW>, dim3((unsigned)blocks), dim3(64 * NW), 0, s, ev.start, ev.stop, 0, p);
  return hipGetLastError();
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
  if (a.qh != nullptr) {
    if (!std::is_same<T, bf16>::value || !a.kh || !a.vt || a.q_stride != 1 || a.head_dim != 64 ||
        a.dim != 64 * a.heads || a.ld_ctx % 8 ||
        (a.mode == ATTN_SPATIAL ? (a.win_w % 8 || a.tokens_in % (a.win_h * a.win_w)) : a.mode != ATTN_GLOBAL))
      return hipErrorInvalidValue;
    return attn_hm_go(a, s, ev);
  }
  p.vt = (const T*)a.vt;
  attn_band(p.l_lo, p.l_hi);
  p.m_band = attn_tile0_band();
  p.splits = 1;
  p.batch_rows = 0;
  p.part_o = a.part_o;
  p.part_ml = a.part_ml;
  if (a.vt) {
    p.splits = attention_splits(a.batch, p.windows, p.n_q, p.n_kv, a.heads);
    const bool ksw = attention_split_in_workgroup(p.splits, p.n_kv);
    if (p.splits > 1 && (a.head_dim % 4 || (!ksw && (!a.part_o || !a.part_ml)))) return hipErrorInvalidValue;
    // large global or spatial windows: 32x32 MFMA kernel on K and V^T
    if (!std::is_same<T, bf16>::value ||
        !attention_takes_vt(DType::BF16, a.mode, p.n_q, a.head_dim, a.win_w, a.tokens_in,
                            (int64_t)a.batch * a.tokens_in * a.ld_qkv))
      return hipErrorInvalidValue;
    if constexpr (std::is_same<T, bf16>::value) {
      // a split of 4 (64-85 query tiles) or 2 over at most 16 key tiles
      // becomes a split among the four waves of each workgroup (128 KB of
      // LDS, one per CU): no partials and no combine launch (Hiera
      // 1024-token blocks: 256 workgroups; 256-token blocks: 128). Each
      // wave loads its own K / V^T tiles, four times the LDS fill of a
      // shared tile, so longer windows (the 4096 keys of the pooled
      // stage-2 transition: 35.8 us against 29 + 3.7 for the combine) keep
      // the split over workgroups.
      if (ksw) {
        if (a.mode == ATTN_SPATIAL) return attn32_go<ATTN_NW, ATTN_QB, ATTN_SPATIAL, false, true>(p, a.batch, s, ev);
        return pool ? attn32_go<ATTN_NW, ATTN_QB, ATTN_GLOBAL, true, true>(p, a.batch, s, ev)
                    : attn32_go<ATTN_NW, ATTN_QB, ATTN_GLOBAL, false, true>(p, a.batch, s, ev);
      }
      if (a.mode == ATTN_SPATIAL)
        return attn32_go<ATTN_NW, ATTN_QB, ATTN_SPATIAL, false>(p, a.batch, s, ev);
      return pool ? attn32_go<ATTN_NW, ATTN_QB, ATTN_GLOBAL, true>(p, a.batch, s, ev)
                  : attn32_go<ATTN_NW, ATTN_QB, ATTN_GLOBAL, false>(p, a.batch, s, ev);
    }
  }
  // small query sets: several heads per workgroup, one wave each -- unless
  // that leaves fewer workgroups than CUs (the 64 mask units of a 4096-token
  // Hiera transition): then one head per workgroup (three of its four waves
  // idle, but four times the workgroups; 8.3 -> 6.5 us there)
  if (p.n_q <= 16 && a.heads % 4 == 0 && (int64_t)a.batch * p.windows * (a.heads / 4) < 256) {
    return pool ? attn_go<T, 1, 1, true>(a, p, s, ev) : attn_go<T, 1, 1, false>(a, p, s, ev);
  }
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
