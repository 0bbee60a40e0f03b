// Whole encoder block for one Hiera mask unit in one workgroup.
//
// Mask-unit windows are independent through the entire block: LayerNorm,
// the projections and the MLP act on token rows, and attention never leaves
// the window (Hiera plan, "MaskUnitAttention"). So for small mask units
// (64 tokens, width <= 128) a workgroup reads the window's 64 token rows
// once, keeps every intermediate in LDS (h, q|k|v, V^T, ctx, x1, h2, u) and
// writes the 64 output rows once: HBM traffic is x in, y out and the
// (L2-resident) weights, instead of seven kernels' worth of round trips.
//
// Weights are read straight from global memory into MFMA fragments (each
// 16-row weight tile is fetched once per workgroup and reused for all four
// 16-token tiles); activations come from LDS. All products are 16x16x32
// bf16 MFMAs with fp32 accumulation, with the weight tile as the A operand
// so that a lane ends with 4 consecutive output columns of one token.
#include "common.h"
#include "launch.h"

#include <hip/hip_ext.h>

namespace vit {

namespace {

constexpr int TW = 64;             // tokens per mask unit
constexpr int DP = 128;            // padded width (K of the D-wide products)
#ifndef FUSED_WAVES
#define FUSED_WAVES 16
#endif
constexpr int NWF = FUSED_WAVES;   // waves per workgroup
constexpr int HPR = NWF / 4;       // heads per attention round (4 waves of 16 queries each)
constexpr int XS = DP + 16;        // LDS row stride of the D-wide buffers (elements; +16: 40 % fewer bank conflicts than +8)
constexpr int VTS = TW + 8;        // V^T row stride
constexpr int QS_MAX = 3 * DP + 8;  // q|k|v row stride for the widest supported block
constexpr int US_MAX = 512 + 8;     // u row stride for the widest supported MLP
constexpr int A_MAX = (TW * QS_MAX + HPR * 64 * VTS) > (TW * US_MAX) ? (TW * QS_MAX + HPR * 64 * VTS) : (TW * US_MAX);
constexpr int BIAS_MAX = 3 * DP + DP + 512 + DP;  // b_q|b_k|b_v, b_o, b_1, b_2 (fp32)
// bf16 elements; fp32 LN params, biases and (q8_row weights) the row scales last
constexpr int LDS_ELEMS = 3 * TW * XS + A_MAX + 2 * 4 * DP + 2 * BIAS_MAX + 2 * BIAS_MAX;

struct FusedParams {
  const bf16* x;
  bf16* y;
  const float *ln1_g, *ln1_b, *ln2_g, *ln2_b;
  const bf16 *wq, *wk, *wv;  // qkv weight rows for q, k and v (each [D, D])
  const float *bq, *bk, *bv;
  const bf16* wo;
  const float* bo;
  const bf16* w1;
  const float* b1;
  const bf16* w2;
  const float* b2;
  int tokens, n_windows, dim, heads, head_dim, mlp, qs, us;  // qs/us: LDS row strides of q|k|v and u
  float eps, inv_dim, scale_log2;
  // q8_row weights: the matrices above are int8 payloads (row stride = K
  // bytes) and these their float16 row scales
  const _Float16 *sq, *sk, *sv, *so, *s1, *s2;
};

__device__ __forceinline__ float gelu_erf_d(float v) { return gelu_erf_as(v); }
__device__ __forceinline__ float gelu_tanh_d(float v) { return gelu_tanh_fast(v); }

// Row LayerNorm of the window's 64 rows (src -> dst, both LDS, stride XS),
// 8 lanes per row; columns D..DP-1 of dst are written as zeros so that dst
// can feed a K=DP product.
__device__ __forceinline__ void ln_rows(const bf16* src, bf16* dst, const float* g, const float* bta, int D, float inv_d,
                                        float eps) {
  constexpr int LPR = NWF;             // lanes per row: 64 rows over 64*NWF threads
  constexpr int CPL = (DP / 8) / LPR;  // 16-byte chunks per lane
  static_assert(CPL >= 1 && LPR <= 64, "LayerNorm lane split");
  const int tid = threadIdx.x;
  const int row = tid / LPR, l8 = tid % LPR;
  const int nch = D / 8;
  float v[CPL][8];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = l8 + LPR * i;
    if (c < nch) {
      unpack16<bf16>(ld16(src + row * XS + c * 8), v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[i][e];
    }
  }
  static_assert(LPR == 16, "row reductions are 16-lane DPP");
  s = row16_sum(s);
  const float mean = s * inv_d;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i)
    if (l8 + LPR * i < nch)
#pragma unroll
      for (int e = 0; e < 8; ++e) q += (v[i][e] - mean) * (v[i][e] - mean);
  q = row16_sum(q);
  const float inv = __builtin_amdgcn_rsqf(q * inv_d + eps);  // hardware rsq, ~1 ulp
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = l8 + LPR * i;
    float o[8];
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[i][e] - mean) * inv * g[c * 8 + e] + bta[c * 8 + e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = 0.f;
    }
    st16(dst + row * XS + c * 8, pack16<bf16>(o));
  }
}

// Weight fragments of one product, held in registers: this wave's 16-row
// weight tiles nt = wave + i*NWF (i < NTM) for K steps kk < KSM (16x32 each,
// zero past N or kreal). Loading them one phase ahead hides the L2 latency
// behind the previous phase's work. Every load is issued unconditionally (at
// a clamped address, its value then selected away), so that the compiler
// can count outstanding loads exactly and the products wait only for their
// own fragments.
template <int NTM, int KSM>
struct WFrags {
  u32x4 f[NTM][KSM];
  // wrow(n): start of weight row n (bf16, or int8 payload when Q8: its 8
  // values are widened to bf16, exactly since |q| <= 127)
  template <bool Q8, typename Wsel>
  __device__ __forceinline__ void load(Wsel wrow, int N, int kreal) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int fr = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < NTM; ++i) {
      const int nt = wave + i * NWF;
      const bool nok = nt * 16 < N;
      const void* wr = wrow(nok ? nt * 16 + fr : 0);
#pragma unroll
      for (int kk = 0; kk < KSM; ++kk) {
        const int k = kk * 32 + g * 8;
        const bool ok = nok && k < kreal;
        const int kc = ok ? k : 0;  // kreal >= 8
        if constexpr (Q8) {
          // (int8 payloads are widened as they arrive; loaded under the
          // lane's own condition, which keeps the widening's registers short-lived)
          if (!ok) {
            f[i][kk] = u32x4{0, 0, 0, 0};
          } else {
            const u32x2 q = *reinterpret_cast<const u32x2*>(static_cast<const int8_t*>(wr) + k);
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (float)(int8_t)((q[e / 4] >> (8 * (e % 4))) & 0xFF);
            f[i][kk] = pack16<bf16>(v);
          }
        } else {
          const u32x4 w = ld16(static_cast<const bf16*>(wr) + kc);
          f[i][kk] = ok ? w : u32x4{0, 0, 0, 0};
        }
      }
    }
  }
  // C[64, N] = LDS A[64, K] * W^T; epi(m, n, v) gets 4 consecutive columns
  // n..n+3 of token m. Each A fragment is read once per wave and used for
  // all of the wave's weight tiles; each weight fragment serves 4 token
  // tiles. K steps past kreal multiply zero weights by a finite A fragment
  // (the last real step's), so the step loop has no branches.
  // With bias0 (fp32, LDS), the accumulators start from bias0[n..n+3].
  template <typename Epi>
  __device__ __forceinline__ void gemm(const bf16* As, int lda, int N, int kreal, const float* bias0, Epi epi) const {
    const int wave = threadIdx.x >> 6;
    int nv = 0;
#pragma unroll
    for (int i = 0; i < NTM; ++i) nv += (wave + i * NWF) * 16 < N ? 1 : 0;
    gemm_nv<NTM>(nv, As, lda, kreal, bias0, epi);
  }

 private:
  template <int NV, typename Epi>
  __device__ __forceinline__ void gemm_nv(int nv, const bf16* As, int lda, int kreal, const float* bias0, Epi epi) const {
    if constexpr (NV > 1) {
      if (nv < NV) {
        gemm_nv<NV - 1>(nv, As, lda, kreal, bias0, epi);
        return;
      }
    } else {
      if (nv < 1) return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int fr = lane & 15, g = lane >> 4;
    const int klast = (kreal + 31) / 32 - 1;
    f32x4 acc0[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
      acc0[i] = bias0 ? *reinterpret_cast<const f32x4*>(bias0 + (wave + i * NWF) * 16 + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < TW / 16; ++mt) {
      f32x4 acc[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] = acc0[i];
      const bf16* arow = As + (mt * 16 + fr) * lda + g * 8;
#pragma unroll
      for (int kk = 0; kk < KSM; ++kk) {
        const u32x4 a = ld16(arow + (kk < klast ? kk : klast) * 32);
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] = Mma<bf16>::step(f[i][kk], a, acc[i]);
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) epi(mt * 16 + fr, (wave + i * NWF) * 16 + 4 * g, acc[i]);
    }
  }
};

// Workgroup barrier that waits only for this wave's LDS operations, so
// weight loads issued for a later phase stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool TANH, bool Q8>
__global__ __launch_bounds__(64 * NWF) void block_mask_unit_kernel(FusedParams p) {
  // one static allocation sized for the largest supported block (static LDS
  // can use the CU's full 160 KB)
  __shared__ __attribute__((aligned(16))) bf16 smem[LDS_ELEMS];
  bf16* xs = smem;                   // x rows            [TW][XS]
  bf16* cs = xs + TW * XS;           // h, then ctx, then h2
  bf16* x1s = cs + TW * XS;          // x1 rows
  bf16* qkvs = x1s + TW * XS;        // q|k|v rows        [TW][qs]
  bf16* vts = qkvs + TW * p.qs;      // V^T of one round's heads [HPR][64][VTS]
  bf16* uss = qkvs;                  // u rows (after attention) [TW][us]
  float* lnp = reinterpret_cast<float*>(smem + 3 * TW * XS + A_MAX);  // LN1/LN2 g, b [4][DP]
  float* bqkv = lnp + 4 * DP;          // [3D] biases of q|k|v
  float* bo_s = bqkv + 3 * DP;         // [D]
  float* b1_s = bo_s + DP;             // [mlp]
  float* b2_s = b1_s + 512;            // [D]
  float* sqkv = b2_s + DP;             // Q8: row scales, laid out like the biases
  float* so_s = sqkv + 3 * DP;
  float* s1_s = so_s + DP;
  float* s2_s = s1_s + 512;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = p.dim, hd = p.head_dim;
  const int win = blockIdx.x % p.n_windows, b = blockIdx.x / p.n_windows;
  const int64_t row0 = (int64_t)b * p.tokens + win;  // global row of token t: row0 + t * n_windows

  // Q8: the accumulator of output column n..n+3 times its row scales
  // (bf16 weights: the products start from the bias, so v already holds it)
  auto scaled = [&](f32x4 v, const float* sc, const float* bias, int n) {
    if constexpr (Q8) v = v * *reinterpret_cast<const f32x4*>(sc + n) + *reinterpret_cast<const f32x4*>(bias + n);
    return v;
  };
  auto bias0 = [&](const float* bias) -> const float* { return Q8 ? nullptr : bias; };
  // row start of a weight matrix with rows of K values
  auto wrow_of = [&](const bf16* w, int64_t n, int K) -> const void* {
    if constexpr (Q8) return reinterpret_cast<const int8_t*>(w) + n * K;
    return w + n * K;
  };
  // ---- x rows of the window, the LN parameters and the biases -> LDS;
  // q|k|v weights -> registers. Every global read of this phase is issued
  // before the first LDS store (addresses clamped, values selected), so they
  // overlap in one round trip, and the weights last, so that the stores
  // wait only for the small reads ahead of them.
  constexpr int NT = 64 * NWF;
  static_assert(TW * (DP / 8) <= NT && 4 * DP <= NT && BIAS_MAX <= 2 * NT, "prologue covers");
  const int nch = D / 8;
  const bool x_ok = tid < TW * nch;
  const int xt = x_ok ? tid / nch : 0, xc = x_ok ? tid - (tid / nch) * nch : 0;
  const u32x4 xv = ld16(p.x + (row0 + (int64_t)xt * p.n_windows) * D + xc * 8);
  const bool l_ok = tid < 4 * D;
  const int lwhich = l_ok ? tid / D : 0, lc = l_ok ? tid - (tid / D) * D : 0;
  const float* lsrc = lwhich == 0 ? p.ln1_g : lwhich == 1 ? p.ln1_b : lwhich == 2 ? p.ln2_g : p.ln2_b;
  const float lv = lsrc[lc];
  // biases (and Q8 row scales) e < 5D + mlp: q|k|v, o, 2, then 1
  const int nb = 5 * D + p.mlp;
  float bvv[2], svv[2];
  int boff[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int e0 = tid + r * NT, e = e0 < nb ? e0 : 0;
    int seg = e < D ? 0 : e < 2 * D ? 1 : e < 3 * D ? 2 : e < 4 * D ? 3 : e < 5 * D ? 4 : 5;
    const int i = seg < 5 ? e - seg * D : e - 5 * D;
    const float* bsrc = seg == 0 ? p.bq : seg == 1 ? p.bk : seg == 2 ? p.bv : seg == 3 ? p.bo : seg == 4 ? p.b2 : p.b1;
    bvv[r] = bsrc[i];
    if constexpr (Q8) {
      const _Float16* ssrc = seg == 0 ? p.sq : seg == 1 ? p.sk : seg == 2 ? p.sv : seg == 3 ? p.so : seg == 4 ? p.s2 : p.s1;
      svv[r] = (float)ssrc[i];
    }
    // LDS float offset from bqkv: q|k|v at 0, o at 3DP, 1 at 4DP, 2 at 4DP + 512
    boff[r] = e0 >= nb ? -1 : seg < 3 ? e : seg == 3 ? 3 * DP + i : seg == 4 ? 4 * DP + 512 + i : 4 * DP + i;
  }
  WFrags<(3 * DP / 16 + NWF - 1) / NWF, DP / 32> wqkv;
  wqkv.load<Q8>([&](int n) { return n < D ? wrow_of(p.wq, n, D) : (n < 2 * D ? wrow_of(p.wk, n - D, D) : wrow_of(p.wv, n - 2 * D, D)); },
                3 * D, D);
  if (x_ok) st16(xs + xt * XS + xc * 8, xv);
  if (l_ok) lnp[lwhich * DP + lc] = lv;
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (boff[r] >= 0) {
      bqkv[boff[r]] = bvv[r];
      if constexpr (Q8) sqkv[boff[r]] = svv[r];
    }
  // with at most HPR heads the qkv epilogue writes V transposed straight into
  // vts (one attention round); rows head_dim..63 of each head stay zero
  const bool vt_direct = p.heads <= HPR;
  if (vt_direct) {
    const int pad = 64 - hd;  // multiple of 8
    for (int e = tid; e < p.heads * pad * (TW / 8); e += 64 * NWF) {
      const int hl = e / (pad * (TW / 8)), rem = e - hl * pad * (TW / 8);
      const int r = rem / (TW / 8), c = rem - r * (TW / 8);
      st16(vts + (hl * 64 + hd + r) * VTS + c * 8, u32x4{0, 0, 0, 0});
    }
  }
  lds_barrier();
  // ---- LN1 -> cs
  ln_rows(xs, cs, lnp, lnp + DP, D, p.inv_dim, p.eps);
  WFrags<(DP / 16 + NWF - 1) / NWF, DP / 32> wo;
  wo.load<Q8>([&](int n) { return wrow_of(p.wo, n, D); }, D, D);
  lds_barrier();
  // ---- q|k|v = h W^T + b -> qkvs
  wqkv.gemm(cs, XS, 3 * D, D, bias0(bqkv), [&](int m, int n, f32x4 v) {
    v = scaled(v, sqkv, bqkv, n);
    if (vt_direct && n >= 2 * D) {  // 4 consecutive d of one head (head_dim % 8 == 0)
      const int vv = n - 2 * D, head = vv / hd, d = vv - head * hd;
#pragma unroll
      for (int e = 0; e < 4; ++e) vts[(head * 64 + d + e) * VTS + m] = (bf16)v[e];
    } else {
      store4<bf16>(qkvs + m * p.qs + n, v);
    }
  });
  WFrags<(512 / 16 + NWF - 1) / NWF, DP / 32> w1;
  w1.load<Q8>([&](int n) { return wrow_of(p.w1, n, D); }, p.mlp, D);
  lds_barrier();

  // ---- attention, HPR heads per round (waves 4j..4j+3: head h0 + j)
  const int fr = lane & 15, g = lane >> 4;
  for (int h0 = 0; h0 < p.heads; h0 += HPR) {
    // V^T of the round's heads: [hl][d][key], zero past head_dim
    for (int e = tid; !vt_direct && e < HPR * TW * 8; e += 64 * NWF) {
      const int hl = e / (TW * 8), rem = e - hl * TW * 8;
      const int key = rem >> 3, c = rem & 7;
      const int head = h0 + hl;
      u32x4 v = {0, 0, 0, 0};
      if (head < p.heads && c * 8 < hd) v = ld16(qkvs + key * p.qs + 2 * D + head * hd + c * 8);
      const bf16x8 vv = __builtin_bit_cast(bf16x8, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) vts[(hl * 64 + c * 8 + k) * VTS + key] = vv[k];
    }
    if (!vt_direct) lds_barrier();
    const int hl = wave >> 2, qb = wave & 3, head = h0 + hl;
    if (head < p.heads) {
      // S^T = K Q^T: s[kb][r] = S[q = qb*16 + fr][key = kb*16 + 4g + r]
      u32x4 qf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int off = (ks * 4 + g) * 8;
        qf[ks] = off < hd ? ld16(qkvs + (qb * 16 + fr) * p.qs + head * hd + off) : u32x4{0, 0, 0, 0};
      }
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int off = (ks * 4 + g) * 8;
          const u32x4 kf = off < hd ? ld16(qkvs + (kb * 16 + fr) * p.qs + D + head * hd + off) : u32x4{0, 0, 0, 0};
          s[kb] = Mma<bf16>::step(kf, qf[ks], s[kb]);
        }
      }
      float mx = -1e30f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = pair32_max(pair16_max(mx));
      const float c = p.scale_log2, mc = mx * c;
      float l = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
          s[kb][r] = e;
          l += e;
        }
      l = pair32_sum(pair16_sum(l));
      // O^T = V^T P^T over two 32-key steps
      f32x4 o[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        bf16x8 pv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[r] = (bf16)s[2 * c2][r];
          pv[4 + r] = (bf16)s[2 * c2 + 1][r];
        }
        const u32x4 pf = __builtin_bit_cast(u32x4, pv);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16* vr = vts + (hl * 64 + db * 16 + fr) * VTS + 32 * c2 + 4 * g;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 16);
          o[db] = Mma<bf16>::step(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, o[db]);
        }
      }
      const float inv = 1.0f / l;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 16 + 4 * g;
        if (d < hd) store4<bf16>(cs + (qb * 16 + fr) * XS + head * hd + d, o[db] * inv);
      }
    }
    lds_barrier();
  }

  // ---- x1 = x + ctx W_o^T + b_o -> x1s (cs columns D..DP-1 are still zero)
  wo.gemm(cs, XS, D, D, bias0(bo_s),
      [&](int m, int n, f32x4 v) {
        v = scaled(v, so_s, bo_s, n) + load4<bf16>(xs + m * XS + n);
        store4<bf16>(x1s + m * XS + n, v);
      });
  lds_barrier();
  // ---- LN2 -> cs
  ln_rows(x1s, cs, lnp + 2 * DP, lnp + 3 * DP, D, p.inv_dim, p.eps);
  lds_barrier();
  // ---- u = GELU(h2 W_1^T + b_1) -> uss; fc2's weights are requested first
  // (after LN2's barrier, so issuing them does not hold up LN2)
  WFrags<1, 16> w2;
  w2.load<Q8>([&](int n) { return wrow_of(p.w2, n, p.mlp); }, D, p.mlp);
  w1.gemm(cs, XS, p.mlp, D, bias0(b1_s),
      [&](int m, int n, f32x4 v) {
        v = scaled(v, s1_s, b1_s, n);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = TANH ? gelu_tanh_d(v[e]) : gelu_erf_d(v[e]);
        store4<bf16>(uss + m * p.us + n, v);
      });
  lds_barrier();
  // ---- y = x1 + u W_2^T + b_2 -> global
  w2.gemm(uss, p.us, D, p.mlp, bias0(b2_s),
      [&](int m, int n, f32x4 v) {
        v = scaled(v, s2_s, b2_s, n) + load4<bf16>(x1s + m * XS + n);
        store4<bf16>(p.y + (row0 + (int64_t)m * p.n_windows) * D + n, v);
      });
}

}  // namespace

bool fused_mask_unit_supported(int dim, int heads, int head_dim, int mlp, int window_tokens) {
  return window_tokens == TW && dim % 16 == 0 && dim <= DP && head_dim % 8 == 0 && head_dim <= 64 &&
         heads * head_dim == dim && mlp % 32 == 0 && mlp <= 512;
}

size_t fused_mask_unit_lds_bytes(int dim, int mlp) {
  const size_t qs = 3 * dim + 8, us = mlp + 8;
  const size_t a = TW * qs + HPR * 64 * VTS, u = TW * us;
  return 2 * (3 * TW * XS + (a > u ? a : u));
}

hipError_t launch_block_mask_unit_fused(const FusedMUArgs& a, hipStream_t s, StageEvents ev) {
  FusedParams p;
  p.x = (const bf16*)a.x;
  p.y = (bf16*)a.y;
  p.ln1_g = a.ln1_g;
  p.ln1_b = a.ln1_b;
  p.ln2_g = a.ln2_g;
  p.ln2_b = a.ln2_b;
  p.wq = (const bf16*)a.wq;
  p.wk = (const bf16*)a.wk;
  p.wv = (const bf16*)a.wv;
  p.bq = a.bq;
  p.bk = a.bk;
  p.bv = a.bv;
  p.wo = (const bf16*)a.wo;
  p.bo = a.bo;
  p.w1 = (const bf16*)a.w1;
  p.b1 = a.b1;
  p.w2 = (const bf16*)a.w2;
  p.b2 = a.b2;
  p.tokens = a.tokens;
  p.n_windows = a.n_windows;
  p.dim = a.dim;
  p.heads = a.heads;
  p.head_dim = a.head_dim;
  p.mlp = a.mlp;
  p.qs = 3 * a.dim + 8;
  p.us = a.mlp + 8;
  p.eps = a.eps;
  p.inv_dim = 1.0f / (float)a.dim;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.sq = (const _Float16*)a.sq;
  p.sk = (const _Float16*)a.sk;
  p.sv = (const _Float16*)a.sv;
  p.so = (const _Float16*)a.so;
  p.s1 = (const _Float16*)a.s1;
  p.s2 = (const _Float16*)a.s2;
  const int64_t blocks = (int64_t)a.batch * a.n_windows;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(64 * NWF);
  if (a.q8) {
    if (a.gelu_tanh)
      hipExtLaunchKernelGGL((block_mask_unit_kernel<true, true>), grid, block, 0, s, ev.start, ev.stop, 0, p);
    else
      hipExtLaunchKernelGGL((block_mask_unit_kernel<false, true>), grid, block, 0, s, ev.start, ev.stop, 0, p);
  } else {
    if (a.gelu_tanh)
      hipExtLaunchKernelGGL((block_mask_unit_kernel<true, false>), grid, block, 0, s, ev.start, ev.stop, 0, p);
    else
      hipExtLaunchKernelGGL((block_mask_unit_kernel<false, false>), grid, block, 0, s, ev.start, ev.stop, 0, p);
  }
  return hipGetLastError();
}

}  // namespace vit
