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
#include <numeric>

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
  T* vt;  // transposed copy of columns >= vt_col0 (MFMA path only)
  int vt_col0, vt_tokens, vt_heads, vt_hd;
  bool vt_only;
  // head-major attention operands (GemmArgs::hm_q), MFMA path only
  T* hm_q;
  T* hm_k;
  float hm_qscale;
  bool hm_spatial;
  float hm_rcp[5];  // 1 / (vt_tokens, grid_w, win_h, win_w, tokens_per_frame)
  const float* pos;  // EPI_BIAS_POS: table [rows, N]
  int pos_mode, pos_side;
  // optional float16 scale per output column (per weight row), applied to
  // the accumulator before the bias: weights given as integers (q8_row
  // payloads converted exactly) times a row scale
  const _Float16* ws0;
  const _Float16* ws1;
  const _Float16* ws2;
};

// EPI_POOL's arguments: a fourth weight segment, the pooled output and its
// first column. A type of its own, so that the other kernels' argument
// block (and code) stays as it is.
template <typename T>
struct GemmPoolParams : GemmParams<T> {
  const T* W3;
  const float* b3;
  const _Float16* ws3;
  T* pool_out;
  int64_t ld_pool;
  int pool_col0;
};

// Eight zero floats: the bias of a GEMM without one.
__device__ __attribute__((aligned(16))) const float kZeros8[8] = {};

// Pointer of segment seg; S4 (EPI_POOL) adds a fourth. By value: taking
// the kernel argument block by reference changes how the compiler loads it.
template <bool S4, typename X>
__device__ __forceinline__ X seg_pick(X a0, X a1, X a2, X a3, int seg) {
  if constexpr (S4) return seg == 0 ? a0 : (seg == 1 ? a1 : (seg == 3 ? a3 : a2));
  else return seg == 0 ? a0 : (seg == 1 ? a1 : a2);
}

// Position-table row of token m (EPI_BIAS_POS), see PosMode.
template <typename P>
__device__ __forceinline__ int pos_row(const P& p, int64_t m) {
  const int t = (int)(m % p.tokens_per_frame);
  const int y = t / p.grid_w, x = t - y * p.grid_w;
  if (p.pos_mode == POS_BUCKET) return max(y - 1, 0) * p.pos_side + max(x - 1, 0);
  if (p.pos_mode == POS_TILE) return (y % p.pos_side) * p.pos_side + (x % p.pos_side);
  return t;
}

// n / d for 0 <= n < 2^22 and d >= 1, from a float reciprocal (the product
// is within one of the quotient there) and one correction.
__device__ __forceinline__ int div_small(int n, int d, float rcp) {
  int q = (int)((float)n * rcp);
  const int r = n - q * d;
  return q + (r >= d ? 1 : 0) - (r < 0 ? 1 : 0);
}

// Head-major placement of token row m (frames of vt_tokens tokens): blk0 =
// (frame * windows + window) * heads, wn = tokens per window, i = the
// token's index in its window. Windows are the frame, or (hm_spatial) the
// win_h x win_w tiles of a grid grid_w wide, each read row-major.
template <typename P>
__device__ __forceinline__ void hm_place(const P& p, int m, int& blk0, int& wn, int& i) {
  const int fb = div_small(m, p.vt_tokens, p.hm_rcp[0]), t = m - fb * p.vt_tokens;
  if (!p.hm_spatial) {
    wn = p.vt_tokens;
    blk0 = fb * p.vt_heads;
    i = t;
    return;
  }
  const int y = div_small(t, p.grid_w, p.hm_rcp[1]), x = t - y * p.grid_w;
  const int wy = div_small(y, p.win_h, p.hm_rcp[2]), wx = div_small(x, p.win_w, p.hm_rcp[3]);
  wn = p.win_h * p.win_w;
  blk0 = ((fb * (p.vt_tokens / wn) + wy * (p.grid_w / p.win_w) + wx)) * p.vt_heads;
  i = (y - wy * p.win_h) * p.win_w + (x - wx * p.win_w);
}

__device__ __forceinline__ float gelu_erf_f(float v) { return gelu_erf_as(v); }
__device__ __forceinline__ float gelu_tanh_f(float v) { return gelu_tanh_fast(v); }

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
      f32x4 v = acc[i][j];
      if (p.ws0 != nullptr) {
        const _Float16* sc = (seg == 0 ? p.ws0 : (seg == 1 ? p.ws1 : p.ws2)) + (n - seg * p.seg_cols);
        v *= f32x4{(float)sc[0], (float)sc[1], (float)sc[2], (float)sc[3]};
      }
      if (EPI != EPI_BIAS_POS || bb != nullptr) v += *reinterpret_cast<const f32x4*>(bb + (n - seg * p.seg_cols));
      if (EPI == EPI_BIAS_POS) {
        if (p.pos_mode != POS_NONE) v += *reinterpret_cast<const f32x4*>(p.pos + (int64_t)pos_row(p, m) * p.N + n);
      } else if (EPI == EPI_BIAS_ROPE) {
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

// ---------------------------------------------------------------------------
// bf16 path for K % 16 == 0, K >= 64: 32x32x16 MFMA, operands staged global -> LDS
// directly (global_load_lds, 16 bytes per lane, no register round trip) in a
// ring of 2-4 stages of 64 K columns, and an epilogue that goes through LDS
// so that every global store is a full 16-byte vector of one output row.
// When K % 64 != 0 (K >= 64) the last K tile is loaded as the last 64
// columns of the rows, overlapping the tile before it, and only its MFMA K
// steps past that overlap run.
//
// LDS layout of a stage: [BM token rows | BN weight rows] x 64 bf16 (128 B
// per row = 8 chunks of 16 B). One load instruction of a wave fills 8 rows
// (1 KB, contiguous); the chunk a lane loads is XOR-swizzled by its row so
// that the 32-row fragment reads of an MFMA operand (one 16-byte chunk per
// lane) spread over all banks.
// ---------------------------------------------------------------------------

__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
__device__ __forceinline__ int lds_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
typedef __attribute__((address_space(3))) void* lds_ptr;

// Buffer descriptor of `bytes` bytes from `base` (range-checked: loads past
// the end return zeros); the operands are wave-uniform, readfirstlane keeps
// the descriptor in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t lds_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int nb = (int)min(max(bytes, (int64_t)0), (int64_t)0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(nb), 0x00020000);
}
// 16 bytes per lane from a buffer into LDS (lane l's at lds + 16 l bytes);
// a function of its own so that host compilation of the kernel templates
// never sees the device-only builtin
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, bf16* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, __builtin_amdgcn_readfirstlane(soff), 0, 0);
}

// Workgroup -> output tile. Workgroups are dealt round-robin to the 8 XCDs
// (each with its own L2): each XCD gets a contiguous range of the logical
// tile order, walked in groups of GM tile rows, so the tiles that run
// together on one XCD share A row panels and W column panels in its L2.
template <int GM>
__device__ __forceinline__ void xcd_tile(int bid, int nwg, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int q = nwg / 8, r = nwg % 8, x = bid % 8, local = bid / 8;
  const int t = x < r ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
  const int per_group = GM * tiles_n;
  const int grp = t / per_group, first_m = grp * GM;
  const int gm = min(GM, tiles_m - first_m);
  const int in = t - grp * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

// Scheduling hint for one K step of the main loop: alternate the step's
// MFMAs with the vector-memory loads of the next tile (NV) and the LDS
// fragment reads of the next K step (ND), so that neither the memory nor the
// LDS queue backs up behind a burst of issues while the matrix core idles.
template <int M, int NM, int NV, int ND>
struct Interleave {
  __device__ __forceinline__ static void go() {
    if constexpr (M < NM) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
      if constexpr (M < NV) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one VMEM
      if constexpr (M < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
      Interleave<M + 1, NM, NV, ND>::go();
    }
  }
};

// Wait until at most `ahead` tiles' loads (LPW per wave each) are still in
// flight: s_waitcnt takes an immediate, so one branch per possible count.
template <int A, int LPW>
struct WaitAhead {
  __device__ __forceinline__ static void go(int ahead) {
    if constexpr (A == 0) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else {
      if (ahead >= A)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(A * LPW));
      else
        WaitAhead<A - 1, LPW>::go(ahead);
    }
  }
};

// KW: the waves split K instead of the tile. Each of the four waves owns
// one of a K tile's four MFMA K steps for the whole BM x BN tile, and the
// four partial tiles are summed in LDS before the epilogue. For grids of
// about one workgroup per CU, where one wave per SIMD with one MFMA per K
// step spends most of each step waiting on its LDS fragment reads.
// The RoPE epilogue of the two-workgroups-per-CU tiles needs the register
// budget stated explicitly to stay at two waves per SIMD.
template <int BM, int BN, int WAVES_M, int WAVES_N, int ST, int EPI, bool KT, bool KW>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) __attribute__((
    amdgpu_waves_per_eu(EPI == EPI_BIAS_ROPE && (BM + BN) * 64 * ST * 2 <= 81920 ? 2 : 1))) void gemm_mfma32_kernel(
    typename std::conditional<EPI == EPI_POOL, GemmPoolParams<bf16>, GemmParams<bf16>>::type p) {
  constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  constexpr int BK = 64;
  static_assert(ST >= 2, "at least two LDS stages");
  static_assert(!KW || NW == BK / 16, "KW: one wave per MFMA K step");
  constexpr int TM = KW ? BM / 32 : BM / WAVES_M / 32, TN = KW ? BN / 32 : BN / WAVES_N / 32;  // 32x32 tiles per wave
  constexpr int STAGE = (BM + BN) * BK;                          // bf16 elements
  constexpr int LPW = (BM + BN) / (8 * NW);                      // load instructions per wave per stage
  static_assert((BM + BN) % (8 * NW) == 0, "rows must split evenly over the waves");
  static_assert((ST - 2) * LPW <= 63, "vmcnt counts at most 63 loads");
  constexpr int CROW = BN + 4;  // fp32 row pitch of the epilogue staging tile
  // KW stages NW partial tiles (fp32) in the epilogue
  constexpr int SM = KW && NW * BM * CROW * 2 > ST * STAGE ? NW * BM * CROW * 2 : ST * STAGE;
  __shared__ __attribute__((aligned(1024))) bf16 sm[SM];

  // EPI_POOL: a tile is PB pooled rows; its BM A rows are the four quarter
  // rows of each (local row r: quarter r / PB, pooled row m0 + r % PB)
  constexpr bool POOL = EPI == EPI_POOL;
  constexpr int PB = BM / 4;
  const bf16* W3 = nullptr;
  const float* b3 = nullptr;
  const _Float16* ws3 = nullptr;
  if constexpr (POOL) {
    W3 = p.W3;
    b3 = p.b3;
    ws3 = p.ws3;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_n = (p.N + BN - 1) / BN, tiles_m = POOL ? (p.M / 4 + PB - 1) / PB : (p.M + BM - 1) / BM;

  // Warm the memory-side cache with the whole weight matrix before the first
  // tile: one 4-byte read per 128-byte line, dealt to the threads of the
  // first workgroups. In a chain of blocks each block's weights were last
  // read many blocks ago and sit in HBM; without this every K step of every
  // tile waits on an HBM miss for its W panel, with it the misses overlap
  // the prologue and later W reads hit the Infinity Cache. The value is
  // consumed only by a store that never happens (M >= 1 always).
  uint32_t touch = 0;
  {
    const int lines_per_row = KT ? (p.K + 63) / 64 : p.K / 64;  // kl * 64 < K since K % 16 == 0
    const int64_t lines = (int64_t)p.N * lines_per_row;
    for (int64_t g = (int64_t)blockIdx.x * NT + tid; g < lines; g += (int64_t)gridDim.x * NT) {
      const int n = (int)(g / lines_per_row), kl = (int)(g - (int64_t)n * lines_per_row);
      const int seg = n / p.seg_cols;
      const bf16* base = seg_pick<POOL>(p.W0, p.W1, p.W2, W3, seg);
      touch ^= *reinterpret_cast<const uint32_t*>(base + (int64_t)(n - seg * p.seg_cols) * p.K + kl * 64);
    }
  }

  int tmi, tni;
  xcd_tile<8>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tmi, tni);
  const int m0 = tmi * (POOL ? PB : BM), n0 = tni * BN;

  // Operand tiles by buffer loads straight into LDS. Load j of wave w
  // fills LDS row group L = j * NW + w (rows 8L .. 8L+7, 1 KB): loads
  // j < LA are A rows for every wave, the rest W rows, all of one weight
  // segment (BM and seg_cols are multiples of 8). So every load's buffer
  // descriptor is known at compile time: one for A (from the tile's first
  // row; POOL: from A) and one per W load (from its group's first row to
  // the segment's end). The per-lane byte offset is fixed over K and the K
  // tile is a scalar offset: no per-load vector arithmetic. Rows past M or
  // N read zeros (never stored).
  const int waveu = __builtin_amdgcn_readfirstlane(wave);
  constexpr int LA = BM / 8 / NW;
  static_assert((BM / 8) % NW == 0, "A row groups must split evenly over the waves");
  const __amdgpu_buffer_rsrc_t rsA = POOL ? lds_rsrc(p.A, (int64_t)p.M * p.lda * 2)
                                          : lds_rsrc(p.A + (int64_t)m0 * p.lda, (int64_t)(p.M - m0) * p.lda * 2);
  __amdgpu_buffer_rsrc_t rsW[LPW - LA];
  uint32_t voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int row0 = (j * NW + waveu) * 8, row = row0 + lane / 8;
    const int chunk = (lane & 7) ^ lds_swz(row);
    if (j < LA) {
      if constexpr (POOL) {
        const int q4 = p.tokens_per_frame / 4, pr = min(m0 + row % PB, p.M / 4 - 1);
        const int m = (pr / q4) * p.tokens_per_frame + (row / PB) * q4 + pr % q4;
        voff[j] = (uint32_t)(((int64_t)m * p.lda + chunk * 8) * 2);
      } else {
        voff[j] = (uint32_t)(((int64_t)row * p.lda + chunk * 8) * 2);
      }
    } else {
      const int nf = min(n0 + row0 - BM, p.N - 1);  // the group's first weight row
      const int seg = nf / p.seg_cols, n_in_seg = nf - seg * p.seg_cols;
      const bf16* base = seg_pick<POOL>(p.W0, p.W1, p.W2, W3, seg) + (int64_t)n_in_seg * p.K;
      const int rows_left = min(p.seg_cols, p.N - seg * p.seg_cols) - n_in_seg;
      rsW[j - LA] = lds_rsrc(base, (int64_t)rows_left * p.K * 2);
      voff[j] = (uint32_t)(((int64_t)(row - row0) * p.K + chunk * 8) * 2);
    }
  }
  // KT (K % 64 != 0, K >= 64): the partial last tile is read as the last
  // 64 columns, K-64 .. K-1; its new columns are its last kst K steps
  const int nk = KT ? (p.K + BK - 1) / BK : p.K / BK;  // K tiles
  const int nkf = KT ? p.K / BK : nk;  // full K tiles; tile nkf (if any) is partial
  const int kst = (p.K - nkf * BK) / 16;
  const int klast = p.K - BK;
  // load j of tile kt (LPW per wave per tile)
  auto load = [&](int j, int kt) {
    buf_load_lds16(j < LA ? rsA : rsW[j < LA ? 0 : j - LA], sm + (kt % ST) * STAGE + (j * NW + waveu) * 512, voff[j],
                   (KT ? min(kt * BK, klast) : kt * BK) * 2);
  };
  const int wm = KW ? 0 : wave / WAVES_N, wn = KW ? 0 : wave % WAVES_N;
  const int fr = lane & 31, g = lane >> 5;
  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x16{};
  u32x4 af[2][TN], bfr[2][TM];
  auto frags = [&](int buf, int stage, int ks) {
    const bf16* xs = sm + stage * STAGE;
    const bf16* ws = xs + BM * BK;
    const int chunk = ks * 2 + g;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int row = wn * TN * 32 + i * 32 + fr;
      af[buf][i] = ld16(ws + row * 64 + (chunk ^ lds_swz(row)) * 8);
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int row = wm * TM * 32 + j * 32 + fr;
      bfr[buf][j] = ld16(xs + row * 64 + (chunk ^ lds_swz(row)) * 8);
    }
  };

  constexpr int KS = BK / 16;              // MFMA K steps per tile
  constexpr int LPK = (LPW + 1) / 2;       // tile kt+ST-1's loads per K step, over the first two steps
  // tiles 0 .. ST-2 in flight before the loop
  for (int t = 0; t < ST - 1 && t < nk; ++t)
#pragma unroll
    for (int j = 0; j < LPW; ++j) load(j, t);
  for (int kt = 0; kt < nkf; ++kt) {
    // this wave's loads of tile kt have landed (the later tiles' loads, issued
    // after them, may still be in flight); after the barrier every wave's
    // have, and every wave is done reading the stage refilled next
    WaitAhead<ST - 2, LPW>::go(min(ST - 2, nk - 1 - kt));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const bool more = kt + ST - 1 < nk;
    const int stage = kt % ST;
    if constexpr (KW) {
      frags(0, stage, wave);
      if (more) {
#pragma unroll
        for (int j = 0; j < LPW; ++j) load(j, kt + ST - 1);
      }
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[0][i]),
                                                             __builtin_bit_cast(bf16x8, bfr[0][j]), acc[i][j], 0, 0, 0);
      continue;
    }
    frags(0, stage, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (more) {
#pragma unroll
        for (int j = 0; j < LPW; ++j)
          if (j / LPK == ks) load(j, kt + ST - 1);
      }
      if (ks + 1 < KS) frags((ks + 1) & 1, stage, ks + 1);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[ks & 1][i]),
                                                             __builtin_bit_cast(bf16x8, bfr[ks & 1][j]), acc[i][j], 0, 0, 0);
      if (ks + 1 < KS)
        Interleave<0, TN * TM, LPK, TN + TM>::go();
      else
        Interleave<0, TN * TM, LPK, 0>::go();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (KT && kst > 0) {
    // the partial tile: its loads were the last issued; K steps KS-kst .. KS-1
    // hold columns nkf*64 .. K-1
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int stage = nkf % ST, ks0 = KS - kst;
    if (KW && wave >= ks0) {
      frags(0, stage, wave);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[0][i]),
                                                             __builtin_bit_cast(bf16x8, bfr[0][j]), acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int ks = 1; ks < (KW ? 1 : KS); ++ks) {
      if (ks >= ks0) {
        if (ks == ks0) frags(ks & 1, stage, ks);
        if (ks + 1 < KS) frags((ks + 1) & 1, stage, ks + 1);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[ks & 1][i]),
                                                               __builtin_bit_cast(bf16x8, bfr[ks & 1][j]), acc[i][j], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: accumulators -> LDS (fp32, row-major) -> 8 columns per
  // thread with bias / RoPE / GELU / residual -> one 16-byte store per row
  // chunk. Lane (fr, g) of 32x32 tile (i, j) holds row j*32+fr, columns
  // i*32 + 8q + 4g + e in register 4q + e.
  //
  // Every global load of the epilogue is issued ahead of the stores: the
  // bias once per tile right after the main loop, the residual / RoPE /
  // position rows of a pass before that pass's staging. A load placed
  // between the stores of the chunk loops would wait out a full memory
  // round trip each time (the compiler cannot move a load above a store
  // that may alias it, and the wait for a load also waits for every store
  // issued before it).
  constexpr int PR0 = (ST * STAGE * 2) / (CROW * 4);
  constexpr int PR = KW || PR0 >= BM ? BM : (PR0 >= BM / 2 ? BM / 2 : BM / 4);
  static_assert(!POOL || PR == BM, "EPI_POOL stages the whole tile at once");
  static_assert(PR >= BM / 4 && PR % 32 == 0, "LDS too small for the epilogue");
  float* cs = reinterpret_cast<float*>(sm);
  float* cw = cs + (KW ? wave * BM * CROW : 0);  // this wave's staging tile
  constexpr int WROWS = BM / WAVES_M;
  constexpr int G8 = BN / 8;
  // per-column weight scales of this lane's columns (4 float16 per (i, q)),
  // loaded once per tile; columns past N take the last valid scale and are
  // never stored
  u32x2 scl[TN][4];
  if (p.ws0 != nullptr) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = min(n0 + wn * TN * 32 + i * 32 + 8 * q + 4 * g, p.N - 4);
        const int seg = n / p.seg_cols;
        scl[i][q] = *reinterpret_cast<const u32x2*>(seg_pick<POOL>(p.ws0, p.ws1, p.ws2, ws3, seg) + (n - seg * p.seg_cols));
      }
  }
  // Chunk k of a pass (e = tid + k NT) covers row e / G8 and columns
  // (e % G8) * 8 .. + 7: its columns repeat with period DC in k, so a
  // thread needs the bias of DC column groups only (1 for BN = 64, 128, 256
  // with NT = 256, 256, 512; 3 for BN = 192). Likewise the V^T copy below
  // (one column cc = e % BN per iteration) with period DCV.
  constexpr int CH = (PR * G8 + NT - 1) / NT;
  constexpr bool CH_EVEN = (PR * G8) % NT == 0;
  constexpr int DC = G8 / std::gcd(G8, NT % G8);
  constexpr bool VT = EPI == EPI_BIAS || EPI == EPI_BIAS_ROPE;
  constexpr int CHV = ((PR / 8) * BN + NT - 1) / NT;
  constexpr bool CHV_EVEN = ((PR / 8) * BN) % NT == 0;
  constexpr int DCV = BN / std::gcd(BN, NT % BN);
  static_assert(!POOL || DC == 1, "EPI_POOL: one column group per thread");
  f32x4 bsv[DC][2];
  float bvt[VT ? DCV : 1];
#pragma unroll
  for (int k = 0; k < DC; ++k) {
    // columns past N take the last valid group's bias (never stored)
    const int n = min(n0 + ((tid + k * NT) % G8) * 8, p.N - 8);
    const int seg = n / p.seg_cols;
    const float* bp = seg_pick<POOL>(p.b0, p.b1, p.b2, b3, seg);
    // no bias (EPI_BIAS_POS may have none): eight zeros; a load either way,
    // without a branch around it
    const float* bq = bp != nullptr ? bp + (n - seg * p.seg_cols) : kZeros8;
    bsv[k][0] = *reinterpret_cast<const f32x4*>(bq);
    bsv[k][1] = *reinterpret_cast<const f32x4*>(bq + 4);
  }
  if constexpr (VT) {
#pragma unroll
    for (int k = 0; k < DCV; ++k) {
      const int n = min(n0 + (tid + k * NT) % BN, p.N - 1);
      const int seg = n / p.seg_cols;
      const float* bp = seg_pick<false>(p.b0, p.b1, p.b2, b3, seg);
      bvt[k] = *(bp != nullptr ? bp + (n - seg * p.seg_cols) : kZeros8);
    }
  }
  // RoPE: the table column of each column group (pairs d/2 .. d/2+3 of the
  // head dimension d; a multiple of 8), and the row part below per chunk
  int ropec[EPI == EPI_BIAS_ROPE ? DC : 1];
  if constexpr (EPI == EPI_BIAS_ROPE) {
#pragma unroll
    for (int k = 0; k < DC; ++k) {
      const int n = min(n0 + ((tid + k * NT) % G8) * 8, p.N - 8);
      ropec[k] = p.rope_cols > 0 ? (n % (p.rope_cols / 2)) % p.head_dim : 0;
    }
  }
  u32x4 resv[EPI == EPI_BIAS_RES ? CH : 1];
  f32x4 tab[EPI == EPI_BIAS_ROPE || EPI == EPI_BIAS_POS ? CH : 1][2];
  // RoPE table row of token row m: the token's index in its frame, or
  // (spatial windows) in its window; divisions by float reciprocals
  // (m < 2^22)
  auto rope_row = [&](int m) {
    const int t = m - div_small(m, p.tokens_per_frame, p.hm_rcp[4]) * p.tokens_per_frame;
    if (p.rope_mode != 1) return t;
    const int yy = div_small(t, p.grid_w, p.hm_rcp[1]), xx = t - yy * p.grid_w;
    return (yy - div_small(yy, p.win_h, p.hm_rcp[2]) * p.win_h) * p.win_w + (xx - div_small(xx, p.win_w, p.hm_rcp[3]) * p.win_w);
  };
  // Per-row placement of the tile's rows -- the RoPE table row's float
  // offset, and the head-major q / k and V^T element offsets -- computed
  // once per tile into LDS past the staging area (after the first barrier,
  // when the main loop is done with LDS), so that no chunk of the store
  // loops repeats the index divisions. Where that space does not exist
  // (the K-split form) each chunk computes its own.
  constexpr int RT_OFF = (PR * CROW * 4 * (KW ? NW : 1) + 15) / 16 * 16;  // bytes into sm
  constexpr bool RT = (EPI == EPI_BIAS || EPI == EPI_BIAS_ROPE) && !POOL && RT_OFF + BM * 12 <= SM * 2;
  int* rt = reinterpret_cast<int*>(reinterpret_cast<char*>(sm) + RT_OFF);
  const int wn_u = p.hm_spatial ? p.win_h * p.win_w : p.vt_tokens;  // tokens per head-major window
#pragma unroll
  for (int pass = 0; pass < BM / PR; ++pass) {
    // this pass's residual / position / RoPE rows: chunks 0 .. CH0-1 here,
    // the rest (8 registers per chunk for the tables) at chunk CH0 of the
    // store loop, which keeps two workgroups per CU within the register
    // file. Loaded unconditionally from clamped addresses (rows past M,
    // columns past N: never stored), so that the loads need no branches.
    constexpr bool FETCH = !POOL && (EPI == EPI_BIAS_RES || EPI == EPI_BIAS_ROPE || EPI == EPI_BIAS_POS);
    constexpr int CH0 = EPI == EPI_BIAS_RES ? CH : (CH + 1) / 2;
    const bool want = EPI == EPI_BIAS_RES || (EPI == EPI_BIAS_POS ? p.pos_mode != POS_NONE : p.rope_cols > 0);
    auto fetch = [&](int k) {
      const int e = min(tid + k * NT, PR * G8 - 1);
      const int r = e / G8, c8 = (e - r * G8) * 8;
      const int m = min(m0 + pass * PR + r, p.M - 1), n = min(n0 + c8, p.N - 8);
      if constexpr (EPI == EPI_BIAS_RES) {
        resv[k] = ld16(p.res + (int64_t)m * p.ldres + n);
      } else if constexpr (EPI == EPI_BIAS_POS) {
        const float* pp = p.pos + (int64_t)pos_row(p, m) * p.N + n;
        tab[k][0] = *reinterpret_cast<const f32x4*>(pp);
        tab[k][1] = *reinterpret_cast<const f32x4*>(pp + 4);
      } else if constexpr (EPI == EPI_BIAS_ROPE) {
        // pairs ropec/2 .. +3 of the row (columns past rope_cols read some
        // valid entry, unused)
        const int row_off = RT ? rt[3 * min(pass * PR + r, BM - 1)] : rope_row(m) * p.head_dim;
        const float* cs4 = p.rope + (int64_t)row_off + ropec[k % DC];
        tab[k][0] = *reinterpret_cast<const f32x4*>(cs4);
        tab[k][1] = *reinterpret_cast<const f32x4*>(cs4 + 4);
      }
    };
    // RoPE with the row table: pass 0's first chunks once the table is
    // written; all of a pass's chunks up front where they are few
    constexpr bool RT_ROPE = RT && EPI == EPI_BIAS_ROPE;
    constexpr int F0 = RT_ROPE && CH <= 4 ? CH : CH0;
    if (FETCH && want && (!RT_ROPE || pass > 0)) {
#pragma unroll
      for (int k = 0; k < F0; ++k) fetch(k);
    }
    __syncthreads();
    if (RT && pass == 0) {
      for (int r = tid; r < BM; r += NT) {
        const int m = min(m0 + r, p.M - 1);
        if (EPI == EPI_BIAS_ROPE && p.rope_cols > 0) rt[3 * r] = rope_row(m) * p.head_dim;
        if (p.hm_q != nullptr) {
          int blk0, wn, i;
          hm_place(p, m, blk0, wn, i);
          rt[3 * r + 1] = (blk0 * wn + i) * 64;  // q / k: + (head * wn) * 64 + d
          rt[3 * r + 2] = blk0 * wn * 64 + i;    // V^T: + (head * 64 + d) * wn
        }
      }
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int row = wm * WROWS + j * 32 + fr;
      if (row >= pass * PR && row < (pass + 1) * PR) {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = wn * TN * 32 + i * 32 + 8 * q + 4 * g;
            f32x4 a4 = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            if (p.ws0 != nullptr) {
              const u32x2 h = scl[i][q];
              a4 *= f32x4{(float)__builtin_bit_cast(_Float16, (uint16_t)(h[0] & 0xFFFF)),
                          (float)__builtin_bit_cast(_Float16, (uint16_t)(h[0] >> 16)),
                          (float)__builtin_bit_cast(_Float16, (uint16_t)(h[1] & 0xFFFF)),
                          (float)__builtin_bit_cast(_Float16, (uint16_t)(h[1] >> 16))};
            }
            *reinterpret_cast<f32x4*>(cw + (row - pass * PR) * CROW + col) = a4;
          }
      }
    }
    __syncthreads();
    if constexpr (KW) {
      // sum the NW partial tiles into the first
      for (int e = tid; e < BM * (BN / 4); e += NT) {
        const int r = e / (BN / 4), c4 = (e - r * (BN / 4)) * 4;
        f32x4 v = *reinterpret_cast<const f32x4*>(cs + r * CROW + c4);
#pragma unroll
        for (int w = 1; w < NW; ++w) v += *reinterpret_cast<const f32x4*>(cs + w * BM * CROW + r * CROW + c4);
        *reinterpret_cast<f32x4*>(cs + r * CROW + c4) = v;
      }
      __syncthreads();
    }
    if (FETCH && want && RT_ROPE && pass == 0) {
#pragma unroll
      for (int k = 0; k < F0; ++k) fetch(k);
    }
    if ((EPI == EPI_BIAS || EPI == EPI_BIAS_ROPE) && p.vt != nullptr && n0 + BN > p.vt_col0) {
      // transposed copy of the V columns: one column x 8 consecutive token
      // rows per thread (a 16-byte run of one V^T row); rows are within one
      // frame since vt_tokens % 8 == 0
#pragma unroll
      for (int kv = 0; kv < CHV; ++kv) {
        const int e = tid + kv * NT;
        if (!CHV_EVEN && e >= (PR / 8) * BN) break;
        const int cc = e % BN, rg = e / BN;
        const int m = m0 + pass * PR + rg * 8, n = n0 + cc;
        if (m >= p.M || n >= p.N || n < p.vt_col0) continue;
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = cs[(rg * 8 + k) * CROW + cc] + bvt[kv % DCV];
        const int vv = n - p.vt_col0;
        if (p.hm_q != nullptr) {
          // [frame, window, head, d, i] (head_dim 64): the 8 rows are
          // consecutive tokens of one window row (win_w % 8 == 0), so
          // consecutive i
          if constexpr (RT) {
            st16(p.vt + rt[3 * (pass * PR + rg * 8) + 2] + vv * wn_u, pack16<bf16>(v));
          } else {
            int blk0, wn, i;
            hm_place(p, m, blk0, wn, i);
            st16(p.vt + ((blk0 + (vv >> 6)) * 64 + (vv & 63)) * wn + i, pack16<bf16>(v));
          }
        } else {
          const int hh = vv / p.vt_hd, d = vv - hh * p.vt_hd;
          const int fb = m / p.vt_tokens, t = m - fb * p.vt_tokens;
          st16(p.vt + (((int64_t)fb * p.vt_heads + hh) * p.vt_hd + d) * p.vt_tokens + t, pack16<bf16>(v));
        }
      }
    }
    if constexpr (POOL) {
      const int q4 = p.tokens_per_frame / 4, mp = p.M / 4;
      // columns < pool_col0: every row, back at its own token
      for (int e = tid; e < BM * G8; e += NT) {
        const int r = e / G8, c8 = (e - r * G8) * 8;
        const int n = n0 + c8, pr = m0 + r % PB;
        if (n >= p.pool_col0 || n >= p.N || pr >= mp) continue;
        const int64_t m = (int64_t)(pr / q4) * p.tokens_per_frame + (r / PB) * q4 + pr % q4;
        float v[8];
        *reinterpret_cast<f32x4*>(v) = *reinterpret_cast<const f32x4*>(cs + r * CROW + c8) + bsv[0][0];
        *reinterpret_cast<f32x4*>(v + 4) = *reinterpret_cast<const f32x4*>(cs + r * CROW + c8 + 4) + bsv[0][1];
        st16(p.C + m * p.ldc + n, pack16<bf16>(v));
      }
      // columns >= pool_col0: the max over the four quarter rows, then the bias
      for (int e = tid; e < PB * G8; e += NT) {
        const int i = e / G8, c8 = (e - i * G8) * 8;
        const int n = n0 + c8, pr = m0 + i;
        if (n < p.pool_col0 || n >= p.N || pr >= mp) continue;
        f32x4 lo = *reinterpret_cast<const f32x4*>(cs + i * CROW + c8);
        f32x4 hi = *reinterpret_cast<const f32x4*>(cs + i * CROW + c8 + 4);
#pragma unroll
        for (int q = 1; q < 4; ++q) {
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(cs + (q * PB + i) * CROW + c8);
          const f32x4 h2 = *reinterpret_cast<const f32x4*>(cs + (q * PB + i) * CROW + c8 + 4);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            lo[t] = fmaxf(lo[t], l2[t]);
            hi[t] = fmaxf(hi[t], h2[t]);
          }
        }
        float v[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[t] = lo[t] + bsv[0][0][t];
          v[4 + t] = hi[t] + bsv[0][1][t];
        }
        st16(p.pool_out + (int64_t)pr * p.ld_pool + (n - p.pool_col0), pack16<bf16>(v));
      }
      continue;
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      if (FETCH && F0 < CH && k == F0 && want) {
#pragma unroll
        for (int k2 = F0; k2 < CH; ++k2) fetch(k2);
      }
      const int e = tid + k * NT;
      if (!CH_EVEN && e >= PR * G8) break;
      const int r = e / G8, c8 = (e - r * G8) * 8;
      const int m = m0 + pass * PR + r, n = n0 + c8;
      if (m >= p.M || n >= p.N) continue;
      if (p.vt_only && n >= p.vt_col0) continue;
      const bool to_hm = (EPI == EPI_BIAS || EPI == EPI_BIAS_ROPE) && p.hm_q != nullptr && n < p.vt_col0;
      float v[8];
      *reinterpret_cast<f32x4*>(v) = *reinterpret_cast<const f32x4*>(cs + r * CROW + c8) + bsv[k % DC][0];
      *reinterpret_cast<f32x4*>(v + 4) = *reinterpret_cast<const f32x4*>(cs + r * CROW + c8 + 4) + bsv[k % DC][1];
      if (EPI == EPI_BIAS_POS) {
        if (p.pos_mode != POS_NONE) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v[t] += tab[k][0][t];
            v[4 + t] += tab[k][1][t];
          }
        }
      } else if (EPI == EPI_BIAS_ROPE) {
        if (n < p.rope_cols) {
          const float cc[8] = {tab[k][0][0], tab[k][0][1], tab[k][0][2], tab[k][0][3],
                               tab[k][1][0], tab[k][1][1], tab[k][1][2], tab[k][1][3]};
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            const float a0 = v[2 * pr], a1 = v[2 * pr + 1], co = cc[2 * pr], si = cc[2 * pr + 1];
            v[2 * pr] = a0 * co - a1 * si;
            v[2 * pr + 1] = a1 * co + a0 * si;
          }
        }
      } else if (EPI == EPI_GELU_ERF) {
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = gelu_erf_f(v[t]);
      } else if (EPI == EPI_GELU_TANH) {
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = gelu_tanh_f(v[t]);
      } else if (EPI == EPI_BIAS_RES) {
        if (p.branch) st16(p.branch + (int64_t)m * p.ldbranch + n, pack16<bf16>(v));
        float rv[8];
        unpack16<bf16>(resv[k], rv);
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] += rv[t];
      }
      if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_ROPE) {
        if (to_hm) {
          // q (scaled) or k, 8 consecutive d of one head, to [frame, window, head, i, 64]
          // head_dim is 64 here
          const int dq = p.vt_col0 / 2, isk = n >= dq ? 1 : 0, nn = n - isk * dq;
          const int hh = nn >> 6, d = nn & 63;
          int off;
          if constexpr (RT) {
            off = rt[3 * (pass * PR + r) + 1] + hh * wn_u * 64 + d;
          } else {
            int blk0, wn, i;
            hm_place(p, m, blk0, wn, i);
            off = ((blk0 + hh) * wn + i) * 64 + d;
          }
          float hv[8];
          const float sc = isk ? 1.f : p.hm_qscale;
#pragma unroll
          for (int t2 = 0; t2 < 8; ++t2) hv[t2] = v[t2] * sc;
          st16((isk ? p.hm_k : p.hm_q) + off, pack16<bf16>(hv));
          if (p.vt_only) continue;
        }
      }
      st16(p.C + (int64_t)m * p.ldc + n, pack16<bf16>(v));
    }
  }
  if (p.M <= 0 && touch == 0x5EEDu) p.C[0] = bf16(0.f);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int ST = 2, bool KT = false, bool KW = false>
static hipError_t gemm32_go(const GemmParams<bf16>& p, int epi, hipStream_t s, StageEvents ev) {
  const int64_t tiles = (int64_t)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  dim3 grid((unsigned)tiles), block(64 * WAVES_M * WAVES_N);
  switch (epi) {
    case EPI_BIAS: hipExtLaunchKernelGGL((gemm_mfma32_kernel<BM, BN, WAVES_M, WAVES_N, ST, EPI_BIAS, KT, KW>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_BIAS_ROPE: hipExtLaunchKernelGGL((gemm_mfma32_kernel<BM, BN, WAVES_M, WAVES_N, ST, EPI_BIAS_ROPE, KT, KW>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_GELU_ERF: hipExtLaunchKernelGGL((gemm_mfma32_kernel<BM, BN, WAVES_M, WAVES_N, ST, EPI_GELU_ERF, KT, KW>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_GELU_TANH: hipExtLaunchKernelGGL((gemm_mfma32_kernel<BM, BN, WAVES_M, WAVES_N, ST, EPI_GELU_TANH, KT, KW>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_BIAS_POS: hipExtLaunchKernelGGL((gemm_mfma32_kernel<BM, BN, WAVES_M, WAVES_N, ST, EPI_BIAS_POS, KT, KW>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    default: hipExtLaunchKernelGGL((gemm_mfma32_kernel<BM, BN, WAVES_M, WAVES_N, ST, EPI_BIAS_RES, KT, KW>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
  }
  return hipGetLastError();
}

// EPI_POOL: 64x64 tiles of 16 pooled rows (64 A rows)
template <int ST, bool KT>
static hipError_t gemm32_pool_go(const GemmPoolParams<bf16>& p, hipStream_t s, StageEvents ev) {
  const int64_t tiles = (int64_t)((p.M / 4 + 15) / 16) * ((p.N + 63) / 64);
  hipExtLaunchKernelGGL((gemm_mfma32_kernel<64, 64, 2, 2, ST, EPI_POOL, KT, false>), dim3((unsigned)tiles), dim3(256),
                        0, s, ev.start, ev.stop, 0, p);
  return hipGetLastError();
}

template <typename T>
static GemmParams<T> make_params(const GemmArgs& a) {
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
  p.vt = (T*)a.vt;
  p.vt_col0 = a.vt ? a.vt_col0 : a.N;
  p.vt_tokens = a.vt_tokens;
  p.vt_heads = a.vt_heads;
  p.vt_hd = a.vt_hd;
  p.vt_only = a.vt != nullptr && a.vt_only;
  p.hm_q = (T*)a.hm_q;
  p.hm_k = (T*)a.hm_k;
  p.hm_qscale = a.hm_qscale;
  p.hm_spatial = a.hm_spatial;
  p.hm_rcp[0] = 1.0f / (float)(a.vt_tokens > 0 ? a.vt_tokens : 1);
  p.hm_rcp[1] = 1.0f / (float)(a.grid_w > 0 ? a.grid_w : 1);
  p.hm_rcp[2] = 1.0f / (float)(a.win_h > 0 ? a.win_h : 1);
  p.hm_rcp[3] = 1.0f / (float)(a.win_w > 0 ? a.win_w : 1);
  p.hm_rcp[4] = 1.0f / (float)(a.tokens_per_frame > 0 ? a.tokens_per_frame : 1);
  p.ws0 = (const _Float16*)a.wscale[0];
  p.ws1 = (const _Float16*)(a.wscale[1] ? a.wscale[1] : a.wscale[0]);
  p.ws2 = (const _Float16*)(a.wscale[2] ? a.wscale[2] : a.wscale[0]);
  p.pos = a.pos;
  p.pos_mode = a.pos ? a.pos_mode : POS_NONE;
  p.pos_side = a.pos_side > 0 ? a.pos_side : 1;
  return p;
}

template <typename T, int BM, int BN, int WTM, int WTN>
static hipError_t gemm_go(const GemmArgs& a, hipStream_t s, StageEvents ev) {
  const GemmParams<T> p = make_params<T>(a);
  const int64_t tiles = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  dim3 grid((unsigned)tiles), block(256);
  switch (a.epi) {
    case EPI_BIAS: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_BIAS>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_BIAS_ROPE: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_BIAS_ROPE>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_GELU_ERF: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_GELU_ERF>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_GELU_TANH: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_GELU_TANH>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    case EPI_BIAS_POS: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_BIAS_POS>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
    default: hipExtLaunchKernelGGL((gemm_kernel<T, BM, BN, WTM, WTN, EPI_BIAS_RES>), grid, block, 0, s, ev.start, ev.stop, 0, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, DType dt, hipStream_t s, StageEvents ev) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const bool mfma32 = gemm_uses_mfma(dt, a.K, a.lda);
  if (a.vt && (!mfma32 || (a.epi != EPI_BIAS && a.epi != EPI_BIAS_ROPE) || a.M % 8 || a.vt_tokens <= 0 ||
               a.vt_tokens % 8 || a.vt_col0 % 8 || a.vt_hd <= 0 || (a.N - a.vt_col0) != a.vt_heads * a.vt_hd))
    return hipErrorInvalidValue;
  // RoPE rows and head-major placement divide row indices by float reciprocals
  if (a.epi == EPI_BIAS_ROPE && a.M >= (1 << 22)) return hipErrorInvalidValue;
  if (a.hm_q && (!a.vt || !a.hm_k || a.vt_hd != 64 || a.vt_col0 != 2 * a.vt_heads * 64 || a.M >= (1 << 22) ||
                 (int64_t)a.M * a.vt_heads * 64 >= (1LL << 31) ||
                 (a.hm_spatial && (a.win_w % 8 || a.grid_w % a.win_w || a.vt_tokens % (a.win_h * a.win_w)))))
    return hipErrorInvalidValue;
  // the pooled form addresses A's rows by 32-bit byte offsets from its start
  if (a.epi == EPI_POOL && (int64_t)a.M * a.lda * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  if (a.epi == EPI_POOL) {
    const int T = a.tokens_per_frame;
    if (!mfma32 || a.vt || T <= 0 || T % 4 || a.M % T || a.pool_col0 % 8 || a.pool_col0 > a.N || !a.pool_out)
      return hipErrorInvalidValue;
    GemmPoolParams<bf16> p;
    static_cast<GemmParams<bf16>&>(p) = make_params<bf16>(a);
    p.W3 = (const bf16*)(a.W[3] ? a.W[3] : a.W[0]);
    p.b3 = a.bias[3] ? a.bias[3] : a.bias[0];
    p.ws3 = (const _Float16*)(a.wscale[3] ? a.wscale[3] : a.wscale[0]);
    p.pool_out = (bf16*)a.pool_out;
    p.ld_pool = a.ld_pool;
    p.pool_col0 = a.pool_col0;
    const int64_t tiles = (int64_t)((a.M / 4 + 15) / 16) * ((a.N + 63) / 64);
    if (a.K % 64) return tiles < 512 ? gemm32_pool_go<4, true>(p, s, ev) : gemm32_pool_go<2, true>(p, s, ev);
    return tiles < 512 ? gemm32_pool_go<4, false>(p, s, ev) : gemm32_pool_go<2, false>(p, s, ev);
  }
  if (dt == DType::F32) return gemm_go<float, 64, 64, 2, 2>(a, s, ev);
  if (mfma32) {
    // One full wave of 256x256 tiles fills the 256 CUs. Otherwise two
    // workgroups per CU: 128x128 tiles, or for products of >= 9e9 FLOP
    // 128x192 / 192x128 tiles where 192 divides N / M exactly (fewer, larger
    // tiles with no ragged edge; 3-8 % faster on the SigLIP and SAM3 MLP and
    // qkv shapes; since the epilogue issues its loads ahead of its stores
    // also on the out-projections: SAM3 5184x1024x1024 22.1 -> 20.5 us,
    // SigLIP 8192x768x768 18.6 -> 18.2 us)
    const GemmParams<bf16> p = make_params<bf16>(a);
    const int64_t t128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
    if (a.K % 64 != 0) {
      // a partial last K tile (the Hiera widths 112 and 224): only 2-4 K
      // tiles, so per-tile prologue and epilogue dominate and 64x64 tiles
      // (more of them in flight) beat 128x128 (c3a qkv 16384x672x112:
      // 7.7 us against 10.2); four stages where the grid is small
      if (t128 < 192) return gemm32_go<64, 64, 2, 2, 4, true>(p, a.epi, s, ev);
      return gemm32_go<64, 64, 2, 2, 2, true>(p, a.epi, s, ev);
    }
    const int64_t t256 = (int64_t)((a.M + 255) / 256) * ((a.N + 255) / 256);
    if (t256 >= 224 && t256 <= 256) return gemm32_go<256, 256, 2, 4>(p, a.epi, s, ev);
    if (2.0 * a.M * a.N * a.K >= 9e9) {
      // at most one workgroup per CU (e.g. fc2, N = 768 or 1024): four LDS
      // stages (all 160 KB), since no second workgroup hides load latency
      // (13 % faster on the SAM3 fc2, 8 % on SigLIP's), and eight waves of
      // 96x32 / 32x96 so that each SIMD has two (SAM3 fc2 61.3 -> 58.0 us,
      // out-projection 20.3 -> 18.8; SigLIP fc2 44.1 -> 43.4, 17.7 -> 17.2)
      const int64_t t_n192 = (int64_t)((a.M + 127) / 128) * (a.N / 192);
      const int64_t t_m192 = (int64_t)(a.M / 192) * ((a.N + 127) / 128);
      if (a.N % 192 == 0) {
        if (t_n192 <= 256) return gemm32_go<128, 192, 4, 2, 4>(p, a.epi, s, ev);
        return gemm32_go<128, 192, 2, 2>(p, a.epi, s, ev);
      }
      if (a.M % 192 == 0) {
        if (t_m192 <= 256) return gemm32_go<192, 128, 2, 4, 4>(p, a.epi, s, ev);
        return gemm32_go<192, 128, 2, 2>(p, a.epi, s, ev);
      }
    }
    // small products (e.g. 1024 tokens x 448 columns): 128x128 tiles would
    // leave most CUs idle, so 64x64 tiles (one 32x32 block per wave) with
    // four LDS stages: a lone workgroup per CU has nothing else to hide its
    // load latency behind. With a long K (the Hiera fc2, K = 1792 / 3584)
    // the waves split K instead (13.2 -> 12.3 us on the 1024x448x1792 fc2);
    // for short K the partial-tile reduction costs more than it saves
    // Up to 256 such tiles the waves split K over smaller tiles instead,
    // 32x32 (up to 128 64x64 tiles) or 32x64 (up to 256), for four times or
    // twice the workgroups. Hiera 1024 and 256 token blocks, per launch:
    // out-projection 5.45 -> 4.51 / 7.20 -> 5.10 us, fc2 9.85 -> 7.26 /
    // 16.2 -> 10.0; 256 tokens: qkv (with V^T) 8.01 -> 7.19, fc1 8.07 ->
    // 7.25. (Two LDS stages above 256 tiles won alone, 7.44 -> 7.21 us on
    // the 1024-token qkv, but lost inside the block.)
    const int64_t t64 = (int64_t)((a.M + 63) / 64) * ((a.N + 63) / 64);
    if (t128 < 192 && a.epi != EPI_BIAS_POS) {
      if (t64 <= 128) return gemm32_go<32, 32, 2, 2, 4, false, true>(p, a.epi, s, ev);
      if (t64 <= 256) return gemm32_go<32, 64, 2, 2, 4, false, true>(p, a.epi, s, ev);
    }
    if (t128 < 192 && a.K >= 1024) return gemm32_go<64, 64, 2, 2, 4, false, true>(p, a.epi, s, ev);
    if (t128 < 192) return gemm32_go<64, 64, 2, 2, 4>(p, a.epi, s, ev);
    return gemm32_go<128, 128, 2, 2>(p, a.epi, s, ev);
  }
  const int64_t big_tiles = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
  if (big_tiles >= 512) return gemm_go<bf16, 128, 128, 4, 4>(a, s, ev);
  return gemm_go<bf16, 64, 64, 2, 2>(a, s, ev);
}

}  // namespace vit
