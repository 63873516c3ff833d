// MFMA GEMM for gfx950: C[M][N] = A[M][K] * B[N][K]^T with fused A-operand
// producers (plain rows, implicit 3x3 convolution, two row sources side by
// side) and fused epilogues (bias, ReLU).
//
// Serves the dense steps of the EDiT layer ("EDiT: Efficient Diffusion
// Transformers with Linear Compressed Attention" notes): the ConvFusion 3x3
// compressing conv, the query Linear over [X | act] with the 1x1 restore
// folded into its weights (section "ConvFusion"), the key and value Linears
// (section "Spatial Compressor"), the output Linear and the hybrid's text
// Linears (section "MM-EDiT"). Used for fp32 and for bf16 shapes outside the
// direct-to-LDS kernel's range.
//
// Tiling: 256 threads = 4 waves in a WM x WN grid; a block tile BM x BN,
// K in steps of 128 bytes per row (64 bf16 / 32 f32). Tiles pass through
// registers into LDS (double- or single-buffered). An LDS row is 128 bytes =
// 8 chunks of 16 bytes; chunk c of row r is stored at position
// c ^ ((r >> 1) & 7). A 32x32 fragment read touches one chunk in each of 32
// rows per lane half; with this swizzle gfx950 serves it at full LDS read
// bandwidth (~214 B/clk/CU measured), while c ^ (r & 7) or 160-byte padded
// rows measure half that. The epilogue parks the
// fp32 accumulators in LDS and writes each row with 16-byte stores.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace edit {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Segment lookup without indexing the kernel-argument array dynamically.
template <typename P>
__device__ __forceinline__ P pick3(const P (&a)[3], int i) {
  return i == 0 ? a[0] : (i == 1 ? a[1] : a[2]);
}

// Rows of wave tiles the epilogue stages per pass: the largest divisor of
// WM whose fp32 rows fit in the main loop's LDS.
constexpr int epi_group(int WM, int WTM, int crow_bytes, int lds) {
  int k = WM;
  while (k > 1 && (WM % k != 0 || k * WTM * crow_bytes > lds)) --k;
  return k;
}

template <typename T, int BM, int BN, int WM, int WN, int AM, int EM, int STAGES, int PF, int SB, int MM>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs<T> p) {
  constexpr int NT = 64 * WM * WN;              // threads
  constexpr int EPC = Chunk<T>::n;              // elements per 16 B chunk
  constexpr int BK = 8 * EPC;                   // elements per 128 B K step
  constexpr int ROW = 128 / (int)sizeof(T);     // LDS row pitch in elements (128 B, swizzled)
  constexpr int KSTEPS = BK / (512 / MM);        // matrix-core K steps per K tile (16 deep for 32x32, 32 for 16x16)
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / MM, NI = WTN / MM;   // MM x MM blocks per wave
  constexpr int RPP = NT / 8;                   // tile rows loaded per pass
  constexpr int APASS = (BM + RPP - 1) / RPP, BPASS = (BN + RPP - 1) / RPP;
  constexpr int LDS_MAIN = STAGES * (BM + BN) * ROW * (int)sizeof(T);
  constexpr int CROW = BN + 4;
  constexpr int KG = epi_group(WM, WTM, CROW * 4, LDS_MAIN);
  constexpr int RG = KG * WTM;                  // rows staged per epilogue pass
  constexpr int LDS_EPI = RG * CROW * 4;
  constexpr int LDS_BYTES = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
  static_assert(WTM % MM == 0 && WTN % MM == 0 && BN % 8 == 0 && RPP % 16 == 0, "tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + STAGES * BM * ROW;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int NB = (p.N + BN - 1) / BN;
  // Split-K (E_F32): grid row s multiplies K columns [s * kchunk, s * kchunk + Kc).
  const int kbase = EM == E_F32 && p.kchunk ? (int)blockIdx.y * p.kchunk : 0;
  const int Kc = EM == E_F32 && p.kchunk ? min(p.kchunk, p.K - kbase) : p.K;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int m0 = (tile / NB) * BM, n0 = (tile % NB) * BN;
  const int cc = tid & 7;              // 16 B chunk column this thread loads
  const int rr = tid >> 3;             // first tile row this thread loads
  const int ccs = cc ^ ((rr >> 1) & 7);   // its swizzled LDS position (RPP is a multiple of 16)

  // Per-row state of the A producer.
  const T* arow[APASS];
  const T* arow2[AM == A_CAT2 ? APASS : 1];
  int ay[APASS], ax[APASS];
  bool aval[APASS];
#pragma unroll
  for (int j = 0; j < APASS; ++j) {
    const int r = rr + RPP * j;
    const int m = m0 + r;
    aval[j] = (BM % RPP == 0 || r < BM) && m < p.M;
    const int mm = aval[j] ? m : 0;
    arow[j] = p.A + (size_t)mm * p.lda + kbase;
    if (AM == A_CAT2) arow2[AM == A_CAT2 ? j : 0] = p.A2 + (size_t)mm * p.lda2;
    if (AM == A_CONV3) {
      const int hw = p.H * p.W;
      const int q = mm % hw;
      ay[j] = q / p.W;
      ax[j] = q % p.W;
    } else {
      ay[j] = ax[j] = 0;
    }
  }
  const T* brow[BPASS];
  bool bval[BPASS];
#pragma unroll
  for (int j = 0; j < BPASS; ++j) {
    const int r = rr + RPP * j;
    const int n = n0 + r;
    bval[j] = (BN % RPP == 0 || r < BN) && n < p.N;
    const int nn = bval[j] ? n : 0;
    brow[j] = pick3(p.Bseg, nn / p.seg_rows) + (size_t)(nn % p.seg_rows) * p.ldb + kbase;
  }

  // Two register sets for prefetched global tiles (ra0/rb0, ra1/rb1): with
  // PF == 2 tile kt + 2 is requested while tile kt is multiplied, so the LDS
  // store of tile kt + 1 waits on loads issued a whole iteration earlier.
  u32x4 ra0[APASS], rb0[BPASS], ra1[APASS], rb1[BPASS];
  bool aok0[APASS], bok0[BPASS], aok1[APASS], bok1[BPASS];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // Loads never branch: an invalid row or K chunk reads a valid address and
  // the value is replaced by zero when it is stored to LDS (not here, so the
  // wait for the load lands at the store, after the tile's matrix work).
#define EDIT_LOAD_TILES(RA, RB, AOK, BOK, k0_)                                                \
  do {                                                                                        \
    const int k = (k0_) + cc * EPC;                                                           \
    const bool kin = k < Kc;                                                                  \
    int kb = k; /* K index the weights use */                                                 \
    if (AM == A_CONV3) {                                                                      \
      /* K tiles run channel slice outer, tap inner (when BK divides Cin), so a   */          \
      /* slice of the three input rows is reused by all nine taps while cached.   */          \
      int tap, cin;                                                                           \
      if (p.Cin % BK == 0) {                                                                  \
        const int kt_ = (k0_) / BK, nsl = p.Cin / BK;                                         \
        const int sl = kt_ / 9;                                                               \
        tap = kt_ - sl * 9;                                                                   \
        cin = sl * BK + cc * EPC;                                                             \
        kb = tap * p.Cin + cin;                                                               \
        if (kt_ >= 9 * nsl) tap = 9;                                                          \
      } else {                                                                                \
        tap = k / p.Cin;                                                                      \
        cin = k - tap * p.Cin;                                                                \
      }                                                                                       \
      const int dy = tap / 3 - 1, dx = tap % 3 - 1;                                           \
      _Pragma("unroll") for (int j = 0; j < APASS; ++j) {                                     \
        const int yy = ay[j] + dy, xx = ax[j] + dx;                                           \
        AOK[j] = aval[j] && tap < 9 && yy >= 0 && yy < p.H && xx >= 0 && xx < p.W;            \
        const T* src = AOK[j] ? arow[j] + (dy * p.W + dx) * p.Cin + cin : arow[j];            \
        RA[j] = *reinterpret_cast<const u32x4*>(src);                                         \
      }                                                                                       \
    } else {                                                                                  \
      /* A_CAT2: a 16-byte chunk lies in one source (K1 is a multiple of 8) */                \
      const bool sec = AM == A_CAT2 && k >= p.K1;                                             \
      _Pragma("unroll") for (int j = 0; j < APASS; ++j) {                                     \
        AOK[j] = aval[j] && kin;                                                              \
        const T* src = sec ? arow2[AM == A_CAT2 ? j : 0] + (AOK[j] ? k - p.K1 : 0)             \
                           : arow[j] + (AOK[j] ? k : 0);                                      \
        RA[j] = *reinterpret_cast<const u32x4*>(src);                                         \
      }                                                                                       \
    }                                                                                         \
    _Pragma("unroll") for (int j = 0; j < BPASS; ++j) {                                       \
      BOK[j] = bval[j] && kin;                                                                \
      RB[j] = *reinterpret_cast<const u32x4*>(brow[j] + (BOK[j] ? kb : 0));                   \
    }                                                                                         \
  } while (0)

#define EDIT_STORE_TILES(RA, RB, AOK, BOK, buf_, k0_)                                         \
  do {                                                                                        \
    T* a_ = As + (buf_) * BM * ROW;                                                           \
    T* b_ = Bs + (buf_) * BN * ROW;                                                           \
    _Pragma("unroll") for (int j = 0; j < APASS; ++j) {                                       \
      const int r = rr + RPP * j;                                                             \
      if (BM % RPP != 0 && r >= BM) continue;                                                 \
      *reinterpret_cast<u32x4*>(a_ + r * ROW + ccs * EPC) = AOK[j] ? RA[j] : zero4;           \
    }                                                                                         \
    _Pragma("unroll") for (int j = 0; j < BPASS; ++j) {                                       \
      const int r = rr + RPP * j;                                                             \
      if (BN % RPP != 0 && r >= BN) continue;                                                 \
      *reinterpret_cast<u32x4*>(b_ + r * ROW + ccs * EPC) = BOK[j] ? RB[j] : zero4;           \
    }                                                                                         \
  } while (0)

  typedef typename std::conditional<MM == 32, f32x16, f32x4>::type AccT;
  AccT acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc_zero(acc[i][j]);

  typedef typename Frag<T>::type FragT;
  // Lane l feeds row/column fr of an MM-block with the 8 K values of K group
  // kh (32x32x16: two groups of 8; 16x16x32: four).
  const int fr = lane % MM, kh = lane / MM;
  // A fragment covers 8 consecutive K values = one chunk (bf16) or two (f32).
  // Swizzled element offsets of the lane's chunk(s) for each K step: rows
  // fr + MM i all share ((row >> 1) & 7).
  int koff[KSTEPS][2];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int chunk = (s * (512 / MM) + kh * 8) / EPC + (EPC == 4 ? h : 0);
      koff[s][h] = (chunk ^ ((fr >> 1) & 7)) * EPC;
    }

  auto compute = [&](int buf) {
    const T* a = As + buf * BM * ROW + (wm * WTM + fr) * ROW;
    const T* b = Bs + buf * BN * ROW + (wn * WTN + fr) * ROW;
    // Fragments of step s+1 are read while the matrix cores work on step s.
    FragT af[2][MI], bfr[2][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) frag_load2(af[0][i], a + i * MM * ROW, koff[0][0], koff[0][1]);
#pragma unroll
    for (int j = 0; j < NI; ++j) frag_load2(bfr[0][j], b + j * MM * ROW, koff[0][0], koff[0][1]);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int c = s & 1, n = c ^ 1;
      if (s + 1 < KSTEPS) {
#pragma unroll
        for (int i = 0; i < MI; ++i) frag_load2(af[n][i], a + i * MM * ROW, koff[s + 1][0], koff[s + 1][1]);
#pragma unroll
        for (int j = 0; j < NI; ++j) frag_load2(bfr[n][j], b + j * MM * ROW, koff[s + 1][0], koff[s + 1][1]);
      }
      // Optionally pin the reads of step s+1 ahead of the matrix work of
      // step s (costs registers; measured slower at the shapes used here).
      if (SB) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) mma_any(acc[i][j], af[c][i], bfr[c][j]);
      if (SB) __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = (Kc + BK - 1) / BK;
  if (PF == 1) {
    EDIT_LOAD_TILES(ra0, rb0, aok0, bok0, 0);
    EDIT_STORE_TILES(ra0, rb0, aok0, bok0, 0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = STAGES == 2 ? (kt & 1) : 0;
      if (kt + 1 < nk) EDIT_LOAD_TILES(ra0, rb0, aok0, bok0, (kt + 1) * BK);
      compute(cur);
      if (STAGES == 1) __syncthreads();   // single buffer: every wave done reading
      if (kt + 1 < nk) EDIT_STORE_TILES(ra0, rb0, aok0, bok0, STAGES == 2 ? (cur ^ 1) : 0, (kt + 1) * BK);
      __syncthreads();
    }
  } else {
    // Prefetch distance two, unrolled by two so each register set is named.
    EDIT_LOAD_TILES(ra0, rb0, aok0, bok0, 0);
    if (nk > 1) EDIT_LOAD_TILES(ra1, rb1, aok1, bok1, BK);
    EDIT_STORE_TILES(ra0, rb0, aok0, bok0, 0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      // tile kt is in LDS buffer 0, tile kt+1 in flight in set 1
      if (kt + 2 < nk) EDIT_LOAD_TILES(ra0, rb0, aok0, bok0, (kt + 2) * BK);
      compute(0);
      if (STAGES == 1) __syncthreads();
      if (kt + 1 < nk) EDIT_STORE_TILES(ra1, rb1, aok1, bok1, STAGES == 2 ? 1 : 0, (kt + 1) * BK);
      __syncthreads();
      if (kt + 1 >= nk) break;
      // tile kt+1 is in LDS buffer 1, tile kt+2 in flight in set 0
      if (kt + 3 < nk) EDIT_LOAD_TILES(ra1, rb1, aok1, bok1, (kt + 3) * BK);
      compute(STAGES == 2 ? 1 : 0);
      if (STAGES == 1) __syncthreads();
      if (kt + 2 < nk) EDIT_STORE_TILES(ra0, rb0, aok0, bok0, 0, (kt + 2) * BK);
      __syncthreads();
    }
  }
#undef EDIT_LOAD_TILES
#undef EDIT_STORE_TILES

  // Epilogue, KG wave-rows at a time: accumulators -> LDS (fp32) ->
  // bias / ReLU -> 16-byte row stores.
  float* Cs = reinterpret_cast<float*>(smem);
  constexpr int CPR = BN / 8;   // 8-column groups per row
#pragma unroll 1
  for (int eg = 0; eg < WM / KG; ++eg) {
    if (wm / KG == eg) {
      const int rbase = (wm % KG) * WTM;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int r = 0; r < (MM == 32 ? 16 : 4); ++r)
            Cs[(rbase + i * MM + (MM == 32 ? (r >> 2) * 8 + kh * 4 + (r & 3) : kh * 4 + r)) * CROW + wn * WTN +
               j * MM + fr] = acc[i][j][r];
    }
    __syncthreads();
    for (int idx = tid; idx < RG * CPR; idx += NT) {
      const int row = idx / CPR, cg = idx % CPR;
      const int m = m0 + eg * RG + row, n = n0 + cg * 8;
      if (m >= p.M || n >= p.N) continue;
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = Cs[row * CROW + cg * 8 + i];
      if (EM == E_F32) {
        store8(p.Cf + (size_t)blockIdx.y * p.split_stride + (size_t)m * p.ldc + n, v);
        continue;
      }
      float bv[8];
      load8(pick3(p.bias, n / p.seg_rows) + n % p.seg_rows, bv);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += bv[i];
      if (EM == E_RES) {
        load8(p.R + (size_t)m * p.ldr + n, bv);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] += bv[i];
      }
      if (EM == E_BIAS_RELU) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = v[i] > 0.0f ? v[i] : 0.0f;
      }
      store8(p.C + (size_t)m * p.ldc + n, v);
    }
    __syncthreads();
  }
}

template <typename T, int BM, int BN, int WM, int WN, int STAGES = 2, int PF = 1, int SB = 0, int MM = 32>
static hipError_t launch_tiles(const GemmArgs<T>& a, AMode am, EMode em, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const int splits = em == E_F32 && a.kchunk ? (a.K + a.kchunk - 1) / a.kchunk : 1;
  dim3 grid(tiles, splits), block(64 * WM * WN);
#define EDIT_GEMM_CASE(AMV, EMV)                                                               \
  if (am == AMV && em == EMV) {                                                               \
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, AMV, EMV, STAGES, PF, SB, MM>), grid, block, 0, s, a);     \
    return hipGetLastError();                                                                 \
  }
  EDIT_GEMM_CASE(A_PLAIN, E_BIAS)
  EDIT_GEMM_CASE(A_PLAIN, E_BIAS_RELU)
  EDIT_GEMM_CASE(A_CONV3, E_BIAS)
  EDIT_GEMM_CASE(A_CAT2, E_BIAS_RELU)
  EDIT_GEMM_CASE(A_PLAIN, E_F32)
  EDIT_GEMM_CASE(A_PLAIN, E_RES)
  EDIT_GEMM_CASE(A_CONV3, E_RES)
#undef EDIT_GEMM_CASE
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_gemm(const GemmArgs<T>& a, AMode am, EMode em, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.fold.W != nullptr) {
    // the restore fold requested with the conv: on the direct-load kernel (fused there when it can be),
    // else the register-staged conv, then the fold's own kernel
    if (am != A_CONV3) return hipErrorInvalidValue;
    if constexpr (std::is_same<T, bf16>::value) {
      const hipError_t e = launch_gemm_dma(a, am, em, s);
      if (e != hipErrorNotSupported) return e;
      GemmArgs<T> b = a;
      b.fold = FoldArgs{};
      const hipError_t e2 = launch_gemm<T>(b, am, em, s);
      if (e2 != hipSuccess) return e2;
      const FoldArgs& f = a.fold;
      return launch_restore_fold<bf16>(f.W, f.b, f.W2, f.b2, f.C, f.Cr, f.wcat, f.bcat, s);
    }
    return hipErrorInvalidValue;
  }
  if (a.R != nullptr) {
    if (em != E_BIAS) return hipErrorInvalidValue;
    em = E_RES;
  }
  if (em == E_BIAS_GN) {
    // only the direct-load conv has the statistics epilogue
    if constexpr (std::is_same<T, bf16>::value) return launch_gemm_dma(a, am, em, s);
    return hipErrorNotSupported;
  }
  if constexpr (std::is_same<T, bf16>::value) {
    const hipError_t e = launch_gemm_dma(a, am, em, s);
    if (e != hipErrorNotSupported) return e;
  }
  // Tile choice (measured on MI355X at the 16384-token shapes; the loop is
  // bound by LDS traffic and latency, not by the matrix cores, so the
  // 16x16x32 step with its smaller fragments measures slightly ahead):
  //  - N a multiple of 128 (the C x C and 2C x C projections):
  //    128 x 128 tiles, one LDS stage, 2 x 2 waves of 64 x 64;
  //  - otherwise (the C/r-wide 3x3 conv, 96 | N): 128 x 96 tiles, two stages,
  //    2 x 2 waves of 64 x 48 on the 16x16x32 step (48 does not split into
  //    32-wide blocks, and 32 x 96 wave tiles reuse fragments too little).
  if (a.N % 128 == 0) return launch_tiles<T, 128, 128, 2, 2, 1, 1, 0, 16>(a, am, em, s);
  if (a.N % 96 == 0) return launch_tiles<T, 128, 96, 2, 2, 2, 1, 0, 16>(a, am, em, s);
  return launch_tiles<T, 128, 128, 2, 2, 1, 1, 0, 16>(a, am, em, s);
}

template hipError_t launch_gemm<bf16>(const GemmArgs<bf16>&, AMode, EMode, hipStream_t);
template hipError_t launch_gemm<float>(const GemmArgs<float>&, AMode, EMode, hipStream_t);

}  // namespace edit
