// MFMA GEMM for gfx950: C[M][N] = A[M][K] * B[N][K]^T with fused A-operand
// producers (plain rows, implicit 3x3 convolution, GroupNorm + LeakyReLU)
// and fused epilogues (bias, ReLU, residual).
//
// Serves the dense steps of the EDiT layer ("EDiT: Efficient Diffusion
// Transformers with Linear Compressed Attention" notes): the ConvFusion 3x3
// compressing conv and its 1x1 restore with the residual (section
// "ConvFusion"), the query, key and value Linears (sections "ConvFusion" and
// "Spatial Compressor"), the output Linear and the hybrid's text Linears
// (section "MM-EDiT").
//
// Tiling: 256 threads = 4 waves in a WM x WN grid; a block tile BM x BN,
// K in steps of 128 bytes per row (64 bf16 / 32 f32). Tiles pass through
// registers into double-buffered LDS with a 16-byte row pad (conflict-free
// 16-byte fragment reads), one barrier per K step. The epilogue parks the
// fp32 accumulators in LDS and writes each row with 16-byte stores.
#include "common.hpp"
#include "launch.hpp"

namespace edit {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Segment lookup without indexing the kernel-argument array dynamically.
template <typename P>
__device__ __forceinline__ P pick3(const P (&a)[3], int i) {
  return i == 0 ? a[0] : (i == 1 ? a[1] : a[2]);
}

template <typename T, int BM, int BN, int WM, int WN, int AM, int EM>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs<T> p) {
  constexpr int EPC = Chunk<T>::n;              // elements per 16 B chunk
  constexpr int BK = 8 * EPC;                   // elements per 128 B K step
  constexpr int ROW = 72 * 2 / sizeof(T);       // LDS row pitch in elements (144 B)
  constexpr int KSTEPS = BK / 32;               // 32-wide matrix-core steps per K step
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 16, NI = WTN / 16;
  constexpr int APASS = BM / 32, BPASS = BN / 32;
  constexpr int LDS_MAIN = 2 * (BM + BN) * ROW * (int)sizeof(T);
  constexpr int CROW = BN + 4;
  constexpr int LDS_EPI = BM * CROW * 4;
  constexpr int LDS_BYTES = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
  static_assert(WM * WN == 4, "4 waves");
  static_assert(BM % 32 == 0 && BN % 32 == 0 && WTM % 16 == 0 && WTN % 16 == 0, "tile");
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + 2 * BM * ROW;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int NB = (p.N + BN - 1) / BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int m0 = (tile / NB) * BM, n0 = (tile % NB) * BN;
  const int cc = tid & 7;              // 16 B chunk column this thread loads
  const int rr = tid >> 3;             // first row this thread loads

  // Per-row state of the A producer.
  const T* arow[APASS];
  int ay[APASS], ax[APASS], ab[APASS];
  bool aval[APASS];
#pragma unroll
  for (int j = 0; j < APASS; ++j) {
    const int m = m0 + rr + 32 * j;
    aval[j] = m < p.M;
    const int mm = aval[j] ? m : 0;
    arow[j] = p.A + (size_t)mm * p.lda;
    if (AM == A_CONV3) {
      const int hw = p.H * p.W;
      const int r = mm % hw;
      ay[j] = r / p.W;
      ax[j] = r % p.W;
      ab[j] = 0;
    } else if (AM == A_GNACT) {
      ab[j] = mm / p.rows_per_batch;
      ay[j] = ax[j] = 0;
    } else {
      ay[j] = ax[j] = ab[j] = 0;
    }
  }
  const T* brow[BPASS];
  bool bval[BPASS];
#pragma unroll
  for (int j = 0; j < BPASS; ++j) {
    const int n = n0 + rr + 32 * j;
    bval[j] = n < p.N;
    const int nn = bval[j] ? n : 0;
    brow[j] = pick3(p.Bseg, nn / p.seg_rows) + (size_t)(nn % p.seg_rows) * p.ldb;
  }

  u32x4 ra[APASS], rb[BPASS];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  auto load_tiles = [&](int k0) {
    const int k = k0 + cc * EPC;
    if (AM == A_CONV3) {
      const int tap = k / p.Cin, cin = k - tap * p.Cin;
      const int dy = tap / 3 - 1, dx = tap % 3 - 1;
#pragma unroll
      for (int j = 0; j < APASS; ++j) {
        const int yy = ay[j] + dy, xx = ax[j] + dx;
        const bool ok = aval[j] && tap < 9 && yy >= 0 && yy < p.H && xx >= 0 && xx < p.W;
        ra[j] = ok ? *reinterpret_cast<const u32x4*>(arow[j] + (dy * p.W + dx) * p.Cin + cin) : zero4;
      }
    } else {
#pragma unroll
      for (int j = 0; j < APASS; ++j)
        ra[j] = (aval[j] && k < p.K) ? *reinterpret_cast<const u32x4*>(arow[j] + k) : zero4;
    }
#pragma unroll
    for (int j = 0; j < BPASS; ++j)
      rb[j] = (bval[j] && k < p.K) ? *reinterpret_cast<const u32x4*>(brow[j] + k) : zero4;
  };

  auto store_tiles = [&](int buf, int k0) {
    T* a = As + buf * BM * ROW;
    T* b = Bs + buf * BN * ROW;
    if (AM == A_GNACT) {
      const int k = k0 + cc * EPC;
#pragma unroll
      for (int j = 0; j < APASS; ++j) {
        u32x4 v = ra[j];
        if (aval[j] && k < p.K) {
          const T* e = reinterpret_cast<const T*>(&v);
          T o[EPC];
          const float* sc = p.scale + (size_t)ab[j] * p.K + k;
          const float* sh = p.shift + (size_t)ab[j] * p.K + k;
#pragma unroll
          for (int i = 0; i < EPC; ++i) {
            float t = to_f32(e[i]) * sc[i] + sh[i];
            t = t >= 0.0f ? t : 0.01f * t;
            o[i] = from_f32<T>(t);
          }
          v = *reinterpret_cast<const u32x4*>(o);
        }
        *reinterpret_cast<u32x4*>(a + (rr + 32 * j) * ROW + cc * EPC) = v;
      }
    } else {
#pragma unroll
      for (int j = 0; j < APASS; ++j)
        *reinterpret_cast<u32x4*>(a + (rr + 32 * j) * ROW + cc * EPC) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < BPASS; ++j)
      *reinterpret_cast<u32x4*>(b + (rr + 32 * j) * ROW + cc * EPC) = rb[j];
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc_zero(acc[i][j]);

  const int nk = (p.K + BK - 1) / BK;
  load_tiles(0);
  store_tiles(0, 0);
  __syncthreads();

  typedef typename Frag<T>::type FragT;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * BK);
    const T* a = As + cur * BM * ROW + (wm * WTM + fr) * ROW + fk;
    const T* b = Bs + cur * BN * ROW + (wn * WTN + fr) * ROW + fk;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      FragT af[MI], bfr[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) frag_load(af[i], a + i * 16 * ROW + s * 32);
#pragma unroll
      for (int j = 0; j < NI; ++j) frag_load(bfr[j], b + j * 16 * ROW + s * 32);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) mma16(acc[i][j], af[i], bfr[j]);
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1, (kt + 1) * BK);
    __syncthreads();
  }

  // Epilogue: accumulators -> LDS (fp32) -> bias / ReLU / residual -> 16 B stores.
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Cs[(wm * WTM + i * 16 + (lane >> 4) * 4 + r) * CROW + wn * WTN + j * 16 + fr] = acc[i][j][r];
  __syncthreads();

  constexpr int CPR = BN / 8;   // 8-column groups per row
  for (int idx = tid; idx < BM * CPR; idx += 256) {
    const int row = idx / CPR, cg = idx % CPR;
    const int m = m0 + row, n = n0 + cg * 8;
    if (m >= p.M || n >= p.N) continue;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = Cs[row * CROW + cg * 8 + i];
    float bv[8];
    load8(pick3(p.bias, n / p.seg_rows) + n % p.seg_rows, bv);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += bv[i];
    if (EM == E_BIAS_RELU) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] > 0.0f ? v[i] : 0.0f;
    } else if (EM == E_BIAS_RES) {
      float rv[8];
      load8(p.R + (size_t)m * p.ldr + n, rv);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += rv[i];
    }
    store8(p.C + (size_t)m * p.ldc + n, v);
  }
}

template <typename T, int BM, int BN, int WM, int WN>
static hipError_t launch_tiles(const GemmArgs<T>& a, AMode am, EMode em, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  dim3 grid(tiles), block(256);
#define EDIT_GEMM_CASE(AMV, EMV)                                                               \
  if (am == AMV && em == EMV) {                                                               \
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, AMV, EMV>), grid, block, 0, s, a);     \
    return hipGetLastError();                                                                 \
  }
  EDIT_GEMM_CASE(A_PLAIN, E_BIAS)
  EDIT_GEMM_CASE(A_PLAIN, E_BIAS_RELU)
  EDIT_GEMM_CASE(A_CONV3, E_BIAS)
  EDIT_GEMM_CASE(A_GNACT, E_BIAS_RES)
#undef EDIT_GEMM_CASE
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_gemm(const GemmArgs<T>& a, AMode am, EMode em, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.N % 128 != 0 && a.N % 96 == 0) return launch_tiles<T, 128, 96, 2, 2>(a, am, em, s);
  return launch_tiles<T, 128, 128, 2, 2>(a, am, em, s);
}

template hipError_t launch_gemm<bf16>(const GemmArgs<bf16>&, AMode, EMode, hipStream_t);
template hipError_t launch_gemm<float>(const GemmArgs<float>&, AMode, EMode, hipStream_t);

}  // namespace edit
