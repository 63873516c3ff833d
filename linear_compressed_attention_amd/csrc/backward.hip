// Backward pass of the EDiT layer on gfx950: the kernels that are not GEMMs.
//
// Page "EDiT: Efficient Diffusion Transformers with Linear Compressed
// Attention" (ICCV 2025 notes): the layer is trained by distillation
// (section "训练策略", training strategy), which needs the gradient of every forward step
// (sections "ConvFusion", "Spatial Compressor", "Linear-attention formula").
// Each kernel below is the chain rule of one forward step; the GEMM-shaped
// products run on the GEMM kernels (with transposed operands where the
// contraction is over tokens). Every reduction sums in a fixed order, so
// gradients are bit-for-bit reproducible.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace edit {

// ---------------------------------------------------------------------------
// Transpose: out[c][r] = in[r][c] through a 64 x 65 LDS tile, batched over
// blockIdx.z (in + z * zin, out + z * zout). With a shift, z is the 3x3
// conv's tap (ky, kx) = (z / 3, z % 3): out[c][m] = in[m - off][c] where the
// pixel of m - off lies inside its image and reads m through that tap, else
// 0; off = (ky - 1) W + (kx - 1). Rows are tokens b*H*W + y*W + x. Output
// columns rows .. rows_pad - 1 (the row padding of out) are written as zeros.
// With colsum, each block also writes its tile's column sums over its 64 rows
// (the transposed tensor's per-tile row sums, in a fixed order) to
// colsum[(z * cols + c) * gridDim.y + blockIdx.y] (fp32): a bias gradient is
// then a short sum over them instead of another pass over the tensor.
// ---------------------------------------------------------------------------
template <typename T, bool SHIFT>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, int rows, int rows_pad, int cols,
                                                        int ldi, T* __restrict__ out, int ldo, int H, int W,
                                                        long zin, long zout, float* __restrict__ colsum,
                                                        const T* __restrict__ in2) {
  // 64 x 64 tile; every global access is 16 bytes (EPC elements): a load
  // takes EPC consecutive columns of one row, a store EPC consecutive rows
  // of one column. cols, ldi, ldo and rows_pad are multiples of EPC.
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int VPR = 64 / EPC;                 // 16-byte vectors per 64-element tile row
  typedef uint32_t u32x4t __attribute__((ext_vector_type(4)));
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  in = in2 != nullptr && blockIdx.z == 1 ? in2 : in + (long)blockIdx.z * zin;
  out += (long)blockIdx.z * zout;
  const int ky = SHIFT ? (int)blockIdx.z / 3 : 1, kx = SHIFT ? (int)blockIdx.z % 3 : 1;
  for (int v = threadIdx.x; v < 64 * VPR; v += 256) {
    const int i = v / VPR, cv = v % VPR;
    const int r = r0 + i, c = c0 + cv * EPC;
    T e[EPC];
#pragma unroll
    for (int k = 0; k < EPC; ++k) e[k] = from_f32<T>(0.0f);
    if (r < rows && c < cols) {
      size_t src = (size_t)r;
      bool ok = true;
      if (SHIFT) {
        // r is the destination token m'; the source token m = m' - off is
        // valid when its pixel (y, x) reads pixel(m') through tap (ky, kx).
        const int hw = H * W, b = r / hw, q = r - b * hw, y1 = q / W, x1 = q - (q / W) * W;
        const int y = y1 - (ky - 1), x = x1 - (kx - 1);
        ok = y >= 0 && y < H && x >= 0 && x < W;
        src = (size_t)b * hw + (size_t)y * W + x;
      }
      if (ok) *reinterpret_cast<u32x4t*>(e) = *reinterpret_cast<const u32x4t*>(in + src * ldi + c);
    }
#pragma unroll
    for (int k = 0; k < EPC; ++k) tile[i][cv * EPC + k] = to_f32(e[k]);
  }
  __syncthreads();
  if (colsum != nullptr) {
    // wave q adds rows 16q .. 16q + 15 of every column; the four waves' sums meet in LDS
    __shared__ float csum[4][64];
    const int i = threadIdx.x & 63, q = threadIdx.x >> 6;
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) a += tile[q * 16 + k][i];
    csum[q][i] = a;
    __syncthreads();
    if (threadIdx.x < 64 && c0 + i < cols)
      colsum[((long)blockIdx.z * cols + c0 + i) * gridDim.y + blockIdx.y] =
          (csum[0][i] + csum[1][i]) + (csum[2][i] + csum[3][i]);
  }
  for (int v = threadIdx.x; v < 64 * VPR; v += 256) {
    const int i = v / VPR, rv = v % VPR;          // column c0 + i, rows r0 + rv*EPC ..
    const int c = c0 + i, r = r0 + rv * EPC;
    if (c >= cols || r >= rows_pad) continue;
    T e[EPC];
#pragma unroll
    for (int k = 0; k < EPC; ++k) e[k] = from_f32<T>(tile[rv * EPC + k][i]);
    *reinterpret_cast<u32x4t*>(out + (size_t)c * ldo + r) = *reinterpret_cast<const u32x4t*>(e);
  }
}

template <typename T>
hipError_t launch_transpose(const T* in, int rows, int cols, int ldi, T* out, int ldo, hipStream_t s,
                            int rows_pad, int batch, long zin, long zout, float* colsum, const T* in2) {
  if (rows_pad < rows) rows_pad = rows;
  if (rows <= 0 || cols <= 0 || batch <= 0) return hipSuccess;
  constexpr int EPC = 16 / (int)sizeof(T);
  if (cols % EPC || ldi % EPC || ldo % EPC || rows_pad % EPC || zin % EPC || zout % EPC)
    return hipErrorInvalidValue;
  dim3 grid((cols + 63) / 64, (rows_pad + 63) / 64, batch);
  hipLaunchKernelGGL((transpose_kernel<T, false>), grid, dim3(256), 0, s, in, rows, rows_pad, cols, ldi, out, ldo, 1,
                     1, zin, zout, colsum, in2);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_shift_transpose9(const T* in, int B, int H, int W, int cols, int ldi, T* out, int ldo,
                                   hipStream_t s, float* colsum) {
  const int rows = B * H * W;
  if (rows <= 0 || cols <= 0) return hipSuccess;
  constexpr int EPC = 16 / (int)sizeof(T);
  if (cols % EPC || ldi % EPC || ldo % EPC || ldo < rows) return hipErrorInvalidValue;
  dim3 grid((cols + 63) / 64, (ldo + 63) / 64, 9);
  hipLaunchKernelGGL((transpose_kernel<T, true>), grid, dim3(256), 0, s, in, rows, ldo, cols, ldi, out, ldo, H, W,
                     0L, (long)cols * ldo, colsum, nullptr);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bias gradients from the transposes' per-tile sums: out[r] = sum over the n
// row tiles of part[r * n + t], one wave per row, lanes strided over the
// tiles, then a butterfly; a fixed order. out32 (optional) keeps the fp32 sum.
// Rows from rsplit on go to out2 (row r - rsplit) and have no fp32 copy.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void colsum_finalize_kernel(const float* __restrict__ part, int rows, int n,
                                                              T* __restrict__ out, float* __restrict__ out32,
                                                              T* __restrict__ out2, int rsplit) {
  const int r = blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= rows) return;
  const float* p = part + (size_t)r * n;
  float a = 0.0f;
  for (int t = lane; t < n; t += 64) a += p[t];
  a = wave_sum(a);
  if (lane == 0) {
    if (r < rsplit) {
      out[r] = from_f32<T>(a);
      if (out32) out32[r] = a;
    } else {
      out2[r - rsplit] = from_f32<T>(a);
    }
  }
}

template <typename T>
hipError_t launch_colsum_finalize(const float* part, int rows, int n, T* out, hipStream_t s, float* out32, T* out2,
                                  int rsplit) {
  if (rows <= 0) return hipSuccess;
  if (n <= 0) return hipErrorInvalidValue;
  if (out2 == nullptr || rsplit <= 0 || rsplit > rows) rsplit = rows;
  hipLaunchKernelGGL((colsum_finalize_kernel<T>), dim3((rows + 3) / 4), dim3(256), 0, s, part, rows, n, out, out32,
                     out2, rsplit);
  return hipGetLastError();
}

// p[0 .. n) = 0 (a kernel, so that stream capture records no memset node).
template <typename T>
__global__ __launch_bounds__(256) void zero_kernel(T* __restrict__ p, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = from_f32<T>(0.0f);
}

template <typename T>
hipError_t launch_zero(T* p, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((zero_kernel<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K reduction: sum_s part[s][r][c] (row stride cols), s in order, to
// out[(r % rpg) * ldo + (r / rpg) * gstride + c]: rows come in groups of rpg
// (the 3x3 conv's taps, each a [C/r][C] block) that interleave in the
// output row. Four columns per thread.
// ---------------------------------------------------------------------------
template <typename O, typename O2>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S,
                                                            long long stride, int rows, int cols,
                                                            O* __restrict__ out, int ldo, int rpg, int gstride,
                                                            O2* __restrict__ out2, int rsplit,
                                                            const O* __restrict__ bias) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (long long)rows * cols) return;
  const int r = (int)(i / cols), c = (int)(i - (long long)r * cols);
  f32x4 v = *reinterpret_cast<const f32x4*>(part + i);
  for (int s = 1; s < S; ++s) v += *reinterpret_cast<const f32x4*>(part + (size_t)s * stride + i);
  // the column bias of a split-K Linear, added once to the full sum
  if (bias != nullptr)
    for (int j = 0; j < 4; ++j) v[j] += (float)bias[c + j];
  const float o[4] = {v[0], v[1], v[2], v[3]};
  // rows from rsplit on go to the second output
  if (r < rsplit) store4(out + (size_t)(r % rpg) * ldo + (size_t)(r / rpg) * gstride + c, o);
  else store4(out2 + (size_t)((r - rsplit) % rpg) * ldo + (size_t)((r - rsplit) / rpg) * gstride + c, o);
}

template <typename O, typename O2>
hipError_t launch_splitk_reduce(const float* part, int S, long long stride, int rows, int cols, O* out, int ldo,
                                hipStream_t s, int rpg, int gstride, O2* out2, int rsplit, const O* bias) {
  const long long n = (long long)rows * cols;
  if (n <= 0) return hipSuccess;
  if (out2 == nullptr || rsplit <= 0 || rsplit > rows) rsplit = rows;
  if (rpg <= 0) rpg = rsplit;
  if (cols % 4 || ldo % 4 || gstride % 4 || stride % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL((splitk_reduce_kernel<O, O2>), dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, part, S,
                     stride, rows, cols, out, ldo, rpg, gstride, out2, rsplit, bias);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-head products on the matrix cores. A head's d x d state matrix M sits
// in LDS as the A operand of the 32x32x16 step (rows padded to RT*32, K to
// KS*16 with zeros); for bf16 it is held as two bf16 matrices hi + lo
// (hi = bf16(M), lo = bf16(M - hi)), so M times a bf16 token row is formed to
// about fp32 accuracy; for f32 the f32 step takes M itself. A wave takes 32
// tokens as the B operand's columns (lane l: token l % 32, 8 K values from
// 8*(l/32)), and the accumulator holds the product transposed: element r of
// lane l is row 8*(r/4) + 4*(l/32) + r%4 (a channel of the head) of column
// l % 32 (a token). Per-token dot products over the head's channels add
// each half-wave's 16 rows per tile and then the two halves (lanes l, l^32).
// ---------------------------------------------------------------------------
template <typename T, int KS>
struct HeadMat {
  static constexpr int RT = (KS + 1) / 2;                 // 32-row tiles
  static constexpr int KP = KS * 16 + 16 / (int)sizeof(T);  // padded LDS row (16-byte multiple)
  static constexpr int NC = sizeof(T) == 2 ? 2 : 1;       // bf16: hi + lo copies
};

__device__ __forceinline__ bf16x8 frag_ld(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 frag_ld(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
  return r;
}
template <typename F> __device__ __forceinline__ F frag_zero() {
  F r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = 0;
  return r;
}
__device__ __forceinline__ void load4(const bf16* p, float (&v)[4]) {
  const bf16x4 t = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (float)t[i];
}
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
  const f32x4 t = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = t[i];
}
// M (fp32, d x d, row-major at src) into the LDS operand, or its transpose
// (TR): dst row i, column k holds M[i][k] (TR: M[k][i]); dst holds NC copies
// of [RT * 32][KP]. A thread writes 4 consecutive columns of one row as one
// vector per copy (neighbouring threads: neighbouring columns).
__device__ __forceinline__ void store4_lds(bf16* p, const float (&v)[4]) { store4(p, v); }
__device__ __forceinline__ void store4_lds(float* p, const float (&v)[4]) { store4(p, v); }

template <typename T, int KS, bool TR>
__device__ __forceinline__ void head_mat_fill(T* dst, const float* __restrict__ src, int d) {
  using HM = HeadMat<T, KS>;
  constexpr int CP = HM::RT * 32 * HM::KP;
  constexpr int RW = HM::RT * 32;                  // rows of the operand
  constexpr int NQ = (KS * 16) / 4;                // 4-column groups per row
#pragma unroll 4
  for (int e = threadIdx.x; e < RW * NQ; e += blockDim.x) {
    const int row = e / NQ, c0 = (e - row * NQ) * 4;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (row < d && c0 < d) {
      if constexpr (TR) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = src[(size_t)(c0 + j) * d + row];
      } else {
        const f32x4 q = *reinterpret_cast<const f32x4*>(src + (size_t)row * d + c0);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = q[j];
      }
    }
    if constexpr (HM::NC == 2) {
      float hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hi[j] = (float)(bf16)v[j];
        lo[j] = v[j] - hi[j];
      }
      store4_lds(dst + row * HM::KP + c0, hi);
      store4_lds(dst + CP + row * HM::KP + c0, lo);
    } else {
      store4_lds(dst + row * HM::KP + c0, v);
    }
  }
}

// acc[rt] = M[rt-th 32 rows] x B for the wave's 32 tokens.
template <typename T, int KS, int RT>
__device__ __forceinline__ void head_mat_apply(const T* A, const typename Frag<T>::type (&bf)[KS],
                                               f32x16 (&acc)[RT], int lane) {
  using HM = HeadMat<T, KS>;
  constexpr int CP = HM::RT * 32 * HM::KP;
  const int col = lane & 31, kh = 8 * (lane >> 5);
#pragma unroll
  for (int rt = 0; rt < HM::RT; ++rt) acc_zero(acc[rt]);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int rt = 0; rt < HM::RT; ++rt)
#pragma unroll
      for (int c = 0; c < HM::NC; ++c) mma32(acc[rt], frag_ld(A + c * CP + (rt * 32 + col) * HM::KP + ks * 16 + kh), bf[ks]);
}

// The wave's 32-token tiles: tiles_per_wave consecutive tiles from tile0.
__device__ __forceinline__ int head_tile0(int tiles_per_wave) {
  return (blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * tiles_per_wave;
}

// ---------------------------------------------------------------------------
// Linear-attention backward, query side. Per token i and head (section
// "Linear-attention formula", y = q S / (q . z + eps)):
//   den = q . z + eps, t = S dy (t[a] = sum_n S[a][n] dy[n]),
//   dy . y = q . t / den, c = -(dy . y) / den, g = dy / den,
//   dq = t / den + c z, then the outer ReLU of the queries: dq_pre = dq where q > 0.
// dy . y is formed from q and t rather than from the stored y: the two
// terms of dq nearly cancel (y does not change when q is scaled), so y's
// rounding would be amplified. g (T) and c (f32) are kept for the state
// gradient dS = sum q^T g, dz = sum c q. Block: 4 waves of one (sample,
// head); t^T = S dy^T on the matrix cores.
// ---------------------------------------------------------------------------
template <typename T, int KS>
__global__ __launch_bounds__(256) void attn_bwd_q_kernel(const T* __restrict__ dy, const T* __restrict__ q,
                                                         const float* __restrict__ S,
                                                         const float* __restrict__ z, int N, int heads, int d,
                                                         float eps, int tiles_per_wave, T* __restrict__ g_out,
                                                         float* __restrict__ c_out, T* __restrict__ dq_pre) {
  using HM = HeadMat<T, KS>;
  using F = typename Frag<T>::type;
  __shared__ __attribute__((aligned(16))) T As[HM::NC * HM::RT * 32 * HM::KP];
  __shared__ float zs[HM::RT * 32];
  const int h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63;
  const int C = heads * d, col = lane & 31, half = lane >> 5;
  const size_t bh = (size_t)b * heads + h;
  head_mat_fill<T, KS, false>(As, S + bh * d * d, d);
  for (int i = threadIdx.x; i < HM::RT * 32; i += blockDim.x) zs[i] = i < d ? z[bh * d + i] : 0.0f;
  __syncthreads();
  const int t0 = head_tile0(tiles_per_wave);
  for (int t = 0; t < tiles_per_wave; ++t) {
    const int tok0 = (t0 + t) * 32;
    if (tok0 >= N) break;
    const int tok = tok0 + col;
    const bool valid = tok < N;
    const size_t row = ((size_t)b * N + (valid ? tok : 0)) * C + (size_t)h * d;
    F bf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = ks * 16 + 8 * half;
      bf[ks] = valid && k < d ? frag_ld(dy + row + k) : frag_zero<F>();
    }
    f32x16 acc[HM::RT];
    head_mat_apply<T, KS, HM::RT>(As, bf, acc, lane);
    float qv[HM::RT][16];
    float den = 0.0f, qt = 0.0f;
#pragma unroll
    for (int rt = 0; rt < HM::RT; ++rt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int a0 = rt * 32 + 8 * g + 4 * half;
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (valid && a0 < d) load4(q + row + a0, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qv[rt][4 * g + i] = v[i];
          den += v[i] * zs[a0 + i];
          qt += v[i] * acc[rt][4 * g + i];
        }
      }
    den += __shfl_xor(den, 32, kWave) + eps;
    qt += __shfl_xor(qt, 32, kWave);
    const float inv = 1.0f / den;
    const float c = -qt * inv * inv;
    if (!valid) continue;
    if (half == 0) c_out[((size_t)b * N + tok) * heads + h] = c;
#pragma unroll
    for (int rt = 0; rt < HM::RT; ++rt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int a0 = rt * 32 + 8 * g + 4 * half;
        if (a0 >= d) continue;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = acc[rt][4 * g + i] * inv + c * zs[a0 + i];
          o[i] = qv[rt][4 * g + i] > 0.0f ? v : 0.0f;
        }
        store4(dq_pre + row + a0, o);
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = ks * 16 + 8 * half;
      if (k >= d) continue;
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = (float)bf[ks][i] * inv;
      store8(g_out + row + k, o);
    }
  }
}

// Tiles per wave: one (so that a wave's loads never queue behind its own
// earlier stores) until the grid would pass about 4096 blocks.
static int head_tiles_per_wave(int B, int heads, int ntok) {
  const int tiles = (ntok + 31) / 32;
  const int pairs = B * heads;
  const int blocks_per_pair = std::max(1, 4096 / std::max(1, pairs));
  return std::max(1, (tiles + 4 * blocks_per_pair - 1) / (4 * blocks_per_pair));
}

#define EDIT_KS_SWITCH(KSV_MACRO)                                                                          \
  switch ((d + 15) / 16) {                                                                                 \
    KSV_MACRO(1) KSV_MACRO(2) KSV_MACRO(3) KSV_MACRO(4) KSV_MACRO(5) KSV_MACRO(6) KSV_MACRO(7) KSV_MACRO(8) \
    default: return hipErrorInvalidValue;                                                                  \
  }

template <typename T>
hipError_t launch_attn_bwd_q(const T* dy, const T* q, const float* S, const float* z, int B, int N, int heads, int d,
                             float eps, T* g, float* c, T* dq_pre, hipStream_t s) {
  if (d % 8 || d > 128 || N <= 0) return N <= 0 ? hipSuccess : hipErrorInvalidValue;
  const int tpw = head_tiles_per_wave(B, heads, N);
  dim3 grid(((N + 31) / 32 + 4 * tpw - 1) / (4 * tpw), heads, B);
#define EDIT_BQ_CASE(KSV)                                                                                       \
  case KSV:                                                                                                     \
    hipLaunchKernelGGL((attn_bwd_q_kernel<T, KSV>), grid, dim3(256), 0, s, dy, q, S, z, N, heads, d, eps, tpw, g, \
                       c, dq_pre);                                                                              \
    break;
  EDIT_KS_SWITCH(EDIT_BQ_CASE)
#undef EDIT_BQ_CASE
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// State backward (section "Linear-attention formula", S = sum K'^T V',
// z = sum K'): per compressed token j and head,
//   dK'_j = V'_j dS^T + dz, then the keys' ReLU (where K'_j > 0),
//   dV'_j = K'_j dS.
// Writes dkv [B][Nc][2C] in fp32: the keys' gradient before their ReLU | the
// values'. It stays fp32 because its sums over tokens cancel: moving every K'
// by one vector changes the outputs only through V'_j - y_i, a few percent of
// V', so the bias gradients sum terms ~25 times larger than the result, and a
// bf16 rounding of each term would leave errors of a few percent there.
// On the matrix cores: dK'^T = dS V'^T (A operand dS) and dV'^T = dS^T K'^T
// (A operand dS^T), 32 compressed tokens per wave.
// ---------------------------------------------------------------------------
template <typename T, int KS>
__global__ __launch_bounds__(256) void kv_bwd_kernel(const T* __restrict__ kc, const T* __restrict__ vc,
                                                     const float* __restrict__ dS, const float* __restrict__ dz,
                                                     int Nc, int heads, int d, int tiles_per_wave,
                                                     float* __restrict__ dkv) {
  using HM = HeadMat<T, KS>;
  using F = typename Frag<T>::type;
  __shared__ __attribute__((aligned(16))) T A1[HM::NC * HM::RT * 32 * HM::KP];   // dS
  __shared__ __attribute__((aligned(16))) T A2[HM::NC * HM::RT * 32 * HM::KP];   // dS^T
  __shared__ float zs[HM::RT * 32];
  const int h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63;
  const int C = heads * d, col = lane & 31, half = lane >> 5;
  const size_t bh = (size_t)b * heads + h;
  head_mat_fill<T, KS, false>(A1, dS + bh * d * d, d);
  head_mat_fill<T, KS, true>(A2, dS + bh * d * d, d);
  for (int i = threadIdx.x; i < HM::RT * 32; i += blockDim.x) zs[i] = i < d ? dz[bh * d + i] : 0.0f;
  __syncthreads();
  const int t0 = head_tile0(tiles_per_wave);
  for (int t = 0; t < tiles_per_wave; ++t) {
    const int tok0 = (t0 + t) * 32;
    if (tok0 >= Nc) break;
    const int tok = tok0 + col;
    const bool valid = tok < Nc;
    const size_t row = ((size_t)b * Nc + (valid ? tok : 0)) * C + (size_t)h * d;
    float* out = dkv + ((size_t)b * Nc + (valid ? tok : 0)) * 2 * C + (size_t)h * d;
    // Every load of the tile (V', K' as operands, K' for the ReLU mask) is
    // issued before its first store: a load queued behind a store waits for it.
    F bv[KS], bk[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = ks * 16 + 8 * half;
      bv[ks] = valid && k < d ? frag_ld(vc + row + k) : frag_zero<F>();
      bk[ks] = valid && k < d ? frag_ld(kc + row + k) : frag_zero<F>();
    }
    float kv[HM::RT][16];
#pragma unroll
    for (int rt = 0; rt < HM::RT; ++rt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int a0 = rt * 32 + 8 * g + 4 * half;
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (valid && a0 < d) load4(kc + row + a0, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) kv[rt][4 * g + i] = v[i];
      }
    f32x16 acc[HM::RT];
    // keys: dK'^T = dS V'^T, + dz, masked by K' > 0
    head_mat_apply<T, KS, HM::RT>(A1, bv, acc, lane);
    if (valid) {
#pragma unroll
      for (int rt = 0; rt < HM::RT; ++rt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int a0 = rt * 32 + 8 * g + 4 * half;
          if (a0 >= d) continue;
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = kv[rt][4 * g + i] > 0.0f ? acc[rt][4 * g + i] + zs[a0 + i] : 0.0f;
          store4(out + a0, o);
        }
    }
    // values: dV'^T = dS^T K'^T
    head_mat_apply<T, KS, HM::RT>(A2, bk, acc, lane);
    if (valid) {
#pragma unroll
      for (int rt = 0; rt < HM::RT; ++rt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n0 = rt * 32 + 8 * g + 4 * half;
          if (n0 >= d) continue;
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = acc[rt][4 * g + i];
          store4(out + C + n0, o);
        }
    }
  }
}

template <typename T>
hipError_t launch_kv_bwd(const T* kc, const T* vc, const float* dS, const float* dz, int B, int Nc, int heads,
                         int d, float* dkv, hipStream_t s) {
  if (d % 8 || d > 128 || Nc <= 0) return Nc <= 0 ? hipSuccess : hipErrorInvalidValue;
  const int tpw = head_tiles_per_wave(B, heads, Nc);
  dim3 grid(((Nc + 31) / 32 + 4 * tpw - 1) / (4 * tpw), heads, B);
#define EDIT_BKV_CASE(KSV)                                                                                        \
  case KSV:                                                                                                       \
    hipLaunchKernelGGL((kv_bwd_kernel<T, KSV>), grid, dim3(256), 0, s, kc, vc, dS, dz, Nc, heads, d, tpw, dkv); \
    break;
  EDIT_KS_SWITCH(EDIT_BKV_CASE)
#undef EDIT_BKV_CASE
  return hipGetLastError();
}
#undef EDIT_KS_SWITCH

// ---------------------------------------------------------------------------
// Depthwise 3x3 stride-2 backward (section "Spatial Compressor"), over the
// keys and values side by side (2C channels; taps dwk for channels < C, dwv
// above).
// ---------------------------------------------------------------------------

// Input gradient of the depthwise 3x3 stride-2 convs: din[y][x][c] = sum over the taps (ky, kx) with
// y + 1 - ky and x + 1 - kx even of dout[(y + 1 - ky) / 2][(x + 1 - kx) / 2][c] w[ky][kx][c]. A thread takes
// the 2x2 input pixels (2i + a, 2j + e) of one compressed position (i, j) and 8 channels: an even row uses tap
// row 1 at output row i, an odd one tap row 0 at i + 1 and tap row 2 at i (columns alike), so the four pixels
// read only dout at (i, j), (i + 1, j), (i, j + 1), (i + 1, j + 1) (zero past the grid), each once, with all
// nine taps' weights. Taps are added in (ky, kx) order.
template <typename T>
__global__ __launch_bounds__(256) void dw_bwd_input_kernel(const float* __restrict__ dout, int B, int H, int W, int C,
                                                           const T* __restrict__ dwk, const T* __restrict__ dwv,
                                                           T* __restrict__ din) {
  const int Hc = (H + 1) / 2, Wc = (W + 1) / 2;
  const int cpp = (2 * C) / 8;
  const long total = (long)B * Hc * Wc * cpp;
  const long idx = (long)xcd_swizzle(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int c8 = (int)(idx % cpp);
  const long q = idx / cpp;
  const int j = (int)(q % Wc), i = (int)((q / Wc) % Hc), b = (int)(q / ((long)Wc * Hc));
  const int ch2 = 8 * c8, ch = ch2 < C ? ch2 : ch2 - C;
  const T* w = ch2 < C ? dwk : dwv;
  // every load issued before any is used: the four output-gradient pixels (clamped, zeroed past the grid)
  // and the nine taps
  float g[2][2][8], wv[9][8];
#pragma unroll
  for (int dy = 0; dy < 2; ++dy)
#pragma unroll
    for (int dx = 0; dx < 2; ++dx) {
      const int yo = min(i + dy, Hc - 1), xo = min(j + dx, Wc - 1);
      load8(dout + (((size_t)b * Hc + yo) * Wc + xo) * 2 * C + ch2, g[dy][dx]);
    }
#pragma unroll
  for (int t = 0; t < 9; ++t) load8(w + t * C + ch, wv[t]);
  if (i + 1 >= Hc) {
#pragma unroll
    for (int k = 0; k < 8; ++k) g[1][0][k] = g[1][1][k] = 0.0f;
  }
  if (j + 1 >= Wc) {
#pragma unroll
    for (int k = 0; k < 8; ++k) g[0][1][k] = g[1][1][k] = 0.0f;
  }
  float o[2][2][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    o[0][0][k] = 0.0f + g[0][0][k] * wv[4][k];                                   // (1,1) at (i, j)
    o[0][1][k] = (0.0f + g[0][1][k] * wv[3][k]) + g[0][0][k] * wv[5][k];         // (1,0) at j+1, (1,2) at j
    o[1][0][k] = (0.0f + g[1][0][k] * wv[1][k]) + g[0][0][k] * wv[7][k];         // (0,1) at i+1, (2,1) at i
    o[1][1][k] = (((0.0f + g[1][1][k] * wv[0][k]) + g[1][0][k] * wv[2][k]) + g[0][1][k] * wv[6][k]) +
                 g[0][0][k] * wv[8][k];                                           // (0,0) (0,2) (2,0) (2,2)
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int y = 2 * i + a, x = 2 * j + e;
      if (y < H && x < W) store8(din + (((size_t)b * H + y) * W + x) * 2 * C + ch2, o[a][e]);
    }
}

template <typename T>
hipError_t launch_dw_bwd_input(const float* dout, int B, int H, int W, int C, const T* dwk, const T* dwv, T* din,
                               hipStream_t s) {
  const long total = (long)B * ((H + 1) / 2) * ((W + 1) / 2) * (2 * C / 8);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL((dw_bwd_input_kernel<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, dout, B, H, W,
                     C, dwk, dwv, din);
  return hipGetLastError();
}

// Weight gradient of the depthwise convs: for tap t = (ky, kx) and channel c,
//   dw[t][c] = sum_{b, y', x'} dout[y'][x'][c] in[2y'+ky-1][2x'+kx-1][c], db[c] = sum dout[y'][x'][c].
// Also the sum over all input pixels of the input gradient (the preceding
// Linear's bias gradient), from the fp32 dout rather than the rounded input
// gradient: every output pixel's gradient reaches the input through its taps
// that lie inside the image, so
//   sum_pixels din[c] = (sum_t w[t][c]) db[c] - sum_{y', x'} dout[y'][x'][c] sum_{t outside} w[t][c],
// where only border pixels have taps outside; the partials keep that last sum.
// A block takes 32 channel chunks x 8 pixel lanes over kDwPix output pixels;
// each thread keeps 11 x 8 sums, the 8 lanes are added through LDS, and the
// chunk's partial goes to partial[chunk][11][2C]; the chunks are then added
// in order.
constexpr int kDwPix = 32;    // output pixels per partial

template <typename T>
__global__ __launch_bounds__(256) void dw_bwd_weight_partial_kernel(const float* __restrict__ dout,
                                                                    const T* __restrict__ in, const T* __restrict__ dwk,
                                                                    const T* __restrict__ dwv, int B, int H, int W,
                                                                    int C, float* __restrict__ partial) {
  __shared__ float red[8][32 * 8 + 4];
  const int Hc = (H + 1) / 2, Wc = (W + 1) / 2, Pc = B * Hc * Wc;
  const int tid = threadIdx.x, cl = tid & 31, pl = tid >> 5;
  const int c8 = blockIdx.y * 32 + cl, chunk = blockIdx.x;
  const int cpp = (2 * C) / 8;
  const bool active = c8 < cpp;
  const int ch2 = 8 * c8;
  const T* wtap = ch2 < C ? dwk + ch2 : dwv + (ch2 - C);
  float acc[11][8];
#pragma unroll
  for (int t = 0; t < 11; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[t][i] = 0.0f;
  const int p0 = chunk * kDwPix;
  if (active) {
    for (int p = p0 + pl; p < min(Pc, p0 + kDwPix); p += 8) {
      const int xo = p % Wc, yo = (p / Wc) % Hc, b = p / (Wc * Hc);
      // the output gradient and all nine taps' inputs requested (clamped
      // in-image addresses) before any is used; taps outside add nothing
      float g[8], v[9][8];
      load8(dout + (size_t)p * 2 * C + ch2, g);
#pragma unroll
      for (int t = 0; t < 9; ++t) {
        const int yc = min(max(2 * yo + t / 3 - 1, 0), H - 1), xc = min(max(2 * xo + t % 3 - 1, 0), W - 1);
        load8(in + (((size_t)b * H + yc) * W + xc) * 2 * C + ch2, v[t]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[9][i] += g[i];
#pragma unroll
      for (int t = 0; t < 9; ++t) {
        const int yy = 2 * yo + t / 3 - 1, xx = 2 * xo + t % 3 - 1;
        if (yy >= 0 && yy < H && xx >= 0 && xx < W) {
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[t][i] += g[i] * v[t][i];
        }
      }
      // border pixels: dout times the taps that fall outside the image
      if (yo == 0 || 2 * yo + 1 >= H || xo == 0 || 2 * xo + 1 >= W) {
        float wo[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        for (int t = 0; t < 9; ++t) {
          const int yy = 2 * yo + t / 3 - 1, xx = 2 * xo + t % 3 - 1;
          if (yy < 0 || yy >= H || xx < 0 || xx >= W) {
            float wt[8];
            load8(wtap + t * C, wt);
#pragma unroll
            for (int i = 0; i < 8; ++i) wo[i] += wt[i];
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[10][i] += g[i] * wo[i];
      }
    }
  }
  float* out = partial + (size_t)chunk * 11 * 2 * C;
#pragma unroll
  for (int t = 0; t < 11; ++t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[pl][cl * 8 + i] = acc[t][i];
    __syncthreads();
    if (pl == 0 && active) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float s = 0.0f;
#pragma unroll
        for (int l = 0; l < 8; ++l) s += red[l][cl * 8 + i];
        out[(size_t)t * 2 * C + ch2 + i] = s;
      }
    }
    __syncthreads();
  }
}

// Sum the pixel-chunk partials; write dw_k, db_k (channels < C) and
// dw_v, db_v (taps stored [3][3][C] as the weights), and the input gradient's
// sums over pixels bk (channels < C) and bv: (sum_t w[t][c]) db[c] minus the
// border term, from the fp32 sums. A block takes 32 outputs; lane q of the 8
// lanes per output sums chunks q, q + 8, .. in order, then lane 0 adds the 8
// lane sums in order (a fixed order: the result is reproducible bit for bit).
template <typename T>
__global__ __launch_bounds__(256) void dw_bwd_weight_finalize_kernel(const float* __restrict__ partial, int nchunks,
                                                                     int C, const T* __restrict__ wk,
                                                                     const T* __restrict__ wv, T* __restrict__ dwk,
                                                                     T* __restrict__ dbk, T* __restrict__ dwv,
                                                                     T* __restrict__ dbv, T* __restrict__ bk,
                                                                     T* __restrict__ bv) {
  __shared__ float red[2][8][33];
  const int o = threadIdx.x & 31, q = threadIdx.x >> 5;
  const int i = blockIdx.x * 32 + o;
  const bool live = i < 10 * 2 * C;
  const int t = live ? i / (2 * C) : 0, c2 = live ? i - t * 2 * C : 0;
  float s = 0.0f, border = 0.0f;
  if (live) {
#pragma unroll 4
    for (int ch = q; ch < nchunks; ch += 8) {
      const float* pp = partial + (size_t)ch * 11 * 2 * C + c2;
      s += pp[(size_t)t * 2 * C];
      if (t == 9) border += pp[(size_t)10 * 2 * C];
    }
  }
  red[0][q][o] = s;
  red[1][q][o] = border;
  __syncthreads();
  if (q != 0 || !live) return;
  s = 0.0f;
  border = 0.0f;
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    s += red[0][l][o];
    border += red[1][l][o];
  }
  const bool k = c2 < C;
  const int c = k ? c2 : c2 - C;
  if (t < 9) {
    (k ? dwk : dwv)[t * C + c] = from_f32<T>(s);
    return;
  }
  (k ? dbk : dbv)[c] = from_f32<T>(s);
  const T* w = k ? wk : wv;
  float wsum = 0.0f;
#pragma unroll
  for (int tap = 0; tap < 9; ++tap) wsum += to_f32(w[tap * C + c]);
  (k ? bk : bv)[c] = from_f32<T>(wsum * s - border);
}

int dw_bwd_chunks(int B, int H, int W) {
  const int Pc = B * ((H + 1) / 2) * ((W + 1) / 2);
  return (Pc + kDwPix - 1) / kDwPix;
}

template <typename T>
hipError_t launch_dw_bwd_weight(const float* dout, const T* in, const T* wk, const T* wv, int B, int H, int W, int C,
                                float* partial, T* dwk, T* dbk, T* dwv, T* dbv, T* bk, T* bv, hipStream_t s) {
  const int nch = dw_bwd_chunks(B, H, W);
  dim3 grid(nch, (2 * C / 8 + 31) / 32);
  hipLaunchKernelGGL((dw_bwd_weight_partial_kernel<T>), grid, dim3(256), 0, s, dout, in, wk, wv, B, H, W, C,
                     partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dw_bwd_weight_finalize_kernel<T>), dim3((10 * 2 * C + 31) / 32), dim3(256), 0, s, partial,
                     nch, C, wk, wv, dwk, dbk, dwv, dbv, bk, bv);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// GroupNorm + LeakyReLU backward (section "ConvFusion"; GroupNorm over each
// sample's positions and the group's channels, LeakyReLU slope 0.01):
//   da = dact where act >= 0, 0.01 dact below (the sign of act is the sign
//   of its input); xn = (xc - mean) rstd;
//   dbeta[c] = sum da, dgamma[c] = sum da xn;
//   m1 = mean over (sample, group) of gamma da, m2 = mean of gamma da xn;
//   dxc = rstd (gamma da - m1 - xn m2).
// The partial kernel sums da and da xn per channel over 64-token chunks; the
// finalize adds the chunks in order (per sample) and forms dgamma, dbeta
// (summed over samples) and m1, m2 per (sample, group).
// ---------------------------------------------------------------------------
constexpr int kGnbRows = 128;
int gn_bwd_chunks(int N) { return (N + kGnbRows - 1) / kGnbRows; }

// One block per (128-token chunk, 256 channels, sample): 32 lanes of 8
// channels x 8 row lanes, the row lanes added through LDS.
template <typename T>
__global__ __launch_bounds__(256) void gn_bwd_partial_kernel(const T* __restrict__ dact, const T* __restrict__ act,
                                                             const T* __restrict__ xc, const float* __restrict__ stat,
                                                             int N, int C, int G, float* __restrict__ partial) {
  __shared__ float red[2][8][256];
  const int cg = threadIdx.x & 31, rl = threadIdx.x >> 5;
  const int chunk = blockIdx.x, b = blockIdx.z;
  const int c0 = (blockIdx.y * 32 + cg) * 8;
  float s1[8], s2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s1[i] = s2[i] = 0.0f;
  if (c0 < C) {
    const int cpg = C / G;
    float mean[8], rstd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = (c0 + i) / cpg;
      mean[i] = stat[((size_t)b * G + g) * 2];
      rstd[i] = stat[((size_t)b * G + g) * 2 + 1];
    }
    const int n1 = min(N, (chunk + 1) * kGnbRows);
    for (int n = chunk * kGnbRows + rl; n < n1; n += 8) {
      const size_t i0 = ((size_t)b * N + n) * C + c0;
      float a[8], da[8], x[8];
      load8(act + i0, a);
      load8(dact + i0, da);
      load8(xc + i0, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float dd = a[i] >= 0.0f ? da[i] : 0.01f * da[i];
        s1[i] += dd;
        s2[i] += dd * (x[i] - mean[i]) * rstd[i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    red[0][rl][cg * 8 + i] = s1[i];
    red[1][rl][cg * 8 + i] = s2[i];
  }
  __syncthreads();
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c < C) {
    float t1 = 0.0f, t2 = 0.0f;
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      t1 += red[0][l][threadIdx.x];
      t2 += red[1][l][threadIdx.x];
    }
    float* out = partial + (((size_t)b * gridDim.x + chunk) * C + c) * 2;
    out[0] = t1;
    out[1] = t2;
  }
}

// One block per (group, sample): threads (channel of the group, chunk lane)
// sum strided chunks, then each channel's lanes in order; per (sample,
// group) m1, m2; block (g, 0) also writes dgamma, dbeta of its channels,
// summed over the samples in order.
template <typename T>
__global__ __launch_bounds__(256) void gn_bwd_finalize_kernel(const float* __restrict__ partial, int nchunks, int B,
                                                              int N, int C, int G, const T* __restrict__ gamma,
                                                              float* __restrict__ m12, T* __restrict__ dgamma,
                                                              T* __restrict__ dbeta) {
  __shared__ float r1[256], r2[256], t1s[256], t2s[256];
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int cg = C / G, lanes = 256 / cg;
  const int ci = tid % cg, lane = tid / cg;
  auto chunk_sums = [&](int bb, float& a1, float& a2) {
    a1 = a2 = 0.0f;
    if (lane < lanes)
      for (int ch = lane; ch < nchunks; ch += lanes) {
        const float* p = partial + (((size_t)bb * nchunks + ch) * C + g * cg + ci) * 2;
        a1 += p[0];
        a2 += p[1];
      }
  };
  float a1, a2;
  chunk_sums(b, a1, a2);
  r1[tid] = a1;
  r2[tid] = a2;
  __syncthreads();
  float s1 = 0.0f, s2 = 0.0f;     // per channel ci (threads tid < cg)
  if (tid < cg)
    for (int l = 0; l < lanes; ++l) {
      s1 += r1[l * cg + tid];
      s2 += r2[l * cg + tid];
    }
  __syncthreads();
  if (tid < cg) {
    const float gm = to_f32(gamma[g * cg + tid]);
    t1s[tid] = gm * s1;
    t2s[tid] = gm * s2;
  }
  __syncthreads();
  if (tid == 0) {
    float q1 = 0.0f, q2 = 0.0f;
    for (int i = 0; i < cg; ++i) { q1 += t1s[i]; q2 += t2s[i]; }
    const float inv = 1.0f / ((float)N * (float)cg);
    m12[((size_t)b * G + g) * 2] = q1 * inv;
    m12[((size_t)b * G + g) * 2 + 1] = q2 * inv;
  }
  if (b != 0) return;
  // dgamma, dbeta over the samples, in sample order
  float d1 = s1, d2 = s2;
  for (int bb = 1; bb < B; ++bb) {
    __syncthreads();
    chunk_sums(bb, a1, a2);
    r1[tid] = a1;
    r2[tid] = a2;
    __syncthreads();
    if (tid < cg)
      for (int l = 0; l < lanes; ++l) {
        d1 += r1[l * cg + tid];
        d2 += r2[l * cg + tid];
      }
  }
  if (tid < cg) {
    dbeta[g * cg + tid] = from_f32<T>(d1);
    dgamma[g * cg + tid] = from_f32<T>(d2);
  }
}

// dxc[m][c] (row stride ldo; channels C .. ldo - 1 written as zeros), eight
// channels per thread.
template <typename T>
__global__ __launch_bounds__(256) void gn_bwd_apply_kernel(const T* __restrict__ dact, const T* __restrict__ act,
                                                           const T* __restrict__ xc, const float* __restrict__ stat,
                                                           const float* __restrict__ m12,
                                                           const T* __restrict__ gamma, int N, int C, int G, long rows,
                                                           int ldo, T* __restrict__ dxc) {
  const int cpr = ldo / 8;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cpr) return;
  const long m = i / cpr;
  const int c0 = (int)(i - m * cpr) * 8;
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c0 < C) {
    const int b = (int)(m / N), cpg = C / G;
    float a[8], da[8], x[8];
    load8(act + m * C + c0, a);
    load8(dact + m * C + c0, da);
    load8(xc + m * C + c0, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int g = (c0 + k) / cpg;
      const float mean = stat[((size_t)b * G + g) * 2], rstd = stat[((size_t)b * G + g) * 2 + 1];
      const float m1 = m12[((size_t)b * G + g) * 2], m2 = m12[((size_t)b * G + g) * 2 + 1];
      const float d = a[k] >= 0.0f ? da[k] : 0.01f * da[k];
      const float xn = (x[k] - mean) * rstd;
      o[k] = rstd * (to_f32(gamma[c0 + k]) * d - m1 - xn * m2);
    }
  }
  store8(dxc + m * ldo + c0, o);
}

template <typename T>
hipError_t launch_gn_bwd(const T* dact, const T* act, const T* xc, const float* stat, const T* gamma, int B, int N,
                         int C, int G, float* partial, float* m12, T* dgamma, T* dbeta, T* dxc, int lddxc,
                         hipStream_t s) {
  if (C / G > 256 || C % 8 != 0 || lddxc < C || lddxc % 8 != 0) return hipErrorInvalidValue;
  const int nch = gn_bwd_chunks(N);
  hipLaunchKernelGGL((gn_bwd_partial_kernel<T>), dim3(nch, (C + 255) / 256, B), dim3(256), 0, s, dact, act, xc, stat,
                     N, C, G, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gn_bwd_finalize_kernel<T>), dim3(G, B), dim3(256), 0, s, partial, nch, B, N, C, G, gamma, m12,
                     dgamma, dbeta);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long rows = (long)B * N, total = rows * (lddxc / 8);
  hipLaunchKernelGGL((gn_bwd_apply_kernel<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, dact, act, xc,
                     stat, m12, gamma, N, C, G, rows, lddxc, dxc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small fp32 product for the folded query weights' gradient:
//   out[i][j] = add[i][j] + ru[i] rv[j] + sum_k A[i][k] B[j][k]
// (A fp32 [M][lda], B [N][ldb], both K-contiguous), on the fp32 matrix cores
// (32x32x2 steps). A block of four waves takes a 64 x 64 output tile, each
// wave 32 x 32; K goes through LDS in chunks of 32 (B converted to fp32 as it
// is staged), rows padded to 33 floats so that the 32 rows of a fragment read
// fall in distinct banks. Lane l supplies row l % 32 of A and column l % 32
// of B at the same k, so the product is the full fp32 sum over k.
// ---------------------------------------------------------------------------
constexpr int kSmKc = 32;

template <typename TB, typename TO>
__global__ __launch_bounds__(256) void small_nt_kernel(int M, int N, int K, const float* __restrict__ A, int lda,
                                                       const TB* __restrict__ Bm, int ldb,
                                                       const float* __restrict__ add, int ldadd,
                                                       const float* __restrict__ ru, const TB* __restrict__ rv,
                                                       TO* __restrict__ out, int ldo) {
  __shared__ float As[64][kSmKc + 1];
  __shared__ float Bs[64][kSmKc + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
  const int fr = lane & 31, fk = lane >> 5;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  // A: 64 rows x 8 float4 along K (two per thread); B: 64 rows x 4 groups of 8 along K (one per thread); zero
  // past M, N and K. A chunk's loads are issued before the previous chunk's products, so their latency overlaps.
  f32x4 av[2];
  float bv[8];
  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = tid + 256 * h, r = e >> 3, k = k0 + (e & 7) * 4;
      av[h] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (i0 + r < M && k < K) av[h] = *reinterpret_cast<const f32x4*>(A + (size_t)(i0 + r) * lda + k);
    }
    const int r = tid >> 2, k = k0 + (tid & 3) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) bv[q] = 0.0f;
    if (j0 + r < N && k < K) load8(Bm + (size_t)(j0 + r) * ldb + k, bv);
  };
  load_chunk(0);
  for (int k0 = 0; k0 < K; k0 += kSmKc) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = tid + 256 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) As[e >> 3][(e & 7) * 4 + q] = av[h][q];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) Bs[tid >> 2][(tid & 3) * 8 + q] = bv[q];
    __syncthreads();
    if (k0 + kSmKc < K) load_chunk(k0 + kSmKc);
#pragma unroll
    for (int kk = 0; kk < kSmKc; kk += 2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[wr + fr][kk + fk], Bs[wc + fr][kk + fk], acc, 0, 0, 0);
    __syncthreads();
  }
  // accumulator r of lane l: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32 of the wave's tile
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + wr + 8 * (r >> 2) + 4 * fk + (r & 3), j = j0 + wc + fr;
    if (i < M && j < N) {
      float v = acc[r];
      if (add) v += add[(size_t)i * ldadd + j];
      if (ru) v += ru[i] * to_f32(rv[j]);
      out[(size_t)i * ldo + j] = from_f32<TO>(v);
    }
  }
}

template <typename TB, typename TO>
hipError_t launch_small_nt(int M, int N, int K, const float* A, int lda, const TB* Bm, int ldb, const float* add,
                           int ldadd, TO* out, int ldo, hipStream_t s, const float* ru, const TB* rv) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % 8 || lda % 4 || ldb % 8) return hipErrorInvalidValue;
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL((small_nt_kernel<TB, TO>), grid, dim3(256), 0, s, M, N, K, A, lda, Bm, ldb, add, ldadd, ru, rv,
                     out, ldo);
  return hipGetLastError();
}


// fp32 rows to one output, bf16 rows to the other (one launch for two weight gradients)
template hipError_t launch_splitk_reduce<float, bf16>(const float*, int, long long, int, int, float*, int, hipStream_t,
                                                      int, int, bf16*, int, const float*);

#define EDIT_INST(T)                                                                                               \
  template hipError_t launch_transpose<T>(const T*, int, int, int, T*, int, hipStream_t, int, int, long, long,    \
                                          float*, const T*);                                                     \
  template hipError_t launch_shift_transpose9<T>(const T*, int, int, int, int, int, T*, int, hipStream_t, float*); \
  template hipError_t launch_colsum_finalize<T>(const float*, int, int, T*, hipStream_t, float*, T*, int);        \
  template hipError_t launch_zero<T>(T*, long, hipStream_t);                                                       \
  template hipError_t launch_splitk_reduce<T, T>(const float*, int, long long, int, int, T*, int, hipStream_t,   \
                                                 int, int, T*, int, const T*);                                    \
  template hipError_t launch_attn_bwd_q<T>(const T*, const T*, const float*, const float*, int, int, int, int,     \
                                           float, T*, float*, T*, hipStream_t);                                    \
  template hipError_t launch_kv_bwd<T>(const T*, const T*, const float*, const float*, int, int, int, int, float*, \
                                       hipStream_t);                                                               \
  template hipError_t launch_dw_bwd_input<T>(const float*, int, int, int, int, const T*, const T*, T*, hipStream_t); \
  template hipError_t launch_dw_bwd_weight<T>(const float*, const T*, const T*, const T*, int, int, int, int, float*, \
                                              T*, T*, T*, T*, T*, T*, hipStream_t);                                \
  template hipError_t launch_gn_bwd<T>(const T*, const T*, const T*, const float*, const T*, int, int, int, int,   \
                                       float*, float*, T*, T*, T*, int, hipStream_t);
EDIT_INST(bf16)
EDIT_INST(float)
#undef EDIT_INST
template hipError_t launch_small_nt<bf16, bf16>(int, int, int, const float*, int, const bf16*, int, const float*, int,
                                               bf16*, int, hipStream_t, const float*, const bf16*);
template hipError_t launch_small_nt<float, float>(int, int, int, const float*, int, const float*, int, const float*,
                                                  int, float*, int, hipStream_t, const float*, const float*);

}  // namespace edit
