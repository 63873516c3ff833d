// Backward pass of the EDiT layer on gfx950: the kernels that are not GEMMs.
//
// Page "EDiT: Efficient Diffusion Transformers with Linear Compressed
// Attention" (ICCV 2025 notes): the layer is trained by distillation
// (section "Distillation"), which needs the gradient of every forward step
// (sections "ConvFusion", "Spatial Compressor", "Linear-attention formula").
// Each kernel below is the chain rule of one forward step; the GEMM-shaped
// products run on the GEMM kernels (with transposed operands where the
// contraction is over tokens). Every reduction sums in a fixed order, so
// gradients are bit-for-bit reproducible.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace edit {

// ---------------------------------------------------------------------------
// Transpose: out[c][r] = in[r][c] through a 64 x 65 LDS tile. With a shift
// (the 3x3 conv's tap (ky, kx)): out[c][m] = in[m - off][c] where the pixel
// of m - off lies inside its image and reads m through that tap, else 0;
// off = (ky - 1) W + (kx - 1). Rows are tokens b*H*W + y*W + x. Output
// columns rows .. rows_pad - 1 (the row padding of out) are written as zeros.
// ---------------------------------------------------------------------------
template <typename T, bool SHIFT>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, int rows, int rows_pad, int cols,
                                                        int ldi, T* __restrict__ out, int ldo, int H, int W, int ky,
                                                        int kx) {
  // 64 x 64 tile; every global access is 16 bytes (EPC elements): a load
  // takes EPC consecutive columns of one row, a store EPC consecutive rows
  // of one column. cols, ldi, ldo and rows_pad are multiples of EPC.
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int VPR = 64 / EPC;                 // 16-byte vectors per 64-element tile row
  typedef uint32_t u32x4t __attribute__((ext_vector_type(4)));
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
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
                            int rows_pad) {
  if (rows_pad < rows) rows_pad = rows;
  if (rows <= 0 || cols <= 0) return hipSuccess;
  constexpr int EPC = 16 / (int)sizeof(T);
  if (cols % EPC || ldi % EPC || ldo % EPC || rows_pad % EPC) return hipErrorInvalidValue;
  dim3 grid((cols + 63) / 64, (rows_pad + 63) / 64);
  hipLaunchKernelGGL((transpose_kernel<T, false>), grid, dim3(256), 0, s, in, rows, rows_pad, cols, ldi, out, ldo, 1,
                     1, 1, 1);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_shift_transpose(const T* in, int B, int H, int W, int cols, T* out, int ldo, int ky, int kx,
                                  hipStream_t s) {
  const int rows = B * H * W;
  if (rows <= 0 || cols <= 0) return hipSuccess;
  constexpr int EPC = 16 / (int)sizeof(T);
  if (cols % EPC || ldo % EPC || ldo < rows) return hipErrorInvalidValue;
  dim3 grid((cols + 63) / 64, (ldo + 63) / 64);
  hipLaunchKernelGGL((transpose_kernel<T, true>), grid, dim3(256), 0, s, in, rows, ldo, cols, cols, out, ldo, H, W,
                     ky, kx);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Column sums (bias gradients): out[c] = sum_r in[r][c]. A block sums 256
// rows of 256 columns: 32 lanes of 8 columns (16-byte loads) x 8 row lanes,
// the row lanes added through LDS (partial[chunk][c]); then the chunks in
// order. cols and ld are multiples of 8.
// ---------------------------------------------------------------------------
constexpr int kColChunk = 256;
int colsum_chunks(int rows) { return (rows + kColChunk - 1) / kColChunk; }

template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T* __restrict__ in, int rows, int cols, int ld,
                                                             float* __restrict__ partial) {
  __shared__ float red[8][256];
  const int cg = threadIdx.x & 31, rl = threadIdx.x >> 5, ch = blockIdx.y;
  const int c0 = (blockIdx.x * 32 + cg) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  if (c0 < cols) {
    const int r1 = min(rows, (ch + 1) * kColChunk);
#pragma unroll 8
    for (int r = ch * kColChunk + rl; r < r1; r += 8) {
      float v[8];
      load8(in + (size_t)r * ld + c0, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rl][cg * 8 + i] = acc[i];
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < cols) {
    float t = 0.0f;
#pragma unroll
    for (int l = 0; l < 8; ++l) t += red[l][threadIdx.x];
    partial[(size_t)ch * cols + c] = t;
  }
}

// Writes out[c] (T) and, when given, out32[c] (the same sum in f32).
template <typename T>
__global__ __launch_bounds__(256) void colsum_finalize_kernel(const float* __restrict__ partial, int nchunks,
                                                              int cols, T* __restrict__ out,
                                                              float* __restrict__ out32) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  float s = 0.0f;
  for (int ch = 0; ch < nchunks; ++ch) s += partial[(size_t)ch * cols + c];
  out[c] = from_f32<T>(s);
  if (out32) out32[c] = s;
}

template <typename T>
hipError_t launch_colsum(const T* in, int rows, int cols, int ld, float* partial, T* out, hipStream_t s,
                         float* out32) {
  if (cols <= 0) return hipSuccess;
  const int nch = colsum_chunks(rows);
  hipLaunchKernelGGL((colsum_partial_kernel<T>), dim3((cols + 255) / 256, nch), dim3(256), 0, s, in, rows, cols, ld,
                     partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((colsum_finalize_kernel<T>), dim3((cols + 255) / 256), dim3(256), 0, s, partial, nch, cols, out,
                     out32);
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
// Split-K reduction: out[r][c] = sum_s part[s][r][c] (ld cols), s in order.
// ---------------------------------------------------------------------------
template <typename O>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S,
                                                            long long stride, int rows, int cols,
                                                            O* __restrict__ out, int ldo) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)rows * cols) return;
  const int r = (int)(i / cols), c = (int)(i - (long long)r * cols);
  float v = 0.0f;
  for (int s = 0; s < S; ++s) v += part[(size_t)s * stride + i];
  out[(size_t)r * ldo + c] = from_f32<O>(v);
}

template <typename O>
hipError_t launch_splitk_reduce(const float* part, int S, long long stride, int rows, int cols, O* out, int ldo,
                                hipStream_t s) {
  const long long n = (long long)rows * cols;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((splitk_reduce_kernel<O>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, S, stride,
                     rows, cols, out, ldo);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Linear-attention backward, query side. Per token i and head (section
// "Linear-attention formula", y = q S / (q . z + eps)):
//   den = q . z + eps, t = S dy (t[a] = sum_n S[a][n] dy[n]),
//   dy . y = q . t / den, c = -(dy . y) / den, g = dy / den,
//   dq = t / den + c z, then the outer ReLU of the queries: dq_pre = dq where q > 0.
// dy . y is formed from q, S and dy in fp32 rather than from the stored y:
// the two terms of dq nearly cancel (y does not change when q is scaled), so
// y's rounding would be amplified. One thread per token (256 per block, one
// head); the token's dy in registers, S row-major in LDS (a row of S is read
// as broadcast 16-byte words); t is formed twice, eight outputs at a time
// (once for dy . y, once for dq). g (T) and c (f32) are kept for the state
// gradient dS = sum q^T g, dz = sum c q.
// ---------------------------------------------------------------------------
constexpr int kBwdTok = 256;

// acc[i] += sum_n r[n] M[(a0 + i) * d + n], i < 8 (M row-major in LDS).
template <int d>
__device__ __forceinline__ void rows8_dot(const float* M, int a0, const float (&r)[d], float (&acc)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float* row = M + (a0 + i) * d;
    float s = 0.0f;
#pragma unroll
    for (int n = 0; n < d; n += 4) {
      const f32x4 m = *reinterpret_cast<const f32x4*>(row + n);
      s += r[n] * m[0] + r[n + 1] * m[1] + r[n + 2] * m[2] + r[n + 3] * m[3];
    }
    acc[i] += s;
  }
}

template <typename T, int DC>
__global__ __launch_bounds__(kBwdTok) void attn_bwd_q_kernel(const T* __restrict__ dy, const T* __restrict__ q,
                                                             const float* __restrict__ S,
                                                             const float* __restrict__ z, int N, int heads,
                                                             float eps, T* __restrict__ g_out,
                                                             float* __restrict__ c_out, T* __restrict__ dq_pre) {
  constexpr int d = 8 * DC;
  __shared__ __attribute__((aligned(16))) float Ss[d * d];
  __shared__ float zs[d];
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int C = heads * d;
  const size_t bh = (size_t)b * heads + h;
  for (int i = tid; i < d * d; i += kBwdTok) Ss[i] = S[bh * d * d + i];
  for (int i = tid; i < d; i += kBwdTok) zs[i] = z[bh * d + i];
  __syncthreads();
  const int tok = blockIdx.x * kBwdTok + tid;
  if (tok >= N) return;
  const size_t row = ((size_t)b * N + tok) * C + (size_t)h * d;
  float dv[d];
  float den = eps;
#pragma unroll
  for (int c8 = 0; c8 < DC; ++c8) {
    float qv[8], v[8];
    load8(q + row + 8 * c8, qv);
    load8(dy + row + 8 * c8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      den += qv[i] * zs[8 * c8 + i];
      dv[8 * c8 + i] = v[i];
    }
  }
  const float inv = 1.0f / den;
  float qt = 0.0f;
#pragma unroll 1
  for (int a0 = 0; a0 < d; a0 += 8) {
    float t[8] = {0, 0, 0, 0, 0, 0, 0, 0}, qv[8];
    rows8_dot<d>(Ss, a0, dv, t);
    load8(q + row + a0, qv);
#pragma unroll
    for (int i = 0; i < 8; ++i) qt += qv[i] * t[i];
  }
  const float c = -qt * inv * inv;
  c_out[((size_t)b * N + tok) * heads + h] = c;
#pragma unroll
  for (int c8 = 0; c8 < DC; ++c8) {
    float go[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) go[i] = dv[8 * c8 + i] * inv;
    store8(g_out + row + 8 * c8, go);
  }
#pragma unroll 1
  for (int a0 = 0; a0 < d; a0 += 8) {
    float t[8] = {0, 0, 0, 0, 0, 0, 0, 0}, qv[8], o[8];
    rows8_dot<d>(Ss, a0, dv, t);
    load8(q + row + a0, qv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = t[i] * inv + c * zs[a0 + i];
      o[i] = qv[i] > 0.0f ? v : 0.0f;
    }
    store8(dq_pre + row + a0, o);
  }
}

template <typename T>
hipError_t launch_attn_bwd_q(const T* dy, const T* q, const float* S, const float* z, int B, int N, int heads, int d,
                             float eps, T* g, float* c, T* dq_pre, hipStream_t s) {
  dim3 grid((N + kBwdTok - 1) / kBwdTok, heads, B);
  switch (d / 8) {
#define EDIT_BQ_CASE(DCV)                                                                                       \
  case DCV:                                                                                                     \
    hipLaunchKernelGGL((attn_bwd_q_kernel<T, DCV>), grid, dim3(kBwdTok), 0, s, dy, q, S, z, N, heads, eps, g, c, \
                       dq_pre);                                                                                 \
    break;
    EDIT_BQ_CASE(1) EDIT_BQ_CASE(2) EDIT_BQ_CASE(3) EDIT_BQ_CASE(4) EDIT_BQ_CASE(5) EDIT_BQ_CASE(6)
    EDIT_BQ_CASE(7) EDIT_BQ_CASE(8) EDIT_BQ_CASE(9) EDIT_BQ_CASE(10) EDIT_BQ_CASE(11) EDIT_BQ_CASE(12)
    EDIT_BQ_CASE(13) EDIT_BQ_CASE(14) EDIT_BQ_CASE(15) EDIT_BQ_CASE(16)
#undef EDIT_BQ_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// State backward (section "Linear-attention formula", S = sum K'^T V',
// z = sum K'): per compressed token j and head,
//   dK'_j = V'_j dS^T + dz, then the keys' ReLU (where K'_j > 0),
//   dV'_j = K'_j dS.
// Writes dkv [B][Nc][2C]: the keys' gradient before their ReLU | the values'.
// One thread per token, its V' and K' rows in registers; dS and dS^T
// row-major in LDS, eight outputs at a time.
// ---------------------------------------------------------------------------
template <typename T, int DC>
__global__ __launch_bounds__(kBwdTok) void kv_bwd_kernel(const T* __restrict__ kc, const T* __restrict__ vc,
                                                         const float* __restrict__ dS, const float* __restrict__ dz,
                                                         int Nc, int heads, T* __restrict__ dkv) {
  constexpr int d = 8 * DC;
  __shared__ __attribute__((aligned(16))) float Ss[d * d];    // dS[a][n]
  __shared__ __attribute__((aligned(16))) float St[d * d];    // dS^T: St[n][a] = dS[a][n]
  __shared__ float zs[d];
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int C = heads * d;
  const size_t bh = (size_t)b * heads + h;
  for (int i = tid; i < d * d; i += kBwdTok) {
    const float v = dS[bh * d * d + i];
    const int a = i / d, n = i - a * d;
    Ss[i] = v;
    St[n * d + a] = v;
  }
  for (int i = tid; i < d; i += kBwdTok) zs[i] = dz[bh * d + i];
  __syncthreads();
  const int tok = blockIdx.x * kBwdTok + tid;
  if (tok >= Nc) return;
  const size_t row = ((size_t)b * Nc + tok) * C + (size_t)h * d;
  T* out = dkv + ((size_t)b * Nc + tok) * 2 * C + (size_t)h * d;
  float r[d];
  // keys: dK'[a] = sum_n dS[a][n] V'[n] + dz[a], masked by K' > 0
#pragma unroll
  for (int c8 = 0; c8 < DC; ++c8) {
    float v[8];
    load8(vc + row + 8 * c8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[8 * c8 + i] = v[i];
  }
#pragma unroll 1
  for (int a0 = 0; a0 < d; a0 += 8) {
    float acc[8], kv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = zs[a0 + i];
    rows8_dot<d>(Ss, a0, r, acc);
    load8(kc + row + a0, kv);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = kv[i] > 0.0f ? acc[i] : 0.0f;
    store8(out + a0, acc);
  }
  // values: dV'[n] = sum_m K'[m] dS[m][n] = (dS^T K')[n]
#pragma unroll
  for (int c8 = 0; c8 < DC; ++c8) {
    float k[8];
    load8(kc + row + 8 * c8, k);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[8 * c8 + i] = k[i];
  }
#pragma unroll 1
  for (int n0 = 0; n0 < d; n0 += 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    rows8_dot<d>(St, n0, r, acc);
    store8(out + C + n0, acc);
  }
}

template <typename T>
hipError_t launch_kv_bwd(const T* kc, const T* vc, const float* dS, const float* dz, int B, int Nc, int heads,
                         int d, T* dkv, hipStream_t s) {
  dim3 grid((Nc + kBwdTok - 1) / kBwdTok, heads, B);
  switch (d / 8) {
#define EDIT_BKV_CASE(DCV)                                                                                  \
  case DCV:                                                                                                 \
    hipLaunchKernelGGL((kv_bwd_kernel<T, DCV>), grid, dim3(kBwdTok), 0, s, kc, vc, dS, dz, Nc, heads, dkv); \
    break;
    EDIT_BKV_CASE(1) EDIT_BKV_CASE(2) EDIT_BKV_CASE(3) EDIT_BKV_CASE(4) EDIT_BKV_CASE(5) EDIT_BKV_CASE(6)
    EDIT_BKV_CASE(7) EDIT_BKV_CASE(8) EDIT_BKV_CASE(9) EDIT_BKV_CASE(10) EDIT_BKV_CASE(11) EDIT_BKV_CASE(12)
    EDIT_BKV_CASE(13) EDIT_BKV_CASE(14) EDIT_BKV_CASE(15) EDIT_BKV_CASE(16)
#undef EDIT_BKV_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Depthwise 3x3 stride-2 backward (section "Spatial Compressor"), over the
// keys and values side by side (2C channels; taps dwk for channels < C, dwv
// above). Input gradient: input pixel (y, x) got tap (ky, kx) of output
// (y', x') when y = 2y' + ky - 1 and x = 2x' + kx - 1, so
//   d_in[y][x][c] = sum over those taps of dout[y'][x'][c] w[ky][kx][c]
// (taps visited in (ky, kx) order). One thread per pixel and 8 channels.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dw_bwd_input_kernel(const T* __restrict__ dout, int B, int H, int W, int C,
                                                           const T* __restrict__ dwk, const T* __restrict__ dwv,
                                                           T* __restrict__ din) {
  const int Hc = (H + 1) / 2, Wc = (W + 1) / 2;
  const int cpp = (2 * C) / 8;
  const long total = (long)B * H * W * cpp;
  const long idx = (long)xcd_swizzle(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int c8 = (int)(idx % cpp);
  const long pix = idx / cpp;
  const int x = (int)(pix % W), y = (int)((pix / W) % H), b = (int)(pix / ((long)W * H));
  const int ch2 = 8 * c8, ch = ch2 < C ? ch2 : ch2 - C;
  const T* w = ch2 < C ? dwk : dwv;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int ky = 0; ky < 3; ++ky) {
    const int yy = y + 1 - ky;                 // = 2 y'
    if (yy < 0 || (yy & 1) || (yy >> 1) >= Hc) continue;
#pragma unroll
    for (int kx = 0; kx < 3; ++kx) {
      const int xx = x + 1 - kx;
      if (xx < 0 || (xx & 1) || (xx >> 1) >= Wc) continue;
      float g[8], wv[8];
      load8(dout + (((size_t)b * Hc + (yy >> 1)) * Wc + (xx >> 1)) * 2 * C + ch2, g);
      load8(w + (ky * 3 + kx) * C + ch, wv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += g[i] * wv[i];
    }
  }
  store8(din + (size_t)pix * 2 * C + ch2, acc);
}

template <typename T>
hipError_t launch_dw_bwd_input(const T* dout, int B, int H, int W, int C, const T* dwk, const T* dwv, T* din,
                               hipStream_t s) {
  const long total = (long)B * H * W * (2 * C / 8);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL((dw_bwd_input_kernel<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, dout, B, H, W,
                     C, dwk, dwv, din);
  return hipGetLastError();
}

// Weight gradient of the depthwise convs: for tap t = (ky, kx) and channel c,
//   dw[t][c] = sum_{b, y', x'} dout[y'][x'][c] in[2y'+ky-1][2x'+kx-1][c], db[c] = sum dout[y'][x'][c].
// A block takes 32 channel chunks x 8 pixel lanes over kDwPix output pixels;
// each thread keeps 10 x 8 sums, the 8 lanes are added through LDS, and the
// chunk's partial goes to partial[chunk][10][2C]; the chunks are then added
// in order.
constexpr int kDwPix = 128;   // output pixels per partial

template <typename T>
__global__ __launch_bounds__(256) void dw_bwd_weight_partial_kernel(const T* __restrict__ dout,
                                                                    const T* __restrict__ in, int B, int H, int W,
                                                                    int C, float* __restrict__ partial) {
  __shared__ float red[8][32 * 8 + 4];
  const int Hc = (H + 1) / 2, Wc = (W + 1) / 2, Pc = B * Hc * Wc;
  const int tid = threadIdx.x, cl = tid & 31, pl = tid >> 5;
  const int c8 = blockIdx.y * 32 + cl, chunk = blockIdx.x;
  const int cpp = (2 * C) / 8;
  const bool active = c8 < cpp;
  const int ch2 = 8 * c8;
  float acc[10][8];
#pragma unroll
  for (int t = 0; t < 10; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[t][i] = 0.0f;
  const int p0 = chunk * kDwPix;
  if (active) {
    for (int p = p0 + pl; p < min(Pc, p0 + kDwPix); p += 8) {
      const int xo = p % Wc, yo = (p / Wc) % Hc, b = p / (Wc * Hc);
      float g[8];
      load8(dout + (size_t)p * 2 * C + ch2, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[9][i] += g[i];
#pragma unroll
      for (int ky = 0; ky < 3; ++ky) {
        const int yy = 2 * yo + ky - 1;
        if (yy < 0 || yy >= H) continue;
#pragma unroll
        for (int kx = 0; kx < 3; ++kx) {
          const int xx = 2 * xo + kx - 1;
          if (xx < 0 || xx >= W) continue;
          float v[8];
          load8(in + (((size_t)b * H + yy) * W + xx) * 2 * C + ch2, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[ky * 3 + kx][i] += g[i] * v[i];
        }
      }
    }
  }
  float* out = partial + (size_t)chunk * 10 * 2 * C;
#pragma unroll
  for (int t = 0; t < 10; ++t) {
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

// Sum the pixel-chunk partials in order; write dw_k, db_k (channels < C) and
// dw_v, db_v. Taps are stored [3][3][C] as the weights.
template <typename T>
__global__ __launch_bounds__(256) void dw_bwd_weight_finalize_kernel(const float* __restrict__ partial, int nchunks,
                                                                     int C, T* __restrict__ dwk, T* __restrict__ dbk,
                                                                     T* __restrict__ dwv, T* __restrict__ dbv) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= 10 * 2 * C) return;
  const int t = i / (2 * C), c2 = i - t * 2 * C;
  float s = 0.0f;
  for (int ch = 0; ch < nchunks; ++ch) s += partial[(size_t)ch * 10 * 2 * C + i];
  const bool k = c2 < C;
  const int c = k ? c2 : c2 - C;
  if (t < 9) (k ? dwk : dwv)[t * C + c] = from_f32<T>(s);
  else (k ? dbk : dbv)[c] = from_f32<T>(s);
}

int dw_bwd_chunks(int B, int H, int W) {
  const int Pc = B * ((H + 1) / 2) * ((W + 1) / 2);
  return (Pc + kDwPix - 1) / kDwPix;
}

template <typename T>
hipError_t launch_dw_bwd_weight(const T* dout, const T* in, int B, int H, int W, int C, float* partial, T* dwk,
                                T* dbk, T* dwv, T* dbv, hipStream_t s) {
  const int nch = dw_bwd_chunks(B, H, W);
  dim3 grid(nch, (2 * C / 8 + 31) / 32);
  hipLaunchKernelGGL((dw_bwd_weight_partial_kernel<T>), grid, dim3(256), 0, s, dout, in, B, H, W, C, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dw_bwd_weight_finalize_kernel<T>), dim3((10 * 2 * C + 255) / 256), dim3(256), 0, s, partial,
                     nch, C, dwk, dbk, dwv, dbv);
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

template <typename T>
__global__ __launch_bounds__(256) void gn_bwd_apply_kernel(const T* __restrict__ dact, const T* __restrict__ act,
                                                           const T* __restrict__ xc, const float* __restrict__ stat,
                                                           const float* __restrict__ m12,
                                                           const T* __restrict__ gamma, int N, int C, int G,
                                                           long total, T* __restrict__ dxc) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int c = (int)(i % C);
  const int b = (int)(i / ((long)N * C));
  const int g = c / (C / G);
  const float mean = stat[((size_t)b * G + g) * 2], rstd = stat[((size_t)b * G + g) * 2 + 1];
  const float m1 = m12[((size_t)b * G + g) * 2], m2 = m12[((size_t)b * G + g) * 2 + 1];
  const float a = to_f32(act[i]), da0 = to_f32(dact[i]);
  const float da = a >= 0.0f ? da0 : 0.01f * da0;
  const float xn = (to_f32(xc[i]) - mean) * rstd;
  dxc[i] = from_f32<T>(rstd * (to_f32(gamma[c]) * da - m1 - xn * m2));
}

template <typename T>
hipError_t launch_gn_bwd(const T* dact, const T* act, const T* xc, const float* stat, const T* gamma, int B, int N,
                         int C, int G, float* partial, float* m12, T* dgamma, T* dbeta, T* dxc, hipStream_t s) {
  if (C / G > 256 || C % 8 != 0) return hipErrorInvalidValue;
  const int nch = gn_bwd_chunks(N);
  hipLaunchKernelGGL((gn_bwd_partial_kernel<T>), dim3(nch, (C + 255) / 256, B), dim3(256), 0, s, dact, act, xc, stat,
                     N, C, G, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gn_bwd_finalize_kernel<T>), dim3(G, B), dim3(256), 0, s, partial, nch, B, N, C, G, gamma, m12,
                     dgamma, dbeta);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long total = (long)B * N * C;
  hipLaunchKernelGGL((gn_bwd_apply_kernel<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, dact, act, xc,
                     stat, m12, gamma, N, C, G, total, dxc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight rearrangements for the input-gradient GEMMs (C = A B^T needs B as
// [N][K]): the 3x3 conv's input gradient is a 3x3 conv of dxc with the taps
// mirrored and the channel roles swapped,
//   wflip[ci][t * Co + co] = w[co][8 - t][ci]   (w is [Co][3][3][Ci]).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void conv_weight_flip_kernel(const T* __restrict__ w, int Co, int Ci,
                                                               T* __restrict__ wflip) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)Ci * 9 * Co;
  if (i >= total) return;
  const int ci = (int)(i / (9 * Co)), rest = (int)(i - (long)ci * 9 * Co);
  const int t = rest / Co, co = rest - t * Co;
  wflip[i] = w[((size_t)co * 9 + (8 - t)) * Ci + ci];
}

template <typename T>
hipError_t launch_conv_weight_flip(const T* w, int Co, int Ci, T* wflip, hipStream_t s) {
  const long total = (long)Ci * 9 * Co;
  hipLaunchKernelGGL((conv_weight_flip_kernel<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, w, Co, Ci,
                     wflip);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small fp32 products for the folded query weights' gradients:
//   out[i][j] = (add ? add[i][j] : 0) + (ru ? ru[i] rv[j] : 0) + sum_k A(i, k) B(k, j),
// A(i, k) = A[i * ars + k * acs], B(k, j) = B[k * brs + j * bcs] (any strides,
// so either operand may be read transposed). 64 x 64 output tiles, 16 x 16
// threads with 4 x 4 outputs each, K in steps of 16 through LDS.
// ---------------------------------------------------------------------------
template <typename TA, typename TB, typename TO>
__global__ __launch_bounds__(256) void small_matmul_kernel(int M, int N, int K, const TA* __restrict__ A, long ars,
                                                           long acs, const TB* __restrict__ Bm, long brs, long bcs,
                                                           const float* __restrict__ add, int ldadd,
                                                           const float* __restrict__ ru, const TB* __restrict__ rv,
                                                           TO* __restrict__ out, int ldo) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int kk = e >> 6, r = e & 63;
      const int i = i0 + r, j = j0 + r, k = k0 + kk;
      As[kk][r] = i < M && k < K ? to_f32(A[i * ars + k * acs]) : 0.0f;
      Bs[kk][r] = j < N && k < K ? to_f32(Bm[k * brs + j * bcs]) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = As[kk][ty * 4 + a];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = Bs[kk][tx * 4 + c];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] += av[a] * bv[c];
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = i0 + ty * 4 + a, j = j0 + tx * 4 + c;
      if (i < M && j < N) {
        float v = acc[a][c] + (add ? add[(size_t)i * ldadd + j] : 0.0f);
        if (ru) v += ru[i] * to_f32(rv[j]);
        out[(size_t)i * ldo + j] = from_f32<TO>(v);
      }
    }
}

template <typename TA, typename TB, typename TO>
hipError_t launch_small_matmul(int M, int N, int K, const TA* A, long ars, long acs, const TB* Bm, long brs, long bcs,
                               const float* add, int ldadd, TO* out, int ldo, hipStream_t s, const float* ru,
                               const TB* rv) {
  if (M <= 0 || N <= 0) return hipSuccess;
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL((small_matmul_kernel<TA, TB, TO>), grid, dim3(256), 0, s, M, N, K, A, ars, acs, Bm, brs, bcs,
                     add, ldadd, ru, rv, out, ldo);
  return hipGetLastError();
}

// dx = a + b + c (T inputs, fp32 sum, one rounding).
template <typename T>
__global__ __launch_bounds__(256) void sum3_kernel(const T* __restrict__ a, const T* __restrict__ b,
                                                   const T* __restrict__ c, long n8, T* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float va[8], vb[8], vc[8];
  load8(a + 8 * i, va);
  load8(b + 8 * i, vb);
  load8(c + 8 * i, vc);
#pragma unroll
  for (int k = 0; k < 8; ++k) va[k] += vb[k] + vc[k];
  store8(out + 8 * i, va);
}

template <typename T>
hipError_t launch_sum3(const T* a, const T* b, const T* c, long n, T* out, hipStream_t s) {
  const long n8 = n / 8;
  if (n8 <= 0) return hipSuccess;
  hipLaunchKernelGGL((sum3_kernel<T>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, a, b, c, n8, out);
  return hipGetLastError();
}

#define EDIT_INST(T)                                                                                               \
  template hipError_t launch_transpose<T>(const T*, int, int, int, T*, int, hipStream_t, int);                     \
  template hipError_t launch_shift_transpose<T>(const T*, int, int, int, int, T*, int, int, int, hipStream_t);     \
  template hipError_t launch_colsum<T>(const T*, int, int, int, float*, T*, hipStream_t, float*);                  \
  template hipError_t launch_zero<T>(T*, long, hipStream_t);                                                       \
  template hipError_t launch_splitk_reduce<T>(const float*, int, long long, int, int, T*, int, hipStream_t);       \
  template hipError_t launch_attn_bwd_q<T>(const T*, const T*, const float*, const float*, int, int, int, int,     \
                                           float, T*, float*, T*, hipStream_t);                                    \
  template hipError_t launch_kv_bwd<T>(const T*, const T*, const float*, const float*, int, int, int, int, T*,     \
                                       hipStream_t);                                                               \
  template hipError_t launch_dw_bwd_input<T>(const T*, int, int, int, int, const T*, const T*, T*, hipStream_t);   \
  template hipError_t launch_dw_bwd_weight<T>(const T*, const T*, int, int, int, int, float*, T*, T*, T*, T*,      \
                                              hipStream_t);                                                        \
  template hipError_t launch_gn_bwd<T>(const T*, const T*, const T*, const float*, const T*, int, int, int, int,   \
                                       float*, float*, T*, T*, T*, hipStream_t);                                   \
  template hipError_t launch_conv_weight_flip<T>(const T*, int, int, T*, hipStream_t);                             \
  template hipError_t launch_sum3<T>(const T*, const T*, const T*, long, T*, hipStream_t);
EDIT_INST(bf16)
EDIT_INST(float)
#undef EDIT_INST
template hipError_t launch_small_matmul<float, bf16, bf16>(int, int, int, const float*, long, long, const bf16*, long,
                                                           long, const float*, int, bf16*, int, hipStream_t,
                                                           const float*, const bf16*);
template hipError_t launch_small_matmul<float, float, float>(int, int, int, const float*, long, long, const float*,
                                                             long, long, const float*, int, float*, int, hipStream_t,
                                                             const float*, const float*);

}  // namespace edit
