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
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    float v = 0.0f;
    if (r < rows && c < cols) {
      if (SHIFT) {
        // r is the destination token m'; the source token is m = m' - off,
        // valid when its pixel (y, x) has (y + ky - 1, x + kx - 1) = pixel(m').
        const int hw = H * W, b = r / hw, q = r - b * hw, y1 = q / W, x1 = q - (q / W) * W;
        const int y = y1 - (ky - 1), x = x1 - (kx - 1);
        if (y >= 0 && y < H && x >= 0 && x < W) v = to_f32(in[((size_t)b * hw + (size_t)y * W + x) * ldi + c]);
      } else {
        v = to_f32(in[(size_t)r * ldi + c]);
      }
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows_pad) out[(size_t)c * ldo + r] = from_f32<T>(tile[tx][i]);
  }
}

template <typename T>
hipError_t launch_transpose(const T* in, int rows, int cols, int ldi, T* out, int ldo, hipStream_t s,
                            int rows_pad) {
  if (rows_pad < rows) rows_pad = rows;
  if (rows <= 0 || cols <= 0) return hipSuccess;
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
  dim3 grid((cols + 63) / 64, (ldo + 63) / 64);
  hipLaunchKernelGGL((transpose_kernel<T, true>), grid, dim3(256), 0, s, in, rows, ldo, cols, cols, out, ldo, H, W,
                     ky, kx);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Column sums (bias gradients): out[c] = sum_r in[r][c], rows summed in
// chunks of 256 (partial[chunk][c]), then the chunks in order.
// ---------------------------------------------------------------------------
constexpr int kColChunk = 256;
int colsum_chunks(int rows) { return (rows + kColChunk - 1) / kColChunk; }

template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T* __restrict__ in, int rows, int cols, int ld,
                                                             float* __restrict__ partial) {
  const int c = blockIdx.x * 256 + threadIdx.x, ch = blockIdx.y;
  if (c >= cols) return;
  const int r0 = ch * kColChunk, r1 = min(rows, r0 + kColChunk);
  float s = 0.0f;
  for (int r = r0; r < r1; ++r) s += to_f32(in[(size_t)r * ld + c]);
  partial[(size_t)ch * cols + c] = s;
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
// y's rounding would be amplified. One thread per token (128 per block, one
// head): S is staged transposed in LDS (ST[n][a] = S[a][n], so eight outputs
// read one 32-byte row segment), the token's dy in a padded LDS row; d is a
// runtime value. t is formed twice (once for dy . y, once for dq). g (T) and
// c (f32) are kept for the state gradient dS = sum q^T g, dz = sum c q.
// ---------------------------------------------------------------------------
constexpr int kBwdTok = 128;

__host__ __device__ inline size_t head_bwd_lds(int d) { return ((size_t)d * d + d + (size_t)kBwdTok * (d + 1)) * 4; }

template <typename T>
__global__ __launch_bounds__(kBwdTok) void attn_bwd_q_kernel(const T* __restrict__ dy, const T* __restrict__ q,
                                                             const float* __restrict__ S,
                                                             const float* __restrict__ z, int N, int heads, int d,
                                                             float eps, T* __restrict__ g_out,
                                                             float* __restrict__ c_out, T* __restrict__ dq_pre) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* ST = sm;              // [d][d]
  float* zs = ST + d * d;      // [d]
  float* ds = zs + d;          // [kBwdTok][d + 1]
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, dp = d + 1;
  const int C = heads * d;
  const size_t bh = (size_t)b * heads + h;
  for (int i = tid; i < d * d; i += kBwdTok) {
    const int a = i / d, n = i - a * d;
    ST[n * d + a] = S[bh * d * d + i];
  }
  for (int i = tid; i < d; i += kBwdTok) zs[i] = z[bh * d + i];
  __syncthreads();
  const int tok = blockIdx.x * kBwdTok + tid;
  if (tok >= N) return;
  const size_t row = ((size_t)b * N + tok) * C + (size_t)h * d;
  float* dr = ds + tid * dp;
  float den = eps;
  for (int c8 = 0; c8 < d; c8 += 8) {
    float qv[8], dv[8];
    load8(q + row + c8, qv);
    load8(dy + row + c8, dv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      den += qv[i] * zs[c8 + i];
      dr[c8 + i] = dv[i];
    }
  }
  const float inv = 1.0f / den;
  // t[a0 .. a0+7] = sum_n dy[n] S[a][n]
  auto t8 = [&](int a0, float (&t)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = 0.0f;
    for (int n = 0; n < d; ++n) {
      const float dn = dr[n];
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(ST + n * d + a0);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(ST + n * d + a0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        t[i] += dn * s0[i];
        t[4 + i] += dn * s1[i];
      }
    }
  };
  float qt = 0.0f;
  for (int a0 = 0; a0 < d; a0 += 8) {
    float t[8], qv[8];
    t8(a0, t);
    load8(q + row + a0, qv);
#pragma unroll
    for (int i = 0; i < 8; ++i) qt += qv[i] * t[i];
  }
  const float c = -qt * inv * inv;
  c_out[((size_t)b * N + tok) * heads + h] = c;
  for (int c8 = 0; c8 < d; c8 += 8) {
    float go[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) go[i] = dr[c8 + i] * inv;
    store8(g_out + row + c8, go);
  }
  for (int a0 = 0; a0 < d; a0 += 8) {
    float t[8], qv[8], o[8];
    t8(a0, t);
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
  const size_t lds = head_bwd_lds(d);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_q_kernel<T>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((N + kBwdTok - 1) / kBwdTok, heads, B);
  hipLaunchKernelGGL((attn_bwd_q_kernel<T>), grid, dim3(kBwdTok), lds, s, dy, q, S, z, N, heads, d, eps, g, c,
                     dq_pre);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// State backward (section "Linear-attention formula", S = sum K'^T V',
// z = sum K'): per compressed token j and head,
//   dK'_j = V'_j dS^T + dz, then the keys' ReLU (where K'_j > 0),
//   dV'_j = K'_j dS.
// Writes dkv [B][Nc][2C]: the keys' gradient before their ReLU | the values'.
// Same layout as the query side: the matrix in LDS in the orientation that
// gives eight outputs one row segment (dS^T for the keys, dS for the values),
// the token's row in a padded LDS row.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kBwdTok) void kv_bwd_kernel(const T* __restrict__ kc, const T* __restrict__ vc,
                                                         const float* __restrict__ dS, const float* __restrict__ dz,
                                                         int Nc, int heads, int d, T* __restrict__ dkv) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* Mx = sm;              // [d][d]
  float* zs = Mx + d * d;      // [d]
  float* ts = zs + d;          // [kBwdTok][d + 1]
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, dp = d + 1;
  const int C = heads * d;
  const size_t bh = (size_t)b * heads + h;
  const int tok = blockIdx.x * kBwdTok + tid;
  const bool valid = tok < Nc;
  const size_t row = ((size_t)b * Nc + (valid ? tok : 0)) * C + (size_t)h * d;
  T* out = dkv + ((size_t)b * Nc + (valid ? tok : 0)) * 2 * C + (size_t)h * d;
  float* tr = ts + tid * dp;

  // keys: Mx[n][a] = dS[a][n]
  for (int i = tid; i < d * d; i += kBwdTok) {
    const int a = i / d, n = i - a * d;
    Mx[n * d + a] = dS[bh * d * d + i];
  }
  for (int i = tid; i < d; i += kBwdTok) zs[i] = dz[bh * d + i];
  if (valid)
    for (int c8 = 0; c8 < d; c8 += 8) {
      float v[8];
      load8(vc + row + c8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) tr[c8 + i] = v[i];
    }
  __syncthreads();
  if (valid)
    for (int a0 = 0; a0 < d; a0 += 8) {
      float acc[8], kv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = zs[a0 + i];
      for (int n = 0; n < d; ++n) {
        const float vn = tr[n];
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(Mx + n * d + a0);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(Mx + n * d + a0 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] += vn * s0[i];
          acc[4 + i] += vn * s1[i];
        }
      }
      load8(kc + row + a0, kv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = kv[i] > 0.0f ? acc[i] : 0.0f;
      store8(out + a0, acc);
    }
  __syncthreads();
  // values: Mx[m][a] = dS[m][a]
  for (int i = tid; i < d * d; i += kBwdTok) Mx[i] = dS[bh * d * d + i];
  if (valid)
    for (int c8 = 0; c8 < d; c8 += 8) {
      float k[8];
      load8(kc + row + c8, k);
#pragma unroll
      for (int i = 0; i < 8; ++i) tr[c8 + i] = k[i];
    }
  __syncthreads();
  if (valid)
    for (int a0 = 0; a0 < d; a0 += 8) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
      for (int m = 0; m < d; ++m) {
        const float km = tr[m];
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(Mx + m * d + a0);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(Mx + m * d + a0 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] += km * s0[i];
          acc[4 + i] += km * s1[i];
        }
      }
      store8(out + C + a0, acc);
    }
}

template <typename T>
hipError_t launch_kv_bwd(const T* kc, const T* vc, const float* dS, const float* dz, int B, int Nc, int heads,
                         int d, T* dkv, hipStream_t s) {
  const size_t lds = head_bwd_lds(d);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kv_bwd_kernel<T>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((Nc + kBwdTok - 1) / kBwdTok, heads, B);
  hipLaunchKernelGGL((kv_bwd_kernel<T>), grid, dim3(kBwdTok), lds, s, kc, vc, dS, dz, Nc, heads, d, dkv);
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
constexpr int kGnbRows = 64;
int gn_bwd_chunks(int N) { return (N + kGnbRows - 1) / kGnbRows; }

template <typename T>
__global__ __launch_bounds__(256) void gn_bwd_partial_kernel(const T* __restrict__ dact, const T* __restrict__ act,
                                                             const T* __restrict__ xc, const float* __restrict__ stat,
                                                             int N, int C, int G, float* __restrict__ partial) {
  const int c = blockIdx.y * 256 + threadIdx.x, chunk = blockIdx.x, b = blockIdx.z;
  if (c >= C) return;
  const int cg = C / G, g = c / cg;
  const float mean = stat[((size_t)b * G + g) * 2], rstd = stat[((size_t)b * G + g) * 2 + 1];
  const int n0 = chunk * kGnbRows, n1 = min(N, n0 + kGnbRows);
  float s1 = 0.0f, s2 = 0.0f;
  for (int n = n0; n < n1; ++n) {
    const size_t i = ((size_t)b * N + n) * C + c;
    const float a = to_f32(act[i]), da0 = to_f32(dact[i]);
    const float da = a >= 0.0f ? da0 : 0.01f * da0;
    s1 += da;
    s2 += da * (to_f32(xc[i]) - mean) * rstd;
  }
  const int nch = gridDim.x;
  float* out = partial + (((size_t)b * nch + chunk) * C + c) * 2;
  out[0] = s1;
  out[1] = s2;
}

// One block per (sample, group), one thread per channel of the group; block
// (0, g) also writes dgamma, dbeta of its channels (summed over samples).
template <typename T>
__global__ __launch_bounds__(256) void gn_bwd_finalize_kernel(const float* __restrict__ partial, int nchunks, int B,
                                                              int N, int C, int G, const T* __restrict__ gamma,
                                                              float* __restrict__ m12, T* __restrict__ dgamma,
                                                              T* __restrict__ dbeta) {
  __shared__ float r1[256], r2[256];
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int cg = C / G;
  float s1 = 0.0f, s2 = 0.0f;
  if (tid < cg) {
    const int c = g * cg + tid;
    for (int ch = 0; ch < nchunks; ++ch) {
      const float* p = partial + (((size_t)b * nchunks + ch) * C + c) * 2;
      s1 += p[0];
      s2 += p[1];
    }
    const float gm = to_f32(gamma[c]);
    r1[tid] = gm * s1;
    r2[tid] = gm * s2;
    if (b == 0) {
      float t1 = 0.0f, t2 = 0.0f;
      for (int bb = 0; bb < B; ++bb)
        for (int ch = 0; ch < nchunks; ++ch) {
          const float* p = partial + (((size_t)bb * nchunks + ch) * C + c) * 2;
          t1 += p[0];
          t2 += p[1];
        }
      dbeta[c] = from_f32<T>(t1);
      dgamma[c] = from_f32<T>(t2);
    }
  }
  __syncthreads();
  if (tid == 0) {
    float a1 = 0.0f, a2 = 0.0f;
    for (int i = 0; i < cg; ++i) { a1 += r1[i]; a2 += r2[i]; }
    const float inv = 1.0f / ((float)N * (float)cg);
    m12[((size_t)b * G + g) * 2] = a1 * inv;
    m12[((size_t)b * G + g) * 2 + 1] = a2 * inv;
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
  if (C / G > 256) return hipErrorInvalidValue;
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
template hipError_t launch_small_matmul<bf16, float, bf16>(int, int, int, const bf16*, long, long, const float*, long,
                                                           long, const float*, int, bf16*, int, hipStream_t,
                                                           const float*, const float*);
template hipError_t launch_small_matmul<float, float, float>(int, int, int, const float*, long, long, const float*,
                                                             long, long, const float*, int, float*, int, hipStream_t,
                                                             const float*, const float*);

}  // namespace edit
