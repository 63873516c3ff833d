// GroupNorm statistics (ConvFusion) and the Spatial Compressor's depthwise
// 3x3 stride-2 convolution, both memory-bound, channel-last and coalesced.
//
// Page "EDiT: Efficient Diffusion Transformers with Linear Compressed
// Attention" (ICCV 2025 notes): section "ConvFusion" puts GroupNorm after
// the 3x3 compressing conv; section "Spatial Compressor" shrinks the key and
// value grids with a 3x3 depthwise conv of stride 2 and puts a ReLU on the
// keys only.
#include "common.hpp"
#include "launch.hpp"

namespace edit {

constexpr int kGnMaxRows = 4;     // pixels one thread keeps in registers

// A statistics chunk is as many pixels as the block holds in registers:
// 256 / (C/8) pixel rows in parallel, kGnMaxRows each. Four rows per thread
// give ~600 blocks at 16384 pixels and C = 288 (16 rows gave 147 blocks,
// too few to cover the chip: 10.8 us for 9.4 MB).
static int gn_chunk_px(int C) { return (256 / (C / 8)) * kGnMaxRows; }
int groupnorm_chunks(int HW, int C) { return (HW + gn_chunk_px(C) - 1) / gn_chunk_px(C); }

struct Welford { float n, mean, m2; };

__device__ __forceinline__ Welford chan_merge(Welford a, Welford b) {
  if (b.n == 0.0f) return a;
  if (a.n == 0.0f) return b;
  const float n = a.n + b.n, d = b.mean - a.mean;
  Welford r;
  r.n = n;
  r.mean = a.mean + d * (b.n / n);
  r.m2 = a.m2 + b.m2 + d * d * (a.n * b.n / n);
  return r;
}

// One block per (chunk of kGnPix pixels, sample). The chunk's values stay in
// registers: exact per-channel mean, then per-channel sum of squared
// deviations, then the group's channels merged (equal counts):
//   mean_g = avg_c mean_c,  M2_g = sum_c M2_c + cnt * sum_c (mean_c - mean_g)^2.
// partial[b][chunk][g] = (mean_g, M2_g) over cnt * C/G values.
template <typename T>
__global__ __launch_bounds__(256) void gn_partial_kernel(const T* __restrict__ x, int HW, int C, int G,
                                                         int chunk_px, float* __restrict__ partial, int nchunks) {
  __shared__ float red[2048];
  __shared__ float mean_s[2048];
  __shared__ float m2_s[2048];
  const int chunk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int tpr = C / 8;                  // threads per pixel row (C <= 2048)
  const int rows_par = 256 / tpr;
  const int p0 = chunk * chunk_px, p1 = min(HW, p0 + chunk_px), cnt = p1 - p0;
  const int c8 = tid % tpr, rl = tid / tpr;
  const bool active = rl < rows_par;
  const T* base = x + (size_t)b * HW * C + c8 * 8;

  float v[kGnMaxRows][8];
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.0f;
#pragma unroll
  for (int r = 0; r < kGnMaxRows; ++r) {
    const int p = p0 + rl + r * rows_par;
    if (active && p < p1) {
      load8(base + (size_t)p * C, v[r]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[r][i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] += v[r][i];
  }
  if (active)
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rl * C + c8 * 8 + i] = s[i];
  __syncthreads();
  for (int c = tid; c < C; c += 256) {
    float t = 0.0f;
    for (int r = 0; r < rows_par; ++r) t += red[r * C + c];
    mean_s[c] = t / (float)cnt;
  }
  __syncthreads();
  float m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { s[i] = 0.0f; m[i] = active ? mean_s[c8 * 8 + i] : 0.0f; }
#pragma unroll
  for (int r = 0; r < kGnMaxRows; ++r) {
    const int p = p0 + rl + r * rows_par;
    if (active && p < p1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) { const float d = v[r][i] - m[i]; s[i] += d * d; }
    }
  }
  if (active)
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rl * C + c8 * 8 + i] = s[i];
  __syncthreads();
  for (int c = tid; c < C; c += 256) {
    float t = 0.0f;
    for (int r = 0; r < rows_par; ++r) t += red[r * C + c];
    m2_s[c] = t;
  }
  __syncthreads();
  const int cg = C / G;
  for (int g = tid; g < G; g += 256) {
    float mg = 0.0f;
    for (int c = 0; c < cg; ++c) mg += mean_s[g * cg + c];
    mg /= (float)cg;
    float m2 = 0.0f;
    for (int c = 0; c < cg; ++c) {
      const float d = mean_s[g * cg + c] - mg;
      m2 += m2_s[g * cg + c] + (float)cnt * d * d;
    }
    float* out = partial + (((size_t)b * nchunks + chunk) * G + g) * 2;
    out[0] = mg;
    out[1] = m2;
  }
}

// One block per (group, sample): each thread Chan-merges a strided subset
// of the chunk partials, then a fixed-shape LDS tree merges the 256 results,
// so the statistics are bit-for-bit reproducible. Folds gamma / beta into
// per-channel scale / shift: GN(x) = x * scale + shift.
template <typename T>
__global__ __launch_bounds__(256) void gn_finalize_kernel(const float* __restrict__ partial, int HW, int C,
                                                         int G, int chunk_px, int nchunks, const T* __restrict__ gamma,
                                                         const T* __restrict__ beta, float eps,
                                                         float* __restrict__ stat, float* __restrict__ scale,
                                                         float* __restrict__ shift) {
  __shared__ float sn[256], smean[256], sm2[256];
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int cg = C / G;
  Welford acc = {0.0f, 0.0f, 0.0f};
  for (int ch = tid; ch < nchunks; ch += 256) {
    const float* pp = partial + (((size_t)b * nchunks + ch) * G + g) * 2;
    Welford w;
    w.n = (float)(min(chunk_px, HW - ch * chunk_px) * cg);
    w.mean = pp[0];
    w.m2 = pp[1];
    acc = chan_merge(acc, w);
  }
  sn[tid] = acc.n; smean[tid] = acc.mean; sm2[tid] = acc.m2;
  __syncthreads();
  for (int stride = 128; stride > 0; stride >>= 1) {
    if (tid < stride) {
      Welford a = {sn[tid], smean[tid], sm2[tid]};
      Welford o = {sn[tid + stride], smean[tid + stride], sm2[tid + stride]};
      a = chan_merge(a, o);
      sn[tid] = a.n; smean[tid] = a.mean; sm2[tid] = a.m2;
    }
    __syncthreads();
  }
  const float mean = smean[0];
  const float var = sm2[0] / sn[0];
  const float rstd = 1.0f / sqrtf(var + eps);
  if (tid == 0) {
    stat[((size_t)b * G + g) * 2] = mean;
    stat[((size_t)b * G + g) * 2 + 1] = rstd;
  }
  for (int i = tid; i < cg; i += 256) {
    const int c = g * cg + i;
    const float sc = to_f32(gamma[c]) * rstd;
    scale[(size_t)b * C + c] = sc;
    shift[(size_t)b * C + c] = to_f32(beta[c]) - mean * sc;
  }
}

template <typename T>
hipError_t launch_groupnorm_stats(const T* x, int B, int HW, int C, int G, const T* gamma,
                                  const T* beta, float eps, float* partial, int nchunks,
                                  float* stat, float* scale, float* shift, hipStream_t s) {
  const int px = gn_chunk_px(C);
  hipLaunchKernelGGL((gn_partial_kernel<T>), dim3(nchunks, B), dim3(256), 0, s, x, HW, C, G, px, partial, nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gn_finalize_kernel<T>), dim3(G, B), dim3(256), 0, s, partial, HW, C, G, px, nchunks,
                     gamma, beta, eps, stat, scale, shift);
  return hipGetLastError();
}

// Statistics from the conv epilogue's partials: one (mean, M2) per tile of
// `rows` rows and channel. One block per (group, sample) Chan-merges the
// (tile, channel) items of its sample and group, each thread a strided
// subset, then the same fixed LDS tree as above; scale / shift as above.
template <typename T>
__global__ __launch_bounds__(256) void gn_finalize_channels_kernel(const float* __restrict__ partial, int HW, int C,
                                                                   int G, int rows, const T* __restrict__ gamma,
                                                                   const T* __restrict__ beta, float eps,
                                                                   float* __restrict__ stat, float* __restrict__ scale,
                                                                   float* __restrict__ shift) {
  __shared__ float sn[256], smean[256], sm2[256];
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int cg = C / G, tps = HW / rows;
  Welford acc = {0.0f, 0.0f, 0.0f};
  for (int it = tid; it < tps * cg; it += 256) {
    const int tile = b * tps + it / cg, c = g * cg + it % cg;
    const float* pp = partial + ((size_t)tile * C + c) * 2;
    Welford w;
    w.n = (float)rows;
    w.mean = pp[0];
    w.m2 = pp[1];
    acc = chan_merge(acc, w);
  }
  sn[tid] = acc.n; smean[tid] = acc.mean; sm2[tid] = acc.m2;
  __syncthreads();
  for (int stride = 128; stride > 0; stride >>= 1) {
    if (tid < stride) {
      Welford a = {sn[tid], smean[tid], sm2[tid]};
      Welford o = {sn[tid + stride], smean[tid + stride], sm2[tid + stride]};
      a = chan_merge(a, o);
      sn[tid] = a.n; smean[tid] = a.mean; sm2[tid] = a.m2;
    }
    __syncthreads();
  }
  const float mean = smean[0];
  const float var = sm2[0] / sn[0];
  const float rstd = 1.0f / sqrtf(var + eps);
  if (tid == 0) {
    stat[((size_t)b * G + g) * 2] = mean;
    stat[((size_t)b * G + g) * 2 + 1] = rstd;
  }
  for (int i = tid; i < cg; i += 256) {
    const int c = g * cg + i;
    const float sc = to_f32(gamma[c]) * rstd;
    scale[(size_t)b * C + c] = sc;
    shift[(size_t)b * C + c] = to_f32(beta[c]) - mean * sc;
  }
}

template <typename T>
hipError_t launch_groupnorm_finalize_channels(const float* partial, int B, int HW, int C, int G, int rows,
                                              const T* gamma, const T* beta, float eps, float* stat, float* scale,
                                              float* shift, hipStream_t s) {
  if (rows <= 0 || HW % rows != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gn_finalize_channels_kernel<T>), dim3(G, B), dim3(256), 0, s, partial, HW, C, G, rows, gamma,
                     beta, eps, stat, scale, shift);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a = LeakyReLU(x * scale[b][c] + shift[b][c], 0.01): GroupNorm with its
// affine folded into scale / shift, then the ConvFusion activation (section
// "ConvFusion"), once per element, 8 channels per thread (16-byte accesses).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void gn_apply_kernel(const T* __restrict__ x, int HW, int C, size_t n8,
                                                       const float* __restrict__ scale,
                                                       const float* __restrict__ shift, T* __restrict__ a) {
  const size_t i = (size_t)xcd_swizzle(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const size_t e = i * 8;                      // first element (C is a multiple of 8)
  const size_t row = e / C;
  const int c = (int)(e - row * C);
  const int b = (int)(row / HW);
  float v[8], sc[8], sh[8];
  load8(x + e, v);
  load8(scale + (size_t)b * C + c, sc);
  load8(shift + (size_t)b * C + c, sh);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float t = v[k] * sc[k] + sh[k];
    v[k] = t >= 0.0f ? t : 0.01f * t;
  }
  store8(a + e, v);
}

template <typename T>
hipError_t launch_groupnorm_apply(const T* x, int B, int HW, int C, const float* scale, const float* shift, T* a,
                                  hipStream_t s) {
  const size_t n8 = (size_t)B * HW * C / 8;
  if (n8 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n8 + 255) / 256);
  hipLaunchKernelGGL((gn_apply_kernel<T>), dim3(blocks), dim3(256), 0, s, x, HW, C, n8, scale, shift, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Depthwise 3x3, stride 2, zero pad 1 over kv0 [B][H][W][2C]: output pixel
// (y', x') of channel c reads input (2y'+ky-1, 2x'+kx-1). One thread makes
// 8 consecutive channels of one output pixel; consecutive threads walk the
// channels, so every load and store is a coalesced 16-byte access.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dwconv_s2_kernel(const T* __restrict__ kv0, int B, int H, int W, int C,
                                                        const T* __restrict__ dwk, const T* __restrict__ dbk,
                                                        const T* __restrict__ dwv, const T* __restrict__ dbv,
                                                        T* __restrict__ kc, T* __restrict__ vc) {
  const int Hc = (H + 1) / 2, Wc = (W + 1) / 2;
  const int cpp = (2 * C) / 8;                                    // chunks per pixel
  const long total = (long)B * Hc * Wc * cpp;
  const long idx = (long)xcd_swizzle(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int c8 = (int)(idx % cpp);
  const long pix = idx / cpp;
  const int xo = (int)(pix % Wc);
  const int yo = (int)((pix / Wc) % Hc);
  const int b = (int)(pix / ((long)Wc * Hc));
  const int ch2 = c8 * 8;                                         // channel in [0, 2C)
  const bool is_k = ch2 < C;
  const int ch = is_k ? ch2 : ch2 - C;
  const T* w = is_k ? dwk : dwv;
  const T* bias = is_k ? dbk : dbv;

  float acc[8];
  load8(bias + ch, acc);
  const T* img = kv0 + (size_t)b * H * W * 2 * C + ch2;
  // Every tap's load is issued (at a clamped, in-image position) before any
  // is used; a tap outside the image then contributes zero.
  float v[9][8], wv[9][8];
#pragma unroll
  for (int t = 0; t < 9; ++t) {
    const int yy = 2 * yo + t / 3 - 1, xx = 2 * xo + t % 3 - 1;
    const int yc = min(max(yy, 0), H - 1), xcl = min(max(xx, 0), W - 1);
    load8(img + ((size_t)yc * W + xcl) * 2 * C, v[t]);
    load8(w + t * C + ch, wv[t]);
  }
#pragma unroll
  for (int t = 0; t < 9; ++t) {
    const int yy = 2 * yo + t / 3 - 1, xx = 2 * xo + t % 3 - 1;
    const bool in = yy >= 0 && yy < H && xx >= 0 && xx < W;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += in ? wv[t][i] * v[t][i] : 0.0f;
  }
  if (is_k) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] > 0.0f ? acc[i] : 0.0f;
  }
  T* out = (is_k ? kc : vc) + (size_t)pix * C + ch;
  store8(out, acc);
}

template <typename T>
hipError_t launch_dwconv_s2(const T* kv0, int B, int H, int W, int C, const T* dwk, const T* dbk,
                            const T* dwv, const T* dbv, T* kc, T* vc, hipStream_t s) {
  const long total = (long)B * ((H + 1) / 2) * ((W + 1) / 2) * (2 * C / 8);
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL((dwconv_s2_kernel<T>), dim3(blocks), dim3(256), 0, s, kv0, B, H, W, C, dwk, dbk, dwv,
                     dbv, kc, vc);
  return hipGetLastError();
}

#define EDIT_INST(T)                                                                                    \
  template hipError_t launch_groupnorm_apply<T>(const T*, int, int, int, const float*, const float*, T*,  \
                                                hipStream_t);                                           \
  template hipError_t launch_groupnorm_stats<T>(const T*, int, int, int, int, const T*, const T*, float, \
                                                float*, int, float*, float*, float*, hipStream_t);      \
  template hipError_t launch_groupnorm_finalize_channels<T>(const float*, int, int, int, int, int,        \
                                                            const T*, const T*, float, float*, float*,   \
                                                            float*, hipStream_t);                        \
  template hipError_t launch_dwconv_s2<T>(const T*, int, int, int, int, const T*, const T*, const T*,    \
                                          const T*, T*, T*, hipStream_t);
EDIT_INST(bf16)
EDIT_INST(float)
#undef EDIT_INST

}  // namespace edit
