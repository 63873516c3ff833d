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

constexpr int kGnPix = 64;   // pixels per statistics chunk

int groupnorm_chunks(int HW) { return (HW + kGnPix - 1) / kGnPix; }

// One block per (chunk of kGnPix pixels, sample): exact two-pass per-channel
// mean and sum of squared deviations over the chunk.
// partial[b][chunk][c] = (mean, M2).
template <typename T>
__global__ __launch_bounds__(256) void gn_partial_kernel(const T* __restrict__ x, int HW, int C,
                                                         float* __restrict__ partial, int nchunks) {
  __shared__ float red[2048];
  __shared__ float mean_s[2048];
  const int chunk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int tpr = C / 8;                  // threads per pixel row (C <= 2048)
  const int rows_par = 256 / tpr;
  const int p0 = chunk * kGnPix, p1 = min(HW, p0 + kGnPix), cnt = p1 - p0;
  const int c8 = tid % tpr, rl = tid / tpr;
  const bool active = rl < rows_par;
  const T* base = x + (size_t)b * HW * C + c8 * 8;

  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.0f;
  if (active)
    for (int p = p0 + rl; p < p1; p += rows_par) {
      float v[8];
      load8(base + (size_t)p * C, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] += v[i];
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
  if (active)
    for (int p = p0 + rl; p < p1; p += rows_par) {
      float v[8];
      load8(base + (size_t)p * C, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) { const float d = v[i] - m[i]; s[i] += d * d; }
    }
  __syncthreads();
  if (active)
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rl * C + c8 * 8 + i] = s[i];
  __syncthreads();
  float* out = partial + ((size_t)b * nchunks + chunk) * C * 2;
  for (int c = tid; c < C; c += 256) {
    float t = 0.0f;
    for (int r = 0; r < rows_par; ++r) t += red[r * C + c];
    out[2 * c] = mean_s[c];
    out[2 * c + 1] = t;
  }
}

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

// One wave per (group, sample): Chan-merge the chunk partials of the group's
// channels in a fixed order, then fold gamma/beta into per-channel
// scale/shift: GN(x) = x * scale + shift.
template <typename T>
__global__ __launch_bounds__(64) void gn_finalize_kernel(const float* __restrict__ partial, int HW, int C,
                                                         int G, int nchunks, const T* __restrict__ gamma,
                                                         const T* __restrict__ beta, float eps,
                                                         float* __restrict__ stat, float* __restrict__ scale,
                                                         float* __restrict__ shift) {
  const int g = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int cg = C / G, entries = nchunks * cg;
  Welford acc = {0.0f, 0.0f, 0.0f};
  for (int e = lane; e < entries; e += 64) {
    const int chunk = e / cg, c = g * cg + e % cg;
    const float* pp = partial + (((size_t)b * nchunks + chunk) * C + c) * 2;
    Welford w;
    w.n = (float)min(kGnPix, HW - chunk * kGnPix);
    w.mean = pp[0];
    w.m2 = pp[1];
    acc = chan_merge(acc, w);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Welford other;
    other.n = __shfl_xor(acc.n, o, 64);
    other.mean = __shfl_xor(acc.mean, o, 64);
    other.m2 = __shfl_xor(acc.m2, o, 64);
    // Merge in lane order so every lane holds the same bits.
    acc = (lane & o) ? chan_merge(other, acc) : chan_merge(acc, other);
  }
  const float var = acc.m2 / acc.n;
  const float rstd = 1.0f / sqrtf(var + eps);
  if (lane == 0) {
    stat[((size_t)b * G + g) * 2] = acc.mean;
    stat[((size_t)b * G + g) * 2 + 1] = rstd;
  }
  for (int i = lane; i < cg; i += 64) {
    const int c = g * cg + i;
    const float sc = to_f32(gamma[c]) * rstd;
    scale[(size_t)b * C + c] = sc;
    shift[(size_t)b * C + c] = to_f32(beta[c]) - acc.mean * sc;
  }
}

template <typename T>
hipError_t launch_groupnorm_stats(const T* x, int B, int HW, int C, int G, const T* gamma,
                                  const T* beta, float eps, float* partial, int nchunks,
                                  float* stat, float* scale, float* shift, hipStream_t s) {
  hipLaunchKernelGGL((gn_partial_kernel<T>), dim3(nchunks, B), dim3(256), 0, s, x, HW, C, partial, nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gn_finalize_kernel<T>), dim3(G, B), dim3(64), 0, s, partial, HW, C, G, nchunks,
                     gamma, beta, eps, stat, scale, shift);
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
#pragma unroll
  for (int ky = 0; ky < 3; ++ky) {
    const int yy = 2 * yo + ky - 1;
    if (yy < 0 || yy >= H) continue;
#pragma unroll
    for (int kx = 0; kx < 3; ++kx) {
      const int xx = 2 * xo + kx - 1;
      if (xx < 0 || xx >= W) continue;
      float v[8], wv[8];
      load8(img + ((size_t)yy * W + xx) * 2 * C, v);
      load8(w + (ky * 3 + kx) * C + ch, wv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += wv[i] * v[i];
    }
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
  template hipError_t launch_groupnorm_stats<T>(const T*, int, int, int, int, const T*, const T*, float, \
                                                float*, int, float*, float*, float*, hipStream_t);      \
  template hipError_t launch_dwconv_s2<T>(const T*, int, int, int, int, const T*, const T*, const T*,    \
                                          const T*, T*, T*, hipStream_t);
EDIT_INST(bf16)
EDIT_INST(float)
#undef EDIT_INST

}  // namespace edit
