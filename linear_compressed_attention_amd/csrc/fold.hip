// The ConvFusion 1x1 restore folded into the Linear that reads its output.
//
// Page "EDiT: Efficient Diffusion Transformers with Linear Compressed
// Attention" (ICCV 2025 notes), section "ConvFusion": the query Linear reads
// X + Conv1x1(act) with act = LeakyReLU(GN(Conv3x3(X))). A 1x1 convolution is
// a Linear over channels, so for any Linear (W, b):
//   (X + act W2^T + b2) W^T + b = [X | act] [W | W W2]^T + (b + W b2).
// The layer then runs one GEMM of depth C + C/r over the two row sources
// instead of writing and re-reading the restored stream (B x N x C values).
// These kernels build the concatenated weight wcat [C][C + Cr] = [W | W W2]
// and bias bcat [C] = b + W b2 (fp32 sums, one rounding to T).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace edit {

namespace {

// bf16, C % 64 == 0, Cr % 32 == 0. One block per 32 x 32 tile of
// W [W2 | b2 | 0 ...] (tile column Cr / 32 holds b2 in its first column, so
// W b2 comes from the same matrix-core steps); its four waves split the
// depth C in quarters (32x32x16 steps) and add their partial tiles through
// LDS. Every block also copies a slice of W into wcat. R steps of loads are
// issued before their matrix work (R divides C / 64), with no branch between
// them, so a wave waits for memory C / (64 R) times.
template <int R>
__global__ __launch_bounds__(256) void restore_fold_mfma_kernel(const bf16* __restrict__ W,
                                                                const bf16* __restrict__ b,
                                                                const bf16* __restrict__ W2,
                                                                const bf16* __restrict__ b2, int C, int Cr,
                                                                bf16* __restrict__ wcat, bf16* __restrict__ bcat) {
  __shared__ float red[4][32][33];
  const int ldw = C + Cr;
  const int tiles_j = Cr / 32 + 1;
  const int it = blockIdx.x / tiles_j, jt = blockIdx.x % tiles_j;
  const bool bias_tile = jt == tiles_j - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, fh = lane >> 5;

  // Lane l feeds row fr of W (first operand) and column fr of W2 (second
  // operand), K values 8 fh .. 8 fh + 7 of each 16-deep step; accumulator
  // element 4g + e then holds (row 8g + 4fh + e, column fr) of the tile.
  // The second operand's column: W2 column jt*32 + fr (stride Cr), or b2
  // (stride 1) in lane column 0 of the bias tile and zero in the others.
  const int kq = C / 4, k0 = wave * kq, k1 = k0 + kq;
  const bf16* wrow = W + (size_t)(it * 32 + fr) * C + 8 * fh;
  const bf16* col = bias_tile ? b2 + 8 * fh : W2 + (size_t)(8 * fh) * Cr + jt * 32 + fr;
  const size_t stride = bias_tile ? 1 : (size_t)Cr;
  const bool zero_col = bias_tile && fr != 0;
  f32x16 acc;
  acc_zero(acc);
  for (int k = k0; k < k1; k += 16 * R) {
    bf16x8 a[R], v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      a[r] = *reinterpret_cast<const bf16x8*>(wrow + k + 16 * r);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[r][e] = col[(size_t)(k + 16 * r + e) * stride];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (zero_col) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[r][e] = (bf16)0.0f;
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], v[r], acc, 0, 0, 0);
    }
  }
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][8 * g + 4 * fh + e][fr] = acc[4 * g + e];
  __syncthreads();
  if (!bias_tile) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q, i = idx >> 5, j = idx & 31;
      const float s = red[0][i][j] + red[1][i][j] + red[2][i][j] + red[3][i][j];
      wcat[(size_t)(it * 32 + i) * ldw + C + jt * 32 + j] = (bf16)s;
    }
  } else if (tid < 32) {
    const float s = red[0][tid][0] + red[1][tid][0] + red[2][tid][0] + red[3][tid][0];
    bcat[it * 32 + tid] = (bf16)((float)b[it * 32 + tid] + s);
  }

  // [W | .]: 16-byte chunks spread over all blocks.
  const int cpr = C / 8;
  for (int idx = blockIdx.x * 256 + tid; idx < C * cpr; idx += gridDim.x * 256) {
    const int r = idx / cpr, c8 = idx - r * cpr;
    *reinterpret_cast<bf16x8*>(wcat + (size_t)r * ldw + 8 * c8) =
        *reinterpret_cast<const bf16x8*>(W + (size_t)r * C + 8 * c8);
  }
}

// Any element type and shape (C, Cr multiples of 8): one output value per
// thread, grid-stride.
template <typename T>
__global__ __launch_bounds__(256) void restore_fold_kernel(const T* __restrict__ W, const T* __restrict__ b,
                                                           const T* __restrict__ W2, const T* __restrict__ b2,
                                                           int C, int Cr, T* __restrict__ wcat,
                                                           T* __restrict__ bcat) {
  const size_t ldw = (size_t)C + Cr;
  const size_t nprod = (size_t)C * Cr, ncopy = (size_t)C * C, total = nprod + ncopy + C;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (size_t)gridDim.x * 256) {
    if (idx < nprod) {
      const int i = (int)(idx / Cr), j = (int)(idx % Cr);
      float s = 0.0f;
      for (int k = 0; k < C; ++k) s += to_f32(W[(size_t)i * C + k]) * to_f32(W2[(size_t)k * Cr + j]);
      wcat[i * ldw + C + j] = from_f32<T>(s);
    } else if (idx < nprod + ncopy) {
      const size_t e = idx - nprod;
      const size_t i = e / C, k = e % C;
      wcat[i * ldw + k] = W[e];
    } else {
      const int i = (int)(idx - nprod - ncopy);
      float s = 0.0f;
      for (int k = 0; k < C; ++k) s += to_f32(W[(size_t)i * C + k]) * to_f32(b2[k]);
      bcat[i] = from_f32<T>(to_f32(b[i]) + s);
    }
  }
}

}  // namespace

template <typename T>
hipError_t launch_restore_fold(const T* W, const T* b, const T* W2, const T* b2, int C, int Cr, T* wcat, T* bcat,
                               hipStream_t s) {
  if (C <= 0 || Cr <= 0) return hipSuccess;
  if constexpr (std::is_same<T, bf16>::value) {
    if (C % 64 == 0 && Cr % 32 == 0) {
      const dim3 grid((C / 32) * (Cr / 32 + 1));
      const int steps = C / 64;   // 16-deep steps per wave
      if (steps % 6 == 0)
        hipLaunchKernelGGL(restore_fold_mfma_kernel<6>, grid, dim3(256), 0, s, W, b, W2, b2, C, Cr, wcat, bcat);
      else if (steps % 2 == 0)
        hipLaunchKernelGGL(restore_fold_mfma_kernel<2>, grid, dim3(256), 0, s, W, b, W2, b2, C, Cr, wcat, bcat);
      else
        hipLaunchKernelGGL(restore_fold_mfma_kernel<1>, grid, dim3(256), 0, s, W, b, W2, b2, C, Cr, wcat, bcat);
      return hipGetLastError();
    }
  }
  const size_t total = (size_t)C * Cr + (size_t)C * C + C;
  const size_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL((restore_fold_kernel<T>), dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s, W,
                     b, W2, b2, C, Cr, wcat, bcat);
  return hipGetLastError();
}

template hipError_t launch_restore_fold<bf16>(const bf16*, const bf16*, const bf16*, const bf16*, int, int, bf16*,
                                              bf16*, hipStream_t);
template hipError_t launch_restore_fold<float>(const float*, const float*, const float*, const float*, int, int,
                                               float*, float*, hipStream_t);

}  // namespace edit
