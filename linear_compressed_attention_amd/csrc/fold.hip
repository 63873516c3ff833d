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
#include "fold.hpp"
#include "launch.hpp"

namespace edit {

namespace {

// bf16, C % 64 == 0, Cr % 32 == 0: one block per tile of fold.hpp's
// fold_tile; every block also copies a slice of W into wcat.
template <int R>
__global__ __launch_bounds__(256) void restore_fold_mfma_kernel(FoldArgs f) {
  __shared__ float red[4][32][33];
  fold_tile<R>(f, blockIdx.x, red);
  fold_copy(f, blockIdx.x * 256 + threadIdx.x, gridDim.x * 256);
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
      const FoldArgs f{W, b, W2, b2, wcat, bcat, C, Cr};
      if (steps % 6 == 0)
        hipLaunchKernelGGL(restore_fold_mfma_kernel<6>, grid, dim3(256), 0, s, f);
      else if (steps % 2 == 0)
        hipLaunchKernelGGL(restore_fold_mfma_kernel<2>, grid, dim3(256), 0, s, f);
      else
        hipLaunchKernelGGL(restore_fold_mfma_kernel<1>, grid, dim3(256), 0, s, f);
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
