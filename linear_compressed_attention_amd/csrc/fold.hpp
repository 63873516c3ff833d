// The ConvFusion 1x1 restore folded into the Linear that reads its output:
// the bf16 matrix-core work of one 32 x 32 tile, shared by the fold's own
// kernel and by the direct-load conv, which runs it on CUs its tiles leave
// idle.
//
// Page "EDiT: Efficient Diffusion Transformers with Linear Compressed
// Attention" (ICCV 2025 notes), section "ConvFusion": the query Linear reads
// X + Conv1x1(act); a 1x1 convolution is a Linear over channels, so
//   (X + act W2^T + b2) W^T + b = [X | act] [W | W W2]^T + (b + W b2).
// wcat [C][C + Cr] = [W | W W2], bcat [C] = b + W b2 (fp32 sums, one rounding).
#pragma once
#include "common.hpp"

namespace edit {

struct FoldArgs {
  const bf16* W;     // [C][C]
  const bf16* b;     // [C]
  const bf16* W2;    // [C][Cr]
  const bf16* b2;    // [Cr]
  bf16* wcat;        // [C][C + Cr]
  bf16* bcat;        // [C]
  int C, Cr;
};

// Tiles of the fold: (C / 32) x (Cr / 32 + 1); tile column Cr / 32 holds b2
// in its first column, so W b2 comes from the same matrix-core steps.
__device__ __forceinline__ int fold_tiles(const FoldArgs& f) { return (f.C / 32) * (f.Cr / 32 + 1); }

// One 32 x 32 tile of W [W2 | b2 | 0 ...] with 256 threads (C % 64 == 0,
// Cr % 32 == 0): the four waves split the depth C in quarters (32x32x16
// steps; R steps of loads issued before their matrix work, R divides C / 64)
// and add their partial tiles through red (4 x 32 x 33 floats of LDS).
// Lane l feeds row l % 32 of W (first operand) and column l % 32 of W2
// (second operand), K values 8(l / 32) .. +7 of each 16-deep step.
template <int R>
__device__ __forceinline__ void fold_tile(const FoldArgs& f, int tile, float (*red)[32][33]) {
  const int ldw = f.C + f.Cr;
  const int tiles_j = f.Cr / 32 + 1;
  const int it = tile / tiles_j, jt = tile % tiles_j;
  const bool bias_tile = jt == tiles_j - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int kq = f.C / 4, k0 = wave * kq, k1 = k0 + kq;
  const bf16* wrow = f.W + (size_t)(it * 32 + fr) * f.C + 8 * fh;
  const bf16* col = bias_tile ? f.b2 + 8 * fh : f.W2 + (size_t)(8 * fh) * f.Cr + jt * 32 + fr;
  const size_t stride = bias_tile ? 1 : (size_t)f.Cr;
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
  // accumulator element 4g + e is (row 8g + 4fh + e, column fr) of the tile
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
      f.wcat[(size_t)(it * 32 + i) * ldw + f.C + jt * 32 + j] = (bf16)s;
    }
  } else if (tid < 32) {
    const float s = red[0][tid][0] + red[1][tid][0] + red[2][tid][0] + red[3][tid][0];
    f.bcat[it * 32 + tid] = (bf16)((float)f.b[it * 32 + tid] + s);
  }
  __syncthreads();   // red is free for the next tile
}

// [W | .] part of wcat: 16-byte chunks, chunk idx of every stride-th from
// first; eight loads are in flight before their stores.
__device__ __forceinline__ void fold_copy(const FoldArgs& f, int first, int stride) {
  constexpr int U = 8;
  const int ldw = f.C + f.Cr, cpr = f.C / 8, total = f.C * cpr;
  for (int base = first; base < total; base += U * stride) {
    bf16x8 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * stride;
      if (idx < total) {
        const int r = idx / cpr, c8 = idx - r * cpr;
        v[u] = *reinterpret_cast<const bf16x8*>(f.W + (size_t)r * f.C + 8 * c8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * stride;
      if (idx < total) {
        const int r = idx / cpr, c8 = idx - r * cpr;
        *reinterpret_cast<bf16x8*>(f.wcat + (size_t)r * ldw + 8 * c8) = v[u];
      }
    }
  }
}

// The whole fold by the blocks fb = 0 .. nb - 1 of a grid (256 threads each).
template <int R>
__device__ __forceinline__ void fold_blocks(const FoldArgs& f, int fb, int nb, float (*red)[32][33]) {
  for (int t = fb; t < fold_tiles(f); t += nb) fold_tile<R>(f, t, red);
  fold_copy(f, fb * 256 + (int)threadIdx.x, nb * 256);
}

}  // namespace edit
