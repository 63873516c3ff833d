// The ConvFusion 3x3 compressing conv (page "EDiT: Efficient Diffusion
// Transformers with Linear Compressed Attention", ICCV 2025 notes, section
// "ConvFusion": Conv3x3(X), C -> C/r, on the token grid) as an implicit GEMM
// whose K steps are one kernel row of one 64-channel slice, bf16 in and out,
// fp32 accumulation on the 32x32x16 matrix cores.
//
// A tile is 256 consecutive output pixels (R = 256 / L image rows of L
// pixels, L = W for W <= 256, else a 256-pixel segment of one row) x 96
// output channels. K step (s, ky) covers input channels 64 s .. 64 s + 63
// and the three taps (ky, 0..2); its LDS stage holds
//   - A: the R input rows y + ky - 1 of the tile's rows y, each with one
//     pixel more on either side (R (L + 2) pixels of 128 bytes; pixels
//     outside the image read at an offset beyond the buffer resource, so the
//     hardware supplies the zero padding), and
//   - B: the weights of the three taps, rows kx * 96 + output channel.
// Tap (ky, kx) reads its A fragments from the same rows shifted by kx
// pixels, so the input is fetched once per kernel row instead of once per
// tap: against a K step of one tap, ~1.8x fewer bytes and cache lines are
// loaded per matrix-core flop, and every load instruction still moves whole
// 128-byte lines (8 rows of 16 lanes x 16 bytes).
// Pipeline, epilogue (bias, GroupNorm partial statistics of the stored tile,
// 16-byte stores after a half-wave exchange) and the restore-fold blocks
// follow gemm_dma.hip: two 72 KiB stages filled by direct global-to-LDS
// loads, one barrier per K step before its last sub-step.
#include "common.hpp"
#include "launch.hpp"

namespace edit {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr;
constexpr uint32_t kOobH = 0x80000000u;   // beyond every resource used here: loads return zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t halo_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// vmcnt(VM), all LDS reads of this wave done, then the block barrier.
template <int VM>
__device__ __forceinline__ void halo_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t other_half(uint32_t v, bool upper) {
  const auto pr = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return upper ? pr[0] : pr[1];
}

}  // namespace

// Stage geometry for tile rows of L pixels: 8 rows of 128 bytes per load instruction.
template <int L>
struct RowsGeom {
  static constexpr int R = 256 / L;                  // image rows per tile
  static constexpr int AW = L + 2;                   // A row length in pixels
  static constexpr int AROWS = R * AW;               // A rows (pixels) used
  static constexpr int BI = 36;                      // load instructions of B: 3 taps x 96 rows / 8
  static constexpr int NI = ((AROWS + 7) / 8 + BI + 3) / 4 * 4;   // per stage, a multiple of the 4 waves
  static constexpr int AI = NI - BI;                 // of A (the last ones partly padding)
  static constexpr int NPER = NI / 4;                // per wave
  static constexpr int STAGE = NI * 1024;
  static_assert(256 % L == 0 && L % 32 == 0, "tile rows");
  static_assert(NPER < 64, "vmcnt range");
};

template <int L, int EM>
__global__ __launch_bounds__(256, 1) void conv3x3_rows_kernel(GemmArgs<bf16> p, int ntiles) {
#if defined(__HIP_DEVICE_COMPILE__)
  using G = RowsGeom<L>;
  constexpr int BN = 96, WM = 4, TI = 2, CJ = 3, NPER = G::NPER;
  static_assert(2 * G::STAGE + (EM == E_BIAS_GN ? (WM + 1) * BN * 4 : 0) <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char S0[G::STAGE];
  __shared__ __attribute__((aligned(16))) char S1[G::STAGE];
  __shared__ float gnred[EM == E_BIAS_GN ? WM * BN : 1];
  __shared__ float gnmean[EM == E_BIAS_GN ? BN : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // The last fold_blocks blocks compute the restore fold (fold.hpp) on CUs the tiles leave idle.
  const int nblk = (int)gridDim.x - p.fold_blocks;
  if ((int)blockIdx.x >= nblk) {
    float(*red)[32][33] = reinterpret_cast<float(*)[32][33]>(S0);
    const int fb = (int)blockIdx.x - nblk, steps = p.fold.C / 64;
    if (steps % 18 == 0) fold_blocks<18>(p.fold, fb, p.fold_blocks, red);
    else if (steps % 6 == 0) fold_blocks<6>(p.fold, fb, p.fold_blocks, red);
    else if (steps % 2 == 0) fold_blocks<2>(p.fold, fb, p.fold_blocks, red);
    else fold_blocks<1>(p.fold, fb, p.fold_blocks, red);
    return;
  }
  const int Cin = p.Cin, H = p.H, W = p.W;
  const int tiles_n = p.N / BN;
  const int nk = 3 * (Cin / 64);                     // K step kt: slice kt / 3, kernel row kt % 3
  const __amdgpu_buffer_rsrc_t rsX = halo_rsrc(p.A, (uint32_t)((size_t)p.M * Cin * 2));
  const __amdgpu_buffer_rsrc_t rsW = halo_rsrc(p.Bseg[0], (uint32_t)((size_t)p.N * p.ldb * 2));
  const int fr = lane & 31, fh = lane >> 5;

  // Fragment addresses within a stage (the same for every tile and K step). Row r of a stage region
  // holds its 64 channels as 16-byte chunks, chunk c at position c ^ ((r >> 1) & 7) (16 consecutive
  // rows then read all LDS banks once). Sub-step (kx, j) reads K values 16 j .. 16 j + 15: lanes
  // 0..31 chunk 2j, lanes 32..63 chunk 2j + 1.
  // A: output pixel wave * 64 + 32 ti + fr of the tile shifted by kx.
  uint32_t xa[TI][3][4];
#pragma unroll
  for (int ti = 0; ti < TI; ++ti) {
    const int pl = wave * 64 + ti * 32 + fr, r = pl / L, c = pl % L;
#pragma unroll
    for (int kx = 0; kx < 3; ++kx) {
      const int row = r * G::AW + c + kx;
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[ti][kx][j] = (uint32_t)row * 128u + (uint32_t)(((2 * j + fh) ^ ((row >> 1) & 7)) << 4);
    }
  }
  // B: row kx * 96 + 32 cj + fr after A; (row >> 1) & 7 = (fr >> 1) & 7.
  uint32_t wb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wb[j] = (uint32_t)G::AI * 1024u + (uint32_t)fr * 128u + (uint32_t)(((2 * j + fh) ^ ((fr >> 1) & 7)) << 4);

  // Per tile: the load offsets of this wave's instructions k = wave + 4 i (k < AI: A rows 8 k ..
  // 8 k + 7, else B rows 8 (k - AI) ..), lane l filling row l >> 3, chunk position l & 7. An A row's
  // offset is that of its pixel in kernel row 1 (the tile's own image row, always inside the image);
  // kernel row ky moves it by ky - 1 image rows, and amask bit ky says whether that pixel lies inside
  // the image (else the load reads zeros at an offset past the resource).
  static_assert(G::AI % 4 == 0, "every wave issues AI / 4 A loads first, then B loads");
  constexpr int NA = G::AI / 4;                      // i < NA: A rows, else B rows (for every wave)
  static_assert(3 * NA <= 32, "amask bits");
  int m0 = 0, n0 = 0;
  uint32_t doff[NPER], amask = 0;                    // bits 3i .. 3i + 2: kernel rows 0..2 of A load i
#define EDIT_ROWS_TILE(tl_)                                                                        \
  do {                                                                                            \
    const int tile_ = xcd_swizzle((tl_), ntiles);                                                 \
    m0 = (tile_ / tiles_n) * 256;                                                                 \
    n0 = (tile_ % tiles_n) * BN;                                                                  \
    const int b_ = m0 / (H * W), q_ = m0 - b_ * H * W, y0_ = q_ / W, x0_ = q_ - y0_ * W;          \
    _Pragma("unroll") for (int i = 0; i < NPER; ++i) {                                            \
      const int k = wv + 4 * i;                                                                   \
      const int pos = lane & 7;                                                                   \
      if (i < NA) {                                                                               \
        const int row = 8 * k + (lane >> 3), c = pos ^ ((row >> 1) & 7);                         \
        const int r = row / G::AW, cc = row - r * G::AW;                                          \
        const int y = y0_ + r, x = x0_ - 1 + cc;                                                  \
        if (i == 0) amask = 0;                                                                    \
        const bool ok_ = row < G::AROWS && x >= 0 && x < W;                                       \
        if (ok_) {                                                                                \
          _Pragma("unroll") for (int ky = 0; ky < 3; ++ky)                                        \
            if (y + ky - 1 >= 0 && y + ky - 1 < H) amask |= 1u << (3 * i + ky);                   \
        }                                                                                         \
        doff[i] = ok_ ? (uint32_t)((b_ * H + y) * W + x) * (uint32_t)(Cin * 2) + (uint32_t)(c * 16) : 0u; \
      } else {                                                                                    \
        const int row = 8 * (k - G::AI) + (lane >> 3), c = pos ^ ((row >> 1) & 7);               \
        const int kx = row / BN, co = row - kx * BN;                                              \
        doff[i] = (uint32_t)(n0 + co) * (uint32_t)(p.ldb * 2) + (uint32_t)(kx * Cin * 2 + c * 16); \
      }                                                                                           \
    }                                                                                             \
  } while (0)
  // K step kt's loads into stage S: slice kt / 3 and kernel row kt % 3 are uniform offsets (A: ky
  // image rows and 128 bytes per slice; B: 3 ky taps and 128 bytes per slice).
#define EDIT_ROWS_DMA(S, kt_)                                                                      \
  do {                                                                                            \
    const int sl_ = (kt_) / 3, ky_ = (kt_) - 3 * sl_;                                             \
    const uint32_t soA_ = (uint32_t)sl_ * 128u;                                                   \
    const int kyo_ = (ky_ - 1) * W * Cin * 2;          /* in bounds wherever amask allows the load */ \
    const uint32_t soB_ = (uint32_t)sl_ * 128u + (uint32_t)(3 * ky_ * Cin * 2);                   \
    _Pragma("unroll") for (int i = 0; i < NPER; ++i) {                                            \
      const int k = wv + 4 * i;                                                                   \
      if (i < NA) {                                                                               \
        const uint32_t v_ = ((amask >> (3 * i + ky_)) & 1u) ? (uint32_t)((int)doff[i] + kyo_) : kOobH; \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsX, (lds_ptr)((S) + 1024 * k), 16, v_, soA_, 0, 0); \
      } else {                                                                                    \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, (lds_ptr)((S) + 1024 * k), 16, doff[i], soB_, 0, 0); \
      }                                                                                           \
    }                                                                                             \
  } while (0)

  f32x16 acc[TI][CJ];
  bf16x8 xf[2][TI], wf[2][CJ];
  bf16x4 bv[CJ][4];

  // sub-step u = 4 kx + j of a K step
#define EDIT_ROWS_READ(S, u_, set_)                                                                \
  do {                                                                                            \
    _Pragma("unroll") for (int ti = 0; ti < TI; ++ti)                                             \
      xf[set_][ti] = *reinterpret_cast<const bf16x8*>((S) + xa[ti][(u_) >> 2][(u_) & 3]);         \
    _Pragma("unroll") for (int c = 0; c < CJ; ++c)                                                \
      wf[set_][c] = *reinterpret_cast<const bf16x8*>((S) + wb[(u_) & 3] + (((u_) >> 2) * BN + c * 32) * 128); \
  } while (0)
#define EDIT_ROWS_MMA(set_)                                                                        \
  do {                                                                                            \
    _Pragma("unroll") for (int ti = 0; ti < TI; ++ti)                                             \
      _Pragma("unroll") for (int c = 0; c < CJ; ++c)                                              \
        acc[ti][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[set_][c], xf[set_][ti], acc[ti][c], 0, 0, 0); \
  } while (0)
  // each matrix-core step followed by one fragment read of the next sub-step and, in the refill
  // sub-step, LPM of the loads
  constexpr int NM = TI * CJ, NR = TI + CJ, LPM = (NPER + NM - 1) / NM;
#define EDIT_ROWS_PIN(NV)                                                                          \
  do {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < NM; ++i) {                                              \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                          \
      if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              \
      if (LPM * i < (NV)) __builtin_amdgcn_sched_group_barrier(0x020, LPM, 0);                     \
    }                                                                                             \
    __builtin_amdgcn_sched_barrier(0);                                                            \
  } while (0)
#define EDIT_ROWS_SUB(S, u_, nxt_, cur_)                                                           \
  do {                                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    EDIT_ROWS_READ(S, u_, nxt_);                                                                  \
    EDIT_ROWS_MMA(cur_);                                                                          \
    EDIT_ROWS_PIN(0);                                                                             \
  } while (0)
  // Sub-steps 1 .. 11 of the step on stage SC (sub-step 0's fragments are in set 0 on entry).
#define EDIT_ROWS_HEAD(SC)                                                                         \
  EDIT_ROWS_SUB(SC, 1, 1, 0);                                                                     \
  EDIT_ROWS_SUB(SC, 2, 0, 1);                                                                     \
  EDIT_ROWS_SUB(SC, 3, 1, 0);                                                                     \
  EDIT_ROWS_SUB(SC, 4, 0, 1);                                                                     \
  EDIT_ROWS_SUB(SC, 5, 1, 0);                                                                     \
  EDIT_ROWS_SUB(SC, 6, 0, 1);                                                                     \
  EDIT_ROWS_SUB(SC, 7, 1, 0);                                                                     \
  EDIT_ROWS_SUB(SC, 8, 0, 1);                                                                     \
  EDIT_ROWS_SUB(SC, 9, 1, 0);                                                                     \
  EDIT_ROWS_SUB(SC, 10, 0, 1);                                                                    \
  EDIT_ROWS_SUB(SC, 11, 1, 0);
  // Two stages: at the barrier step kk + 1 has landed (nothing else is in flight) and every wave is
  // done reading SC, which is then refilled with step kk + 2.
#define EDIT_ROWS_FULL(SC, SN, kk)                                                                 \
  do {                                                                                            \
    EDIT_ROWS_HEAD(SC)                                                                            \
    halo_barrier<0>();                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    EDIT_ROWS_READ(SN, 0, 0);                                                                     \
    EDIT_ROWS_DMA(SC, (kk) + 2);                                                                  \
    EDIT_ROWS_MMA(1);                                                                             \
    EDIT_ROWS_PIN(NPER);                                                                          \
  } while (0)
#define EDIT_ROWS_TAIL(SC, SN, kk)                                                                 \
  do {                                                                                            \
    EDIT_ROWS_HEAD(SC)                                                                            \
    halo_barrier<0>();                                                                            \
    if ((kk) + 2 < nk) EDIT_ROWS_DMA(SC, (kk) + 2);                                               \
    if ((kk) + 1 < nk) EDIT_ROWS_READ(SN, 0, 0);                                                  \
    EDIT_ROWS_MMA(1);                                                                             \
  } while (0)

  int tl = blockIdx.x;
  EDIT_ROWS_TILE(tl);
  EDIT_ROWS_DMA(S0, 0);
  if (nk > 1) EDIT_ROWS_DMA(S1, 1);
  for (;;) {
    // the tile's bias, requested before anything else is queued behind it
#pragma unroll
    for (int c = 0; c < CJ; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = c * 32 + 8 * g + 4 * fh;
        bv[c][g] = *reinterpret_cast<const bf16x4*>(p.bias[0] + n0 + nl);
      }
#pragma unroll
    for (int t = 0; t < TI; ++t)
#pragma unroll
      for (int c = 0; c < CJ; ++c) acc_zero(acc[t][c]);
    // step 0 landed (the previous tile's stores may still be outstanding behind this tile's loads)
    if (nk > 1) halo_barrier<NPER>();
    else halo_barrier<0>();
    EDIT_ROWS_READ(S0, 0, 0);
    int kt = 0;
    for (; kt + 3 < nk; kt += 2) {
      EDIT_ROWS_FULL(S0, S1, kt);
      EDIT_ROWS_FULL(S1, S0, kt + 1);
    }
    EDIT_ROWS_TAIL(S0, S1, kt);
    if (kt + 1 < nk) EDIT_ROWS_TAIL(S1, S0, kt + 1);
    if (kt + 2 < nk) EDIT_ROWS_TAIL(S0, S1, kt + 2);

    // The stages are free: queue the next tile's first two steps, then write this tile.
    const int em0 = m0, en0 = n0;
    // E_RES: the residual rows at this lane's store positions (as the exchanged stores below: token l & 31,
    // 8 channels from 32 c + 16 j + 8 (l >> 5)), requested before the next tile's loads
    uint4 rres[EM == E_RES ? TI : 1][EM == E_RES ? CJ : 1][2];
    if constexpr (EM == E_RES) {
#pragma unroll
      for (int t = 0; t < TI; ++t)
#pragma unroll
        for (int c = 0; c < CJ; ++c)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            rres[t][c][j] = *reinterpret_cast<const uint4*>(p.R + (size_t)(em0 + wave * 64 + t * 32 + fr) * p.ldr +
                                                            en0 + c * 32 + 16 * j + 8 * fh);
    }
    const int next = tl + nblk;
    if (next < ntiles) {
      EDIT_ROWS_TILE(next);
      EDIT_ROWS_DMA(S0, 0);
      if (nk > 1) EDIT_ROWS_DMA(S1, 1);
    }
    // bias, then 16-byte stores: accumulator quad g of lane l holds channels 8g + 4(l >> 5) .. +3 of
    // token l & 31; lanes l and l ^ 32 swap halves so that each stores 8 consecutive channels.
#pragma unroll
    for (int t = 0; t < TI; ++t) {
      const int m = em0 + wave * 64 + t * 32 + fr;
#pragma unroll
      for (int c = 0; c < CJ; ++c) {
        float f[4][4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) f[g][i] = acc[t][c][4 * g + i] + (float)bv[c][g][i];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int ge = 2 * j, go = 2 * j + 1;
          const int n = en0 + c * 32 + 8 * (fh ? go : ge);
          if constexpr (EM == E_RES) {
            // fp32 halves exchanged, the residual added, one rounding: lane half 0 holds channels n .. n + 3 of
            // its own and n + 4 .. n + 7 of its partner's, half 1 the partner's n .. n + 3 and its own
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float sv = fh ? f[ge][i] : f[go][i];
              const float rv = __builtin_bit_cast(float, other_half(__builtin_bit_cast(uint32_t, sv), fh));
              v[fh ? i : 4 + i] = rv;
              v[fh ? 4 + i : i] = fh ? f[go][i] : f[ge][i];
            }
            const bf16* rb = reinterpret_cast<const bf16*>(&rres[t][c][j]);
            bf16x8 o8;
#pragma unroll
            for (int k = 0; k < 8; ++k) o8[k] = (bf16)(v[k] + (float)rb[k]);
            *reinterpret_cast<bf16x8*>(p.C + (size_t)m * p.ldc + n) = o8;
            continue;
          }
          uint32_t pk[2][2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            bf16x4 b4;
#pragma unroll
            for (int i = 0; i < 4; ++i) b4[i] = (bf16)f[hh ? go : ge][i];
            pk[hh][0] = reinterpret_cast<const uint32_t*>(&b4)[0];
            pk[hh][1] = reinterpret_cast<const uint32_t*>(&b4)[1];
          }
          const uint32_t s0 = fh ? pk[0][0] : pk[1][0];
          const uint32_t s1 = fh ? pk[0][1] : pk[1][1];
          const uint32_t r0 = other_half(s0, fh);
          const uint32_t r1 = other_half(s1, fh);
          uint32_t w[4];
          w[0] = fh ? r0 : pk[0][0];
          w[1] = fh ? r1 : pk[0][1];
          w[2] = fh ? pk[1][0] : r0;
          w[3] = fh ? pk[1][1] : r1;
          *reinterpret_cast<uint4*>(p.C + (size_t)m * p.ldc + n) = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
    if (EM == E_BIAS_GN) {
      // GroupNorm partial statistics of the tile as stored (bf16), per column over its 256 rows (after the
      // stores are issued, so that they drain meanwhile): the exact mean, then the sum of squared deviations
      // from it (as gemm_dma.hip's statistics epilogue: lane sums, four row-local DPP levels, the 16-lane row
      // swap, the waves through LDS).
      auto stored = [&](int t, int c, int k) -> float {
        return (float)(bf16)(acc[t][c][k] + (float)bv[c][k >> 2][k & 3]);
      };
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        float sm[CJ * 16];
#pragma unroll
        for (int c = 0; c < CJ; ++c)
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const float mu = pass ? gnmean[c * 32 + 8 * (k >> 2) + 4 * fh + (k & 3)] : 0.0f;
            float v = 0.0f;
#pragma unroll
            for (int t = 0; t < TI; ++t) {
              const float d = stored(t, c, k) - mu;
              v += pass ? d * d : d;
            }
            sm[c * 16 + k] = v;
          }
#define EDIT_HALO_DPP(CTRL)                                                                        \
        _Pragma("unroll") for (int j = 0; j < CJ * 16; ++j)                                       \
          sm[j] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                          \
              0, __builtin_bit_cast(int, sm[j]), (CTRL), 0xF, 0xF, false));
        EDIT_HALO_DPP(0xB1)
        EDIT_HALO_DPP(0x4E)
        EDIT_HALO_DPP(0x141)
        EDIT_HALO_DPP(0x140)
#undef EDIT_HALO_DPP
#pragma unroll
        for (int j = 0; j < CJ * 16; ++j) {
          const uint32_t u = __builtin_bit_cast(uint32_t, sm[j]);
          const auto pr = __builtin_amdgcn_permlane16_swap(u, u, false, false);
          sm[j] += __builtin_bit_cast(float, (lane & 16) ? pr[0] : pr[1]);
        }
        if (fr == 0) {
#pragma unroll
          for (int c = 0; c < CJ; ++c)
#pragma unroll
            for (int k = 0; k < 16; ++k) gnred[wave * BN + c * 32 + 8 * (k >> 2) + 4 * fh + (k & 3)] = sm[c * 16 + k];
        }
        halo_barrier<63>();   // LDS only: the next tile's loads stay in flight
        if (tid < BN) {
          float v = 0.0f;
#pragma unroll
          for (int w = 0; w < WM; ++w) v += gnred[w * BN + tid];
          if (pass == 0) {
            gnmean[tid] = v / 256.0f;
          } else {
            float* o = p.gnp + ((size_t)(em0 / 256) * p.N + en0 + tid) * 2;
            o[0] = gnmean[tid];
            o[1] = v;
          }
        }
        halo_barrier<63>();
      }
    }
    if (next >= ntiles) break;
    tl = next;
  }
#undef EDIT_ROWS_TAIL
#undef EDIT_ROWS_FULL
#undef EDIT_ROWS_HEAD
#undef EDIT_ROWS_SUB
#undef EDIT_ROWS_PIN
#undef EDIT_ROWS_MMA
#undef EDIT_ROWS_READ
#undef EDIT_ROWS_DMA
#undef EDIT_ROWS_TILE
#endif  // __HIP_DEVICE_COMPILE__
}

namespace {
template <int L, int EM>
hipError_t launch_rows_tiles(const GemmArgs<bf16>& a, hipStream_t s) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const int ntiles = (a.M / 256) * (a.N / 96);
  const int g8 = cus / 8 * 8;
  const int blocks = ntiles <= g8 || a.spread ? ntiles : g8;
  GemmArgs<bf16> b = a;
  b.fold_blocks = 0;
  // the restore fold rides along where the tiles leave at least 16 CUs idle; otherwise it runs after
  const bool fold_here = a.fold.W != nullptr && a.fold.C % 64 == 0 && a.fold.Cr % 32 == 0 && blocks + 16 <= cus;
  if (fold_here) b.fold_blocks = cus - blocks;
  hipLaunchKernelGGL((conv3x3_rows_kernel<L, EM>), dim3(blocks + b.fold_blocks), dim3(256), 0, s, b, ntiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.fold.W == nullptr || fold_here) return e;
  const FoldArgs& f = a.fold;
  return launch_restore_fold<bf16>(f.W, f.b, f.W2, f.b2, f.C, f.Cr, f.wcat, f.bcat, s);
}
}  // namespace

hipError_t launch_conv3x3_halo(const GemmArgs<bf16>& a, EMode em, hipStream_t s) {
  if (em != E_BIAS && em != E_BIAS_GN && em != E_RES) return hipErrorNotSupported;
  if ((em == E_RES) != (a.R != nullptr) || a.Cin % 64 != 0 || a.lda != a.Cin || a.K != 9 * a.Cin ||
      a.ldb != 9 * a.Cin)
    return hipErrorNotSupported;
  if (em == E_RES && (a.ldr % 8 != 0 || a.fold.W != nullptr)) return hipErrorNotSupported;
  if (a.N % 96 != 0 || a.seg_rows != a.N || a.ldc % 8 != 0 || a.ldc < a.N) return hipErrorNotSupported;
  const long hw = (long)a.H * a.W;
  if (hw % 256 != 0 || a.M % hw != 0) return hipErrorNotSupported;
  if (em == E_BIAS_GN && (a.gnp == nullptr || a.gn_rows != 256)) return hipErrorNotSupported;
  // 32-bit buffer offsets stay below the out-of-range marker
  if ((size_t)a.M * a.Cin * 2 >= kOobH || (size_t)a.N * a.ldb * 2 >= kOobH) return hipErrorNotSupported;
  const int L = a.W <= 256 ? a.W : 256;
  if (a.W > 256 && a.W % 256 != 0) return hipErrorNotSupported;
#define EDIT_HALO_CASE(LV)                                                                       \
  if (L == LV)                                                                                    \
    return em == E_BIAS_GN ? launch_rows_tiles<LV, E_BIAS_GN>(a, s)                               \
                           : (em == E_RES ? launch_rows_tiles<LV, E_RES>(a, s) : launch_rows_tiles<LV, E_BIAS>(a, s));
  EDIT_HALO_CASE(32)
  EDIT_HALO_CASE(64)
  EDIT_HALO_CASE(128)
  EDIT_HALO_CASE(256)
#undef EDIT_HALO_CASE
  return hipErrorNotSupported;
}

}  // namespace edit
