// MFMA GEMM for gfx950 with direct global-to-LDS tile loads:
// C[M][N] = A[M][K] * B[N][K]^T (+ bias, optional ReLU), bf16 in and out,
// fp32 accumulation. A is plain rows, two row sources side by side along K,
// or an implicit 3x3 stride-1 pad-1 convolution over a channels-last image.
//
// Serves the dense steps of the EDiT layer ("EDiT: Efficient Diffusion
// Transformers with Linear Compressed Attention" notes): the ConvFusion 3x3
// compressing conv, the query Linear over [X | act] with the 1x1 restore
// folded into its weights (section "ConvFusion"), the key and value Linears
// (section "Spatial Compressor"), the output Linear and the hybrid's text
// Linears (section "MM-EDiT").
//
// Design (4-wave blocks):
//  - Tiles move from HBM/L2 straight into LDS with buffer_load ... lds (16
//    bytes per lane, no register round trip), through a ring of ST stages
//    held in distinct LDS arrays, so that the compiler can tell which stage
//    a fragment read touches and waits only for that stage's loads.
//  - ST = 3 (one block per CU, up to 160 KB): two K steps are in flight
//    while a third is multiplied; the block walks several tiles and queues
//    the next tile's first steps before it writes the current one.
//  - ST = 2 (two blocks per CU, at most 80 KB each, one block per tile):
//    one K step is in flight while the other is multiplied, and the CU's
//    second block covers the wait, the prologue and the epilogue, so every
//    SIMD runs two waves. Measured on MI355X with 128 x 192 tiles: 46 us
//    against 53 us (three stages, persistent) at 16384 x 1152 x 1152,
//    91 against 110 us at 16384 x 2304 x 1152.
//  - Out-of-range rows, and the zero padding of the convolution, read at an
//    offset beyond the buffer resource: the hardware returns zeros, so the
//    loads never branch.
//  - An LDS row is 128 bytes (64 bf16 of K); chunk c of row r sits at
//    position c ^ ((r >> 1) & 7). A DMA instruction fills 8 whole rows, so
//    each lane fetches the chunk that belongs at its fixed LDS position.
//  - 32x32x16 matrix-core steps with the weights as the first operand: an
//    accumulator then holds 4 consecutive output channels of one token. The
//    epilogue pairs the quads of lanes l and l ^ 32 (v_permlane32_swap) so
//    that every lane stores 8 consecutive channels with one 16-byte write.
//  - One barrier per K step, placed before the last quarter of the step's
//    matrix work: by then every wave holds that quarter's fragments in
//    registers, so the stage can be refilled while the quarter runs.
#include "common.hpp"
#include "launch.hpp"

namespace edit {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr;
constexpr uint32_t kOob = 0x80000000u;   // beyond every resource used here: loads return zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer (stride 0); dword 3 selects 32-bit data, the gfx9 default.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Wait until at most VM of this wave's vector-memory loads are outstanding and
// all of its LDS reads are done, then barrier the block. The empty asm
// statements keep the compiler from moving memory accesses across.
template <int VM>
__device__ __forceinline__ void stage_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));   // vmcnt(VM) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The value lane l ^ 32 holds: one v_permlane32_swap exchanges the two
// halves of the wave (no LDS crossbar round trip).
__device__ __forceinline__ uint32_t from_other_half(uint32_t v, bool upper) {
  const auto pr = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return upper ? pr[0] : pr[1];
}

template <typename P>
__device__ __forceinline__ P pick_seg(const P (&a)[3], int i) {
  return i == 0 ? a[0] : (i == 1 ? a[1] : a[2]);
}

}  // namespace

// Blocks resident per CU: two-stage 4-wave blocks pair up; 8-wave blocks and
// three-stage blocks run alone (still two waves per SIMD for 8 waves).
template <int NW, int ST>
constexpr int dma_blocks_per_cu() { return ST == 2 && NW <= 4 ? 2 : 1; }

template <int BM, int BN, int WM, int WN, int AM, int EM, int ST>
__global__ __launch_bounds__(64 * WM * WN, (dma_blocks_per_cu<WM * WN, ST>())) void gemm_dma_kernel(GemmArgs<bf16> p,
                                                                                                     int ntiles) {
  // The body uses gfx950-only types (buffer resources), which the host pass
  // cannot instantiate; it only needs the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;     // tokens x channels per wave
  constexpr int TI = WTM / 32, CJ = WTN / 32;     // 32 x 32 blocks per wave
  constexpr int NA = BM / (8 * NW), NB = BN / (8 * NW);   // DMA instructions per wave per stage
  constexpr int NPER = NA + NB;
  constexpr int STAGE = (BM + BN) * 128;          // bytes per stage
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0 && WTM % 32 == 0 && WTN % 32 == 0, "tile");
  static_assert(BM % 16 == 0, "B rows keep the swizzle phase of their LDS row");
  static_assert(ST * STAGE <= 160 * 1024 / dma_blocks_per_cu<NW, ST>(), "LDS");
  static_assert(2 * NPER < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char S0[STAGE];
  __shared__ __attribute__((aligned(16))) char S1[STAGE];
  __shared__ __attribute__((aligned(16))) char S2[ST == 3 ? STAGE : 16];
  // E_BIAS_GN: per-wave column sums, then the tile's column means.
  static_assert(EM != E_BIAS_GN || WN == 1, "the statistics epilogue has every wave on all BN columns");
  __shared__ float gnred[EM == E_BIAS_GN ? WM * BN : 1];
  __shared__ float gnmean[EM == E_BIAS_GN ? BN : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  // The last fold_blocks blocks of a conv launch compute the restore fold
  // (fold.hpp) on CUs the conv's tiles leave idle; their LDS holds the
  // fold's partial tiles instead of stages.
  const int nblk = (int)gridDim.x - (AM == A_CONV3 ? p.fold_blocks : 0);
  if (AM == A_CONV3 && (int)blockIdx.x >= nblk) {
    float(*red)[32][33] = reinterpret_cast<float(*)[32][33]>(S0);
    const int fb = (int)blockIdx.x - nblk, steps = p.fold.C / 64;
    if (steps % 18 == 0) fold_blocks<18>(p.fold, fb, p.fold_blocks, red);
    else if (steps % 6 == 0) fold_blocks<6>(p.fold, fb, p.fold_blocks, red);
    else if (steps % 2 == 0) fold_blocks<2>(p.fold, fb, p.fold_blocks, red);
    else fold_blocks<1>(p.fold, fb, p.fold_blocks, red);
    return;
  }
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles_mn = ((p.M + BM - 1) / BM) * tiles_n;
  // K steps of the current tile; E_F32 (split K): tile index = split * tiles_mn
  // + output tile, the split covering K range [kb, kb + ktot).
  int nk = AM == A_CONV3 ? 9 * (p.Cin / 64) : (p.K + 63) / 64;
  int ktot = p.K, split = 0;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.A, (uint32_t)((size_t)p.M * p.lda * 2));
  // A_CAT2: K steps 0 .. nk1-1 read A, the rest read A2 (K1 is a multiple of 64).
  const __amdgpu_buffer_rsrc_t rsA2 = make_rsrc(AM == A_CAT2 ? p.A2 : p.A,
                                                (uint32_t)((size_t)p.M * (AM == A_CAT2 ? p.lda2 : p.lda) * 2));
  const int nk1 = AM == A_CAT2 ? p.K1 / 64 : nk;

  // Lane l fills chunk (l & 7) of row (l >> 3) of an 8-row DMA group and
  // fetches the logical chunk stored there.
  const int lr = lane >> 3, pc = lane & 7;
  // The logical chunk a lane fetches, for 8-row groups of even and odd index
  // (row r = 8g + lr is stored with phase (r >> 1) & 7 = (4g + lr / 2) & 7).
  const int cl0 = pc ^ (lr >> 1), cl1 = pc ^ (4 + (lr >> 1));
  // Fragment addressing: lane l reads row (l & 31) of a 32-row block, logical
  // chunk 2s + (l >> 5) for sub-step s (16 K values each).
  const int fr = lane & 31, fh = lane >> 5;
  int fo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fo[s] = fr * 128 + (((2 * s + fh) ^ ((fr >> 1) & 7)) << 4);
  const int xrow = (wm * WTM) * 128;          // this wave's token rows (A region)
  const int wrow = (BM + wn * WTN) * 128;     // this wave's channel rows (B region)

  // Per-tile state. The block walks tiles bid, bid + G, ... (G = grid size, a
  // multiple of 8 when there is more than one round), renumbered so that each
  // XCD takes a contiguous range and its CUs work on neighbouring tiles.
  int m0, n0, nseg0;
  __amdgpu_buffer_rsrc_t rsB;
  const bf16* bias;
  uint32_t aoff[NA], boff[NB];
  uint32_t aoff2[AM == A_CAT2 ? NA : 1];
  uint32_t amask[AM == A_CONV3 ? NA : 1];
#define EDIT_SET_TILE(tl_)                                                                        \
  do {                                                                                            \
    int tile_ = xcd_swizzle((tl_), ntiles);                                                       \
    uint32_t kb_ = 0;                                                                             \
    if (EM == E_F32) {                                                                            \
      split = tile_ / tiles_mn;                                                                   \
      tile_ -= split * tiles_mn;                                                                  \
      kb_ = (uint32_t)split * (uint32_t)p.kchunk;                                                 \
      ktot = min(p.kchunk, p.K - (int)kb_);                                                       \
      nk = (ktot + 63) / 64;                                                                      \
    }                                                                                             \
    m0 = (tile_ / tiles_n) * BM;                                                                  \
    n0 = (tile_ % tiles_n) * BN;                                                                  \
    const int seg_ = n0 / p.seg_rows;   /* BN divides seg_rows */                                 \
    nseg0 = n0 - seg_ * p.seg_rows;                                                               \
    const int seg_n_ = min(p.seg_rows, p.N - seg_ * p.seg_rows);                                  \
    rsB = make_rsrc(pick_seg(p.Bseg, seg_), (uint32_t)((size_t)seg_n_ * p.ldb * 2));              \
    bias = pick_seg(p.bias, seg_) + nseg0;                                                        \
    _Pragma("unroll") for (int a = 0; a < NA; ++a) {                                              \
      const int r = 8 * (a * NW + wave) + lr;                                                     \
      const int c = pc ^ ((r >> 1) & 7);                                                          \
      const int m = m0 + r;                                                                       \
      aoff[a] = m < p.M ? (uint32_t)m * (uint32_t)p.lda * 2u + (uint32_t)c * 16u + 2u * kb_ : kOob; \
      if (AM == A_CAT2)                                                                           \
        aoff2[AM == A_CAT2 ? a : 0] = m < p.M ? (uint32_t)m * (uint32_t)p.lda2 * 2u + (uint32_t)c * 16u : kOob; \
      if (AM == A_CONV3) {                                                                        \
        /* taps (ky, kx) whose input pixel (y + ky - 1, x + kx - 1) is inside the image */       \
        uint32_t mk = 0;                                                                          \
        if (m < p.M) {                                                                            \
          const int q = m % (p.H * p.W), y = q / p.W, x = q % p.W;                                \
          _Pragma("unroll") for (int t = 0; t < 9; ++t) {                                         \
            const int yy = y + t / 3 - 1, xx = x + t % 3 - 1;                                     \
            if (yy >= 0 && yy < p.H && xx >= 0 && xx < p.W) mk |= 1u << t;                        \
          }                                                                                       \
        }                                                                                         \
        amask[AM == A_CONV3 ? a : 0] = mk;                                                        \
      }                                                                                           \
    }                                                                                             \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                              \
      const int r = 8 * (b * NW + wave) + lr;                                                     \
      const int c = pc ^ ((r >> 1) & 7);                                                          \
      boff[b] = n0 + r < p.N ? (uint32_t)(nseg0 + r) * (uint32_t)p.ldb * 2u + (uint32_t)c * 16u + 2u * kb_ : kOob; \
    }                                                                                             \
  } while (0)

  // Issue the loads of K step kt into stage S. Plain A: row offsets plus a
  // uniform K offset. Convolution: K step kt is channel slice kt / 9 of tap
  // kt % 9; the tap shifts the pixel, which may leave the image.
#define EDIT_DMA(S, kt_)                                                                          \
  do {                                                                                            \
    const int kd_ = (kt_);                                                                        \
    uint32_t sa, sb;                                                                              \
    int tap = 0, tapoff = 0;                                                                      \
    if (AM == A_CONV3) {                                                                          \
      const int sl = kd_ / 9;                                                                     \
      tap = kd_ - 9 * sl;                                                                         \
      tapoff = ((tap / 3 - 1) * p.W + (tap % 3 - 1)) * p.Cin * 2;                                 \
      sa = (uint32_t)sl * 128u;                                                                   \
      sb = (uint32_t)(tap * p.Cin + sl * 64) * 2u;                                                \
    } else {                                                                                      \
      sa = sb = (uint32_t)kd_ * 128u;                                                             \
    }                                                                                             \
    /* A_CAT2: a uniform choice of source (scalar selects, no branch) */                         \
    const bool sec_ = AM == A_CAT2 && kd_ >= nk1;                                                 \
    const __amdgpu_buffer_rsrc_t rsa_ = sec_ ? rsA2 : rsA;                                        \
    if (AM == A_CAT2) sa = (uint32_t)(sec_ ? kd_ - nk1 : kd_) * 128u;                             \
    /* K tail: chunks at or past K read zeros (A and B), so they add nothing */                  \
    const bool ktail_ = AM != A_CONV3 && kd_ * 64 + 64 > ktot;                                    \
    const int klim_ = ktot - kd_ * 64;                                                            \
    _Pragma("unroll") for (int a = 0; a < NA; ++a) {                                              \
      uint32_t v = aoff[a];                                                                       \
      if (AM == A_CONV3) v = ((amask[AM == A_CONV3 ? a : 0] >> tap) & 1u) ? v + (uint32_t)tapoff : kOob; \
      if (AM == A_CAT2 && sec_) v = aoff2[AM == A_CAT2 ? a : 0];                                  \
      if (ktail_ && 8 * (((a * NW + wave) & 1) ? cl1 : cl0) >= klim_) v = kOob;                  \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa_, (lds_ptr)((S) + 1024 * (a * NW + wave)), 16, v, \
                                               sa, 0, 0);                                         \
    }                                                                                             \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                              \
      uint32_t v = boff[b];                                                                       \
      if (ktail_ && 8 * (((b * NW + wave) & 1) ? cl1 : cl0) >= klim_) v = kOob;                  \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_ptr)((S) + BM * 128 + 1024 * (b * NW + wave)), \
                                               16, v, sb, 0, 0);                                  \
    }                                                                                             \
  } while (0)
#define EDIT_PREFETCH3()                                                                          \
  do {                                                                                            \
    EDIT_DMA(S0, 0);                                                                              \
    if (nk > 1) EDIT_DMA(S1, 1);                                                                  \
    if (ST == 3 && nk > 2) EDIT_DMA(S2, 2);                                                       \
  } while (0)

  f32x16 acc[TI][CJ];
  bf16x8 xf[2][TI], wf[2][CJ];
  bf16x4 bv[CJ][4];   // the tile's bias, fetched before the next tile's loads are queued

#define EDIT_READ(S, s_, buf_)                                                               \
  do {                                                                                            \
    _Pragma("unroll") for (int t = 0; t < TI; ++t)                                                \
      xf[buf_][t] = *reinterpret_cast<const bf16x8*>((S) + xrow + t * 4096 + fo[s_]);             \
    _Pragma("unroll") for (int c = 0; c < CJ; ++c)                                                \
      wf[buf_][c] = *reinterpret_cast<const bf16x8*>((S) + wrow + c * 4096 + fo[s_]);             \
  } while (0)
#define EDIT_MMA(buf_)                                                                            \
  do {                                                                                            \
    _Pragma("unroll") for (int t = 0; t < TI; ++t)                                                \
      _Pragma("unroll") for (int c = 0; c < CJ; ++c)                                              \
        acc[t][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf_][c], xf[buf_][t], acc[t][c], 0, 0, 0); \
  } while (0)

  // Instruction order inside a sub-step, pinned for the scheduler: each
  // matrix-core step is followed by one fragment read for the next sub-step
  // (and, after the barrier, by two of the refill loads), so LDS latency and
  // load issue hide behind the matrix work.
  constexpr int NM = TI * CJ, NR = TI + CJ;
#define EDIT_PIN_SUBSTEP(NV)                                                                      \
  do {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < NM; ++i) {                                              \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                          \
      if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              \
      if (2 * i < (NV)) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);                         \
    }                                                                                             \
    __builtin_amdgcn_sched_barrier(0);                                                            \
  } while (0)
  // Matrix work on the fragments in set cur_ while the fragments of sub-step
  // s_ of stage S are read into set nxt_.
#define EDIT_SUBSTEP(S, s_, nxt_, cur_)                                                           \
  do {                                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    EDIT_READ(S, s_, nxt_);                                                                       \
    EDIT_MMA(cur_);                                                                               \
    EDIT_PIN_SUBSTEP(0);                                                                          \
  } while (0)

  // One K step on stage SC (holding step kk); SN holds step kk + 1. On entry
  // the fragments of sub-step 0 are in set 0. The steady-state form issues
  // its loads unconditionally, so the loop body is one basic block and the
  // compiler keeps track of which stage each outstanding load fills.
#define EDIT_KSTEP_HEAD(SC)                                                                       \
  EDIT_SUBSTEP(SC, 1, 1, 0);                                                                      \
  EDIT_SUBSTEP(SC, 2, 0, 1);                                                                      \
  EDIT_SUBSTEP(SC, 3, 1, 0);
#define EDIT_KSTEP_FULL(SC, SN, kk)                                                               \
  do {                                                                                            \
    EDIT_KSTEP_HEAD(SC)                                                                           \
    /* step kk+1 landed (only step kk+2's loads may be in flight) and every */                   \
    /* wave is done reading SC: refill SC with step kk+3.                    */                   \
    stage_barrier<NPER>();                                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    EDIT_READ(SN, 0, 0);                                                                          \
    EDIT_DMA(SC, (kk) + 3);                                                                       \
    EDIT_MMA(1);                                                                                  \
    EDIT_PIN_SUBSTEP(NPER);                                                                       \
  } while (0)
#define EDIT_KSTEP_TAIL(SC, SN, kk)                                                               \
  do {                                                                                            \
    EDIT_KSTEP_HEAD(SC)                                                                           \
    if ((kk) + 2 < nk) stage_barrier<NPER>(); else stage_barrier<0>();                            \
    if ((kk) + 3 < nk) EDIT_DMA(SC, (kk) + 3);                                                    \
    if ((kk) + 1 < nk) EDIT_READ(SN, 0, 0);                                                       \
    EDIT_MMA(1);                                                                                  \
  } while (0)

#define EDIT_KSTEP_FULL2(SC, SN, kk)                                                              \
  do {                                                                                            \
    EDIT_KSTEP_HEAD(SC)                                                                           \
    stage_barrier<0>();                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    EDIT_READ(SN, 0, 0);                                                                          \
    EDIT_DMA(SC, (kk) + 2);                                                                       \
    EDIT_MMA(1);                                                                                  \
    EDIT_PIN_SUBSTEP(NPER);                                                                       \
  } while (0)
#define EDIT_KSTEP_TAIL2(SC, SN, kk)                                                              \
  do {                                                                                            \
    EDIT_KSTEP_HEAD(SC)                                                                           \
    stage_barrier<0>();                                                                           \
    if ((kk) + 2 < nk) EDIT_DMA(SC, (kk) + 2);                                                    \
    if ((kk) + 1 < nk) EDIT_READ(SN, 0, 0);                                                       \
    EDIT_MMA(1);                                                                                  \
  } while (0)

  int tl = blockIdx.x;
  EDIT_SET_TILE(tl);
  EDIT_PREFETCH3();
  for (;;) {
    // The tile's bias, requested before anything else is queued behind it.
    if (EM != E_F32) {
#pragma unroll
      for (int c = 0; c < CJ; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = wn * WTN + c * 32 + 8 * g + 4 * fh;
          bv[c][g] = n0 + nl < p.N ? *reinterpret_cast<const bf16x4*>(bias + nl) : bf16x4{};
        }
    }
#pragma unroll
    for (int t = 0; t < TI; ++t)
#pragma unroll
      for (int c = 0; c < CJ; ++c) acc_zero(acc[t][c]);

    // Step 0 landed. Loads complete in issue order; the previous tile's
    // stores, issued after this tile's loads, may still be outstanding.
    if (ST == 3) {
      if (nk > 2) stage_barrier<2 * NPER>();
      else stage_barrier<0>();
    } else {
      if (nk > 1) stage_barrier<NPER>();
      else stage_barrier<0>();
    }
    EDIT_READ(S0, 0, 0);
    int kt = 0;
    if (ST == 3) {
      // Whole rounds of three steps while every step refills its stage, then
      // the at most five steps left.
      for (; kt + 5 < nk; kt += 3) {
        EDIT_KSTEP_FULL(S0, S1, kt);
        EDIT_KSTEP_FULL(S1, S2, kt + 1);
        EDIT_KSTEP_FULL(S2, S0, kt + 2);
      }
      EDIT_KSTEP_TAIL(S0, S1, kt);
      if (kt + 1 < nk) EDIT_KSTEP_TAIL(S1, S2, kt + 1);
      if (kt + 2 < nk) EDIT_KSTEP_TAIL(S2, S0, kt + 2);
      if (kt + 3 < nk) EDIT_KSTEP_TAIL(S0, S1, kt + 3);
      if (kt + 4 < nk) EDIT_KSTEP_TAIL(S1, S2, kt + 4);
    } else {
      for (; kt + 3 < nk; kt += 2) {
        EDIT_KSTEP_FULL2(S0, S1, kt);
        EDIT_KSTEP_FULL2(S1, S0, kt + 1);
      }
      EDIT_KSTEP_TAIL2(S0, S1, kt);
      if (kt + 1 < nk) EDIT_KSTEP_TAIL2(S1, S0, kt + 1);
      if (kt + 2 < nk) EDIT_KSTEP_TAIL2(S0, S1, kt + 2);
    }

    // The last step's barrier came after every wave's last LDS read: the
    // stages are free. Queue the next tile's first three steps, then write
    // this tile from registers while they are in flight.
    const int em0 = m0, en0 = n0, esplit = split;
    const int next = tl + nblk;
    if (next < ntiles) {
      EDIT_SET_TILE(next);
      EDIT_PREFETCH3();
    }
    if (EM == E_F32) {
      // Split-K partial sums in fp32: quad g of lane l is 4 consecutive
      // columns 8g + 4(l >> 5) .. +3 of row l & 31, one 16-byte store.
      float* outp = p.Cf + (size_t)esplit * (size_t)p.split_stride;
#pragma unroll
      for (int t = 0; t < TI; ++t) {
        const int m = em0 + wm * WTM + t * 32 + fr;
#pragma unroll
        for (int c = 0; c < CJ; ++c)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = en0 + wn * WTN + c * 32 + 8 * g + 4 * fh;
            if (m < p.M && n < p.N)
              *reinterpret_cast<f32x4*>(outp + (size_t)m * p.ldc + n) =
                  f32x4{acc[t][c][4 * g], acc[t][c][4 * g + 1], acc[t][c][4 * g + 2], acc[t][c][4 * g + 3]};
          }
      }
      if (next >= ntiles) break;
      tl = next;
      continue;
    }
    if (EM == E_BIAS_GN) {
      // GroupNorm partial statistics of the tile as stored (bf16), per column over its BM rows:
      // the exact mean, then the sum of squared deviations from it. Element k of accumulator (t, c)
      // is column c*32 + 8(k/4) + 4(l>>5) + k%4 of row t*32 + (l & 31). Each lane first adds its TI
      // rows for all its CJ*16 columns; the 32 lanes of a half-wave then add level by level (every
      // level a batch of independent steps: four row-local DPP moves, then the swap of 16-lane
      // rows), and the waves' sums meet in LDS. A fixed order throughout.
      // Column blocks per reduction batch: all of them with a CU to itself; one at a time where two
      // blocks share a CU (their register budget is halved), which changes no sum.
      constexpr int CG = dma_blocks_per_cu<NW, ST>() == 2 ? 1 : CJ;
      constexpr int NV = CG * 16;
      auto stored = [&](int t, int c, int k) -> float {
        return (float)(bf16)(acc[t][c][k] + (float)bv[c][k >> 2][k & 3]);
      };
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int c0 = 0; c0 < CJ; c0 += CG) {
          float sm[NV];
#pragma unroll
          for (int cc = 0; cc < CG; ++cc)
#pragma unroll
            for (int k = 0; k < 16; ++k) {
              const int c = c0 + cc;
              const float mu = pass ? gnmean[c * 32 + 8 * (k >> 2) + 4 * fh + (k & 3)] : 0.0f;
              float v = 0.0f;
#pragma unroll
              for (int t = 0; t < TI; ++t) {
                const float d = stored(t, c, k) - mu;
                v += pass ? d * d : d;
              }
              sm[cc * 16 + k] = v;
            }
          // lane i += lane i^1, i^2 (quad perms), then 7-i within 8, then 15-i within 16 (mirrors)
#define EDIT_DPP_LEVEL(CTRL)                                                                          \
          _Pragma("unroll") for (int j = 0; j < NV; ++j)                                               \
            sm[j] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                            \
                0, __builtin_bit_cast(int, sm[j]), (CTRL), 0xF, 0xF, false));
          EDIT_DPP_LEVEL(0xB1)
          EDIT_DPP_LEVEL(0x4E)
          EDIT_DPP_LEVEL(0x141)
          EDIT_DPP_LEVEL(0x140)
#undef EDIT_DPP_LEVEL
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            // the other 16-lane row of this half-wave (rows 0 <-> 1, 2 <-> 3)
            const uint32_t u = __builtin_bit_cast(uint32_t, sm[j]);
            const auto pr = __builtin_amdgcn_permlane16_swap(u, u, false, false);
            sm[j] += __builtin_bit_cast(float, (lane & 16) ? pr[0] : pr[1]);
          }
          if (fr == 0) {
#pragma unroll
            for (int cc = 0; cc < CG; ++cc)
#pragma unroll
              for (int k = 0; k < 16; ++k)
                gnred[wm * BN + (c0 + cc) * 32 + 8 * (k >> 2) + 4 * fh + (k & 3)] = sm[cc * 16 + k];
          }
        }
        stage_barrier<63>();   // LDS only: the next tile's loads stay in flight
        if (tid < BN) {
          float v = 0.0f;
#pragma unroll
          for (int w = 0; w < WM; ++w) v += gnred[w * BN + tid];
          if (pass == 0) {
            gnmean[tid] = v / (float)BM;
          } else if (en0 + tid < p.N) {
            float* o = p.gnp + ((size_t)(em0 / BM) * p.N + en0 + tid) * 2;
            o[0] = gnmean[tid];
            o[1] = v;
          }
        }
        stage_barrier<63>();
      }
    }
    // Epilogue: bias (+ ReLU). Accumulator quad g of lane l holds channels
    // 8g + 4(l >> 5) .. +3 of token l & 31; lanes l and l ^ 32 swap the
    // halves of g = 2j + 1 (lower lane) and g = 2j (upper lane), so that each
    // lane writes 8 consecutive channels of its token with one 16-byte store.
#pragma unroll
    for (int t = 0; t < TI; ++t) {
      const int m = em0 + wm * WTM + t * 32 + fr;
      // The residual's quads for this row block, all requested before any
      // store of the block (a load behind a store to possibly the same
      // memory would wait for it).
      bf16x4 rr[EM == E_RES ? CJ : 1][4];
      if (EM == E_RES) {
#pragma unroll
        for (int c = 0; c < CJ; ++c)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = en0 + wn * WTN + c * 32 + 8 * g + 4 * fh;
            rr[EM == E_RES ? c : 0][g] = m < p.M && n < p.N
                                              ? *reinterpret_cast<const bf16x4*>(p.R + (size_t)m * p.ldr + n)
                                              : bf16x4{};
          }
      }
#pragma unroll
      for (int c = 0; c < CJ; ++c) {
        float f[4][4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[g][i] = acc[t][c][4 * g + i] + (float)bv[c][g][i];
            if (EM == E_BIAS_RELU) f[g][i] = f[g][i] > 0.0f ? f[g][i] : 0.0f;
          }
        if (EM == E_RES) {
          // residual: quad g holds channels 8g + 4(l >> 5) .. +3 of token m
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) f[g][i] += (float)rr[EM == E_RES ? c : 0][g][i];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int ge = 2 * j, go = 2 * j + 1;
          const int gsel = fh ? go : ge;
          const int n = en0 + wn * WTN + c * 32 + 8 * gsel;
          uint32_t w[4];
          {
            uint32_t pk[2][2];   // bf16 pairs of quads ge, go
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              bf16x4 b4;
#pragma unroll
              for (int i = 0; i < 4; ++i) b4[i] = (bf16)f[h ? go : ge][i];
              pk[h][0] = reinterpret_cast<const uint32_t*>(&b4)[0];
              pk[h][1] = reinterpret_cast<const uint32_t*>(&b4)[1];
            }
            const uint32_t s0 = fh ? pk[0][0] : pk[1][0];
            const uint32_t s1 = fh ? pk[0][1] : pk[1][1];
            const uint32_t r0 = from_other_half(s0, fh);
            const uint32_t r1 = from_other_half(s1, fh);
            w[0] = fh ? r0 : pk[0][0];
            w[1] = fh ? r1 : pk[0][1];
            w[2] = fh ? pk[1][0] : r0;
            w[3] = fh ? pk[1][1] : r1;
          }
          if (m < p.M && n < p.N)
            *reinterpret_cast<uint4*>(p.C + (size_t)m * p.ldc + n) = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
    if (next >= ntiles) break;
    tl = next;
  }
#undef EDIT_KSTEP_HEAD
#undef EDIT_KSTEP_FULL
#undef EDIT_KSTEP_TAIL
#undef EDIT_KSTEP_FULL2
#undef EDIT_KSTEP_TAIL2
#undef EDIT_SUBSTEP
#undef EDIT_PIN_SUBSTEP
#undef EDIT_MMA
#undef EDIT_READ
#undef EDIT_PREFETCH3
#undef EDIT_DMA
#undef EDIT_SET_TILE
#endif  // __HIP_DEVICE_COMPILE__
}

namespace {

template <int BM, int BN, int WM, int WN, int AM, int EM, int ST = 3>
hipError_t launch_dma_tiles(const GemmArgs<bf16>& a, hipStream_t s) {
  // Three stages: one block per CU (3 x (BM + BN) x 128 bytes of LDS); with
  // more tiles than CUs each block walks several tiles, and the grid stays a
  // multiple of 8 so that every XCD keeps its own contiguous tile range.
  // Spread: one block per tile instead (the loop then ends after one tile),
  // so that CUs that another stream's kernels leave free take tiles as they
  // come; measured 3-6% slower than persistent blocks on an idle chip.
  // Two stages with 4-wave blocks: always one block per tile, two resident
  // per CU. Two stages with 8-wave blocks: one block per CU, persistent like
  // three stages (the next tile's two steps are queued before the epilogue).
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  int ntiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (EM == E_F32) ntiles *= (a.K + a.kchunk - 1) / a.kchunk;
  const int g8 = cus / 8 * 8;
  const bool paired = dma_blocks_per_cu<WM * WN, ST>() == 2;
  const int blocks = paired || ntiles <= g8 || a.spread ? ntiles : g8;
  GemmArgs<bf16> b = a;
  b.fold_blocks = 0;
  // The fold rides along when the conv leaves at least 16 CUs idle; otherwise it runs after.
  const bool fold_here = AM == A_CONV3 && a.fold.W != nullptr && a.fold.C % 64 == 0 && a.fold.Cr % 32 == 0 &&
                         blocks + 16 <= cus;
  if (fold_here) b.fold_blocks = cus - blocks;
  hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, WM, WN, AM, EM, ST>), dim3(blocks + b.fold_blocks), dim3(64 * WM * WN), 0,
                     s, b, ntiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || AM != A_CONV3 || a.fold.W == nullptr || fold_here) return e;
  const FoldArgs& f = a.fold;
  return launch_restore_fold<bf16>(f.W, f.b, f.W2, f.b2, f.C, f.Cr, f.wcat, f.bcat, s);
}

}  // namespace

// Returns hipErrorNotSupported (nothing launched) when the shape is outside
// what the kernel handles; the caller then uses the register-staged GEMM.
hipError_t launch_gemm_dma(const GemmArgs<bf16>& a, AMode am, EMode em, hipStream_t s) {
  if (em == E_RES && a.ldr % 4 != 0) return hipErrorNotSupported;
  if (a.K % 8 != 0 || a.N % 8 != 0 || a.ldb % 8 != 0 || a.lda % 8 != 0 || a.ldc % 8 != 0)
    return hipErrorNotSupported;
  // Buffer offsets are 32-bit and must stay below the out-of-range marker.
  if ((size_t)a.M * a.lda * 2 >= kOob) return hipErrorNotSupported;
  if ((size_t)(a.N < a.seg_rows ? a.N : a.seg_rows) * a.ldb * 2 >= kOob) return hipErrorNotSupported;
  const bool n96 = a.N % 96 == 0 && a.seg_rows % 96 == 0, n128 = a.N % 128 == 0 && a.seg_rows % 128 == 0,
             n192 = a.N % 192 == 0 && a.seg_rows % 192 == 0;
  // Measured on MI355X (random bf16 data, 16384 tokens):
  //  - the 3x3 conv (162 K steps): 119 us against 227 us for the register-staged kernel;
  //  - plain-A projections with 128 x 192 tiles, two stages, two blocks per CU: 46 us at
  //    16384 x 1152 x 1152 and 91 us at 16384 x 2304 x 1152 against 63 and 105 us register-staged.
  if (am == A_CONV3 && (em == E_BIAS || em == E_BIAS_GN || em == E_RES)) {
    // the halo-staged kernel where it covers the shape
    const hipError_t e = launch_conv3x3_halo(a, em, s);
    if (e != hipErrorNotSupported) return e;
  }
  if (am == A_CONV3 && (em == E_BIAS || em == E_RES || em == E_BIAS_GN)) {
    if (a.Cin % 64 != 0 || a.lda != a.Cin || a.K != 9 * a.Cin) return hipErrorNotSupported;
    if (em == E_RES) return n96 ? launch_dma_tiles<256, 96, 4, 1, A_CONV3, E_RES>(a, s) : hipErrorNotSupported;
    if (em == E_BIAS_GN) {
      // every tile full and within one sample (H*W a multiple of the tile height gn_rows); 128-row tiles
      // run two stages, two blocks per CU
      if (!n96 || a.gnp == nullptr || (a.gn_rows != 256 && a.gn_rows != 128) || a.M % a.gn_rows != 0)
        return hipErrorNotSupported;
      if (a.gn_rows == 128) return launch_dma_tiles<128, 96, 4, 1, A_CONV3, E_BIAS_GN, 2>(a, s);
      return launch_dma_tiles<256, 96, 4, 1, A_CONV3, E_BIAS_GN>(a, s);
    }
    if (n96) return launch_dma_tiles<256, 96, 4, 1, A_CONV3, E_BIAS>(a, s);
    if (n128) return launch_dma_tiles<256, 128, 2, 2, A_CONV3, E_BIAS>(a, s);
    return hipErrorNotSupported;
  }
  if (am == A_CAT2) {
    // The query Linear over [X | act] with the restore folded in (K = C + C/r).
    if (a.K1 % 64 != 0 || a.K1 >= a.K || a.lda2 % 8 != 0 || (size_t)a.M * a.lda2 * 2 >= kOob)
      return hipErrorNotSupported;
    if (n192 && em == E_BIAS_RELU) return launch_dma_tiles<128, 192, 2, 2, A_CAT2, E_BIAS_RELU, 2>(a, s);
    return hipErrorNotSupported;
  }
  if (am == A_PLAIN && em == E_F32) {
    // Split-K weight gradients (K = tokens): every split is a multiple of 64.
    if (a.kchunk <= 0 || a.kchunk % 64 != 0 || a.ldc % 4 != 0) return hipErrorNotSupported;
    if (n192) return launch_dma_tiles<128, 192, 2, 2, A_PLAIN, E_F32, 2>(a, s);
    if (n96) return launch_dma_tiles<128, 96, 4, 1, A_PLAIN, E_F32, 2>(a, s);
    return hipErrorNotSupported;
  }
  if (am == A_PLAIN && !n192 && n96 && em == E_BIAS) return launch_dma_tiles<128, 96, 4, 1, A_PLAIN, E_BIAS, 2>(a, s);
  if (am == A_PLAIN && n192) {
    if (em == E_RES) return launch_dma_tiles<128, 192, 2, 2, A_PLAIN, E_RES, 2>(a, s);
    if (em == E_BIAS) return launch_dma_tiles<128, 192, 2, 2, A_PLAIN, E_BIAS, 2>(a, s);
    if (em == E_BIAS_RELU) return launch_dma_tiles<128, 192, 2, 2, A_PLAIN, E_BIAS_RELU, 2>(a, s);
  }
  return hipErrorNotSupported;
}

}  // namespace edit
