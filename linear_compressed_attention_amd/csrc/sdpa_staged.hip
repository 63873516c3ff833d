// Softmax attention with the key set staged in LDS (bf16 inputs, fp32
// accumulation): the softmax blocks of the MM-EDiT hybrid layer (EDiT paper,
// section "MM-EDiT: hybrid attention"). Image rows attend over the text keys
// only (a few hundred keys against thousands of queries per head); text rows
// attend over [K'_I ; K_T] (about a thousand keys), taken in splits that are
// merged by sdpa_combine_kernel.
//
// Schedule. The work is a list of 32-query tiles in (split, sample, head,
// tile) order; each block takes a contiguous run of it (one block per CU
// slot, so the grid fills the chip once). For every (split, sample, head)
// segment in its run the block stages that split's keys -- K as [key][dim],
// V^T as [dim][key] -- then its eight waves walk the segment's tiles with no
// barrier. A block restages only where its run crosses into the next segment.
//
// Tile. A wave takes a tile of 32 queries and walks the keys in 32-key
// tiles, two score tiles in flight (the next one's products are issued
// before this one's softmax): the scores S^T = K Q^T of a key tile (one
// 32x32x16 matrix-core product per 16 head dims) sit in registers, lane l
// holding query l % 32 and keys 4h+r, 8+4h+r, 16+4h+r and 24+4h+r (h = l /
// 32, r < 4). Online softmax in the exp2 domain: the key tile's maximum (the
// two lane halves exchanged by v_permlane32_swap), then
// p = 2^((s - m) log2(e) / sqrt(d)) rounded to bf16, and O^T += V^T P^T with
// P^T the second operand straight from those registers (V^T is staged in the
// matching key order). The running maximum m is raised lazily: only when a
// key tile's maximum exceeds it by more than 2^8 in the exponent, so p <= 256
// and most key tiles need no rescale of O and of the row sum. The row sum adds
// the bf16-rounded p (v_dot2 with ones): the normaliser sums the same
// weights the PV product used.
//
// The file is built with -fno-honor-nans (no NaN operands reach these max
// reductions: scores are finite, masked keys are -inf), which lets the
// compiler fold the maxima into v_max3 without canonicalising each operand.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace edit {
namespace {

// Keys staged per split for head dims up to 16 DT: a multiple of the 96-key chunk, K and V^T within the
// 160 KiB of LDS (one block per CU).
template <int DT>
struct StagedGeom {
  static constexpr int KMAX = DT <= 5 ? 384 : 288;
  static constexpr int DK = 16 * DT;               // K row: head dims rounded up to the 16-dim k step
  static constexpr int DV = 32 * ((DT + 1) / 2);   // V^T rows: head dims rounded up to 32-row output tiles
  static constexpr int OT = DV / 32;               // output tiles
  static constexpr int KP = DK + 8, VP = KMAX + 8;  // LDS row pitches (elements): 16 bytes of padding
  static constexpr int VT_BYTES = DV * VP * 2;
  static constexpr int K_BYTES = KMAX * KP * 2;
  // the fused linear part (head dims up to 64): S^T hi and lo, DV rows (zero past the operand's DP rows) of
  // LK = the operand's DK columns plus 16 bytes of padding, and z
  static constexpr bool LIN = DT <= 4;
  static constexpr int LDP = 16 * DT, LK = 32 * ((DT + 1) / 2), LP = LK + 8;
  static constexpr int LIN_BYTES = LIN ? 2 * DV * LP * 2 + LK * 4 : 0;
  static constexpr int BYTES = VT_BYTES + K_BYTES + LIN_BYTES;
  static_assert(KMAX % 96 == 0, "whole chunks");
  static_assert(BYTES <= 160 * 1024, "LDS");
};
constexpr int kThreads = 512, kWaves = kThreads / 64;
constexpr int kTileQ = 32;          // queries per wave tile
constexpr float kLazyLog2 = 8.0f;   // headroom of the running maximum (log2 units)
constexpr double kStageTiles = 3.0;  // a segment's staging, in a wave's 32-key tiles (schedule estimate)

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Position of key k in its 32-key group of V^T: bits 2 and 3 swapped. A 16-key k step of the PV product
// takes k indices 8h .. 8h+7 from lane half h, which holds keys 4h+r and 8+4h+r (r < 4) of that step.
__device__ __forceinline__ int staged_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// The value lane l ^ 32 holds.
__device__ __forceinline__ float other_half(float v, bool upper) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, upper ? pr[0] : pr[1]);
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

constexpr uint32_t kOob = 0x80000000u;   // beyond every resource used here: loads return zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0); dword 3 selects 32-bit data
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4v load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Up to two attention problems of one head geometry in one launch (the hybrid's text rows and image rows):
// their work units are concatenated, job 0's first.
struct StagedJobs {
  SdpaArgs<bf16> job[2];
  int nqt[2];     // query tiles per (split, sample, head) segment
  int units0;     // job 0's units
  int units;      // all units
  int per[2];     // units per block of each job
  int blocks0;    // blocks taking job 0 (the rest take job 1)
};

template <int DT>
__global__ __launch_bounds__(kThreads) void sdpa_staged_kernel(const StagedJobs J) {
  using G = StagedGeom<DT>;
  constexpr int KMAX = G::KMAX, DK = G::DK, DV = G::DV, OT = G::OT, KP = G::KP, VP = G::VP;
  __shared__ __attribute__((aligned(16))) unsigned char lds[G::BYTES];
  bf16* const Vt = reinterpret_cast<bf16*>(lds);
  bf16* const Ks = reinterpret_cast<bf16*>(lds + G::VT_BYTES);
  bf16* const Ls = reinterpret_cast<bf16*>(lds + G::VT_BYTES + G::K_BYTES);   // S^T hi, then lo (fused linear)
  float* const Lz = reinterpret_cast<float*>(lds + G::VT_BYTES + G::K_BYTES + (G::LIN ? 2 * DV * G::LP * 2 : 0));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fq = lane & 31, hh = lane >> 5;
  const bool upper = hh != 0;
  const int d = J.job[0].d;
  const float sl2 = 1.4426950408889634f / sqrtf((float)d);   // log2(e) / sqrt(d)
  const bf16x2 ones2 = {(bf16)1.0f, (bf16)1.0f};

  const int blk = xcd_swizzle((int)blockIdx.x, (int)gridDim.x);
  // this block's run of units: job 0's blocks first, then job 1's (a block takes one job's units only)
  const bool j0 = blk < J.blocks0;
  const int u0 = j0 ? blk * J.per[0] : J.units0 + (blk - J.blocks0) * J.per[1];
  const int u1 = j0 ? min(J.units0, u0 + J.per[0]) : min(J.units, u0 + J.per[1]);
  for (int u = u0; u < u1;) {
    const int jb = u < J.units0 ? 0 : 1, ub = jb ? J.units0 : 0, nqt = J.nqt[jb];
    const SdpaArgs<bf16>& p = J.job[jb];
    const int Nq = p.Nq, Ntot = p.N1 + p.N2;
    const int seg = (u - ub) / nqt, tbase = ub + seg * nqt, ue = min(u1, tbase + nqt);
    const int h = seg % p.heads, rest = seg / p.heads, b = rest % p.B, sp = rest / p.B;
    if (u != u0) __syncthreads();   // every wave is done with the previous segment's keys
    const int k0 = sp * KMAX, n = min(KMAX, Ntot - k0);   // this split's keys

    // ---- stage K (zero past n and past d) and V^T (keys in staged_pos order, zero past n and d) ----
    // Keys [0, n1) come from (k1, v1), keys [n1, n) from (k2, v2), each source read through a buffer
    // resource over this segment's rows: offsets past it (keys or head dims outside the source) read zero.
    // Every load of a thread is issued before any LDS write: one memory round trip for the whole stage.
    const int n1 = max(0, min(n, p.N1 - k0)), n2 = n - n1;
    const int ld1 = p.ldkv1, ld2 = p.ldkv2;
    __amdgpu_buffer_rsrc_t rk1 = make_rsrc(p.q, 0), rv1 = rk1, rk2 = rk1, rv2 = rk1;
    if (n1 > 0) {
      const size_t o = ((size_t)b * p.N1 + k0) * ld1 + (size_t)h * d;
      const uint32_t bytes = (uint32_t)(((size_t)(n1 - 1) * ld1 + d) * 2);
      rk1 = make_rsrc(p.k1 + o, bytes);
      rv1 = make_rsrc(p.v1 + o, bytes);
    }
    if (n2 > 0) {
      const size_t o = ((size_t)b * p.N2 + max(0, k0 - p.N1)) * ld2 + (size_t)h * d;
      const uint32_t bytes = (uint32_t)(((size_t)(n2 - 1) * ld2 + d) * 2);
      rk2 = make_rsrc(p.k2 + o, bytes);
      rv2 = make_rsrc(p.v2 + o, bytes);
    }
    // byte offset of (key, c8) in source 1 / source 2, or past every resource
    auto off1 = [&](int key, int c8) { return key < n1 && c8 < d ? (uint32_t)(key * ld1 + c8) * 2u : kOob; };
    auto off2 = [&](int key, int c8) {
      return key >= n1 && key < n && c8 < d ? (uint32_t)((key - n1) * ld2 + c8) * 2u : kOob;
    };
    constexpr int CK = DK / 8, CV = DV / 8;   // 16-byte chunks per K row / per key of V^T
    constexpr int NK = (KMAX * CK + kThreads - 1) / kThreads, NV = (KMAX * CV + kThreads - 1) / kThreads;
    u32x4v kr[NK], vr[NV];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = tid + kThreads * i, key = e / CK, c8 = (e % CK) * 8;
      kr[i] = load16(rk1, off1(key, c8));
    }
    // V items run key-fastest: each 2-byte store instruction below writes one contiguous run of a row
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + kThreads * i, key = e % KMAX, c8 = (e / KMAX) * 8;
      vr[i] = load16(rv1, off1(key, c8));
    }
    if (n2 > 0) {   // a split that reaches into the second source
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int e = tid + kThreads * i, key = e / CK, c8 = (e % CK) * 8;
        kr[i] |= load16(rk2, off2(key, c8));
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = tid + kThreads * i, key = e % KMAX, c8 = (e / KMAX) * 8;
        vr[i] |= load16(rv2, off2(key, c8));
      }
    }
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = tid + kThreads * i;
      if (e < KMAX * CK) *reinterpret_cast<u32x4v*>(Ks + (e / CK) * KP + (e % CK) * 8) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + kThreads * i, key = e % KMAX, c8 = (e / KMAX) * 8;
      if (e < KMAX * CV) {
        const bf16* v = reinterpret_cast<const bf16*>(&vr[i]);
        const int pos = staged_pos(key);
#pragma unroll
        for (int j = 0; j < 8; ++j) Vt[(c8 + j) * VP + pos] = v[j];
      }
    }
    // the head's state operand for the fused linear part: S^T hi and lo (rows past the operand's LDP rows
    // zero) and z
    const bool linfuse = G::LIN && p.lin_st != nullptr;
    if (linfuse) {
      constexpr int LDP = G::LDP, LK = G::LK, LP = G::LP, LC = LK / 8;
      const bf16* gst = p.lin_st + ((size_t)b * p.heads + h) * 2 * LDP * LK;
      for (int e = tid; e < 2 * DV * LC; e += kThreads) {
        const int part = e / (DV * LC), r = (e / LC) % DV, c8 = (e % LC) * 8;
        u32x4v v = u32x4v{0u, 0u, 0u, 0u};
        if (r < LDP) v = *reinterpret_cast<const u32x4v*>(gst + ((size_t)part * LDP + r) * LK + c8);
        *reinterpret_cast<u32x4v*>(Ls + (part * DV + r) * LP + c8) = v;
      }
      for (int k = tid; k < LK; k += kThreads) Lz[k] = p.lin_zp[((size_t)b * p.heads + h) * LK + k];
    }
    __syncthreads();

    // ---- the segment's query tiles ----
    const bf16* qbase = p.q + (size_t)b * Nq * p.ldq + h * d;
    const int ldq = p.ldq;
    const bool split = p.splits > 1;
    float* pbase = split ? p.part + (((size_t)sp * p.B + b) * p.heads + h) * (size_t)Nq * (d + 2) : nullptr;
    bf16* obase = p.out + (size_t)b * Nq * p.ldo + h * d;
    const int ldo = p.ldo;
    const bf16* bbase = p.blend_src ? p.blend_src + (size_t)b * Nq * p.ldbs + h * d : nullptr;
    const int ldbs = p.ldbs;
    const float* lbase = p.lin_den ? p.lin_den + (size_t)b * Nq * p.heads + h : nullptr;
    const int lstride = p.heads;
    // lane's query fragments: dims 16 s + 8 h .. + 7 of query fq (zero past d); rows past Nq read the last
    // query (their results are not stored)
    auto load_q = [&](bf16x8 (&dst)[DT], int qt) {
      const bf16* row = qbase + (size_t)min(qt * kTileQ + fq, Nq - 1) * ldq + 8 * hh;
#pragma unroll
      for (int s = 0; s < DT; ++s) {
        if (16 * s + 8 * hh < d) dst[s] = *reinterpret_cast<const bf16x8*>(row + 16 * s);
        else frag_zero(dst[s]);
      }
    };
    // up to 64 head dims the next tile's query fragments are requested while this tile is computed (wider
    // heads would need more registers than a wave of this block may hold)
    constexpr bool kPrefetch = DT <= 4;
    bf16x8 qn[DT];
    if (kPrefetch && u + wave < ue) load_q(qn, u + wave - tbase);
    for (int t = u + wave; t < ue; t += kWaves) {
      const int qi = t - tbase;   // tile index in the segment
      const int qrow = qi * kTileQ + fq;
      const bool qv = qrow < Nq;
      bf16x8 qf[DT];
      if (kPrefetch) {
#pragma unroll
        for (int s = 0; s < DT; ++s) qf[s] = qn[s];
        if (t + kWaves < ue) load_q(qn, t + kWaves - tbase);
      } else {
        load_q(qf, qi);
      }
      // the blend rows at this lane's output positions (dims 32 o + 8 j + 4 h .. + 3): requested here, used
      // at the end of the tile (up to 64 head dims; wider heads read them at the end)
      bf16x4 bb[OT][4];
      float lin = 0.0f;
      auto load_blend = [&]() {
        const bf16* brow = bbase + (size_t)min(qrow, Nq - 1) * ldbs + 4 * hh;
#pragma unroll
        for (int o = 0; o < OT; ++o)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            bb[o][j] = 32 * o + 8 * j + 4 * hh < d ? *reinterpret_cast<const bf16x4*>(brow + 32 * o + 8 * j)
                                                   : bf16x4{};
        if (lbase) lin = lbase[(size_t)min(qrow, Nq - 1) * lstride];
      };
      if (kPrefetch && bbase) load_blend();

      f32x16 acc[OT];
#pragma unroll
      for (int o = 0; o < OT; ++o) acc_zero(acc[o]);
      float m = 0.0f, l = 0.0f;
      const bf16* kp0 = Ks + fq * KP + 8 * hh;
      const bf16* vp0 = Vt + fq * VP + 8 * hh;
      const int nkt = (n + 31) / 32;   // 32-key tiles
      // Scores of key tile kt: keys 32 kt + 8 (r / 4) + 4 h + r % 4 for query fq.
      auto scores = [&](f32x16& sc, int kt) {
        const bf16* kp = kp0 + 32 * kt * KP;
        acc_zero(sc);
#pragma unroll
        for (int s = 0; s < DT; ++s) mma32(sc, *reinterpret_cast<const bf16x8*>(kp + 16 * s), qf[s]);
        if (32 * kt + 32 > n) {
          // keys past n (zero rows of K and V): one more k step adds -inf to their scores, A = (-inf, 0, ..)
          // for those keys and B = (1, 0, ..) for every query, both in lane half 0
          bf16x8 am, bx;
          frag_zero(am);
          frag_zero(bx);
          if (!upper) {
            if (32 * kt + fq >= n) am[0] = (bf16)(-INFINITY);
            bx[0] = (bf16)1.0f;
          }
          mma32(sc, am, bx);
        }
      };
      // Softmax of key tile kt's scores and O^T += V^T P^T.
      auto softmax_pv = [&](const f32x16& sc, int kt) {
        float cm = max3(sc[0], sc[1], sc[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) cm = max3(cm, sc[r], sc[r + 1]);
        cm = fmaxf(cm, sc[15]);
        cm = fmaxf(cm, other_half(cm, upper));   // lanes l and l ^ 32 hold the query's two key halves
        if (kt == 0) {
          m = cm;
        } else if (__builtin_amdgcn_ballot_w64((cm - m) * sl2 > kLazyLog2) != 0) {
          const float mn = fmaxf(m, cm), corr = __builtin_amdgcn_exp2f((m - mn) * sl2);
          m = mn;
          l *= corr;
#pragma unroll
          for (int o = 0; o < OT; ++o)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[o][r] *= corr;
        }
        const float msl = m * sl2;
        const bf16* vp = vp0 + 32 * kt;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          bf16x8 pf;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            pf[i] = (bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * s2 + i], sl2, -msl));
#pragma unroll
          for (int i = 0; i < 4; ++i)
            l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[2 * i], pf[2 * i + 1]}, ones2, l, false);
#pragma unroll
          for (int o = 0; o < OT; ++o)
            mma32(acc[o], *reinterpret_cast<const bf16x8*>(vp + o * 32 * VP + 16 * s2), pf);
        }
      };
      // Two score tiles in turn: the next tile's score products are issued before this tile's softmax, so
      // the matrix cores work on them while the exponentials are taken.
      f32x16 sa, sb;
      scores(sa, 0);
      int kt = 0;
#pragma unroll 1
      for (; kt + 1 < nkt; kt += 2) {
        scores(sb, kt + 1);
        softmax_pv(sa, kt);
        if (kt + 2 < nkt) scores(sa, kt + 2);
        softmax_pv(sb, kt + 1);
      }
      if (kt < nkt) softmax_pv(sa, kt);   // an odd last tile
      l += other_half(l, upper);
      // the fused linear part (every lane, before any leaves): y_lin^T = S^T q^T on the matrix cores (the lo
      // part first, then hi, as the apply kernel adds them) and the normaliser q . z + eps, the lane's dims
      // of its query then the other lane half's
      f32x16 yl[G::LIN ? OT : 1];
      float linv = 1.0f;
      if constexpr (G::LIN) {
        if (linfuse) {
          float den = 0.0f;
#pragma unroll
          for (int s = 0; s < DT; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) den += (float)qf[s][i] * Lz[16 * s + 8 * hh + i];
          den += other_half(den, upper);
          linv = den + p.lin_eps;
#pragma unroll
          for (int o = 0; o < OT; ++o) {
            acc_zero(yl[o]);
#pragma unroll
            for (int s = 0; s < DT; ++s) {
              const bf16* ar = Ls + (o * 32 + fq) * G::LP + 16 * s + 8 * hh;
              mma32(yl[o], *reinterpret_cast<const bf16x8*>(ar + DV * G::LP), qf[s]);
              mma32(yl[o], *reinterpret_cast<const bf16x8*>(ar), qf[s]);
            }
          }
        }
      }
      if (!qv) continue;
      if (!kPrefetch && bbase) load_blend();
      if (split) {
        // this split's partial: unnormalised output, max (log2 units), sum
        float* prow = pbase + (size_t)qrow * (d + 2);
#pragma unroll
        for (int o = 0; o < OT; ++o)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int dim = 32 * o + 8 * j + 4 * hh;
            if (dim < d)
              *reinterpret_cast<f32x4*>(prow + dim) =
                  f32x4{acc[o][4 * j], acc[o][4 * j + 1], acc[o][4 * j + 2], acc[o][4 * j + 3]};
          }
        if (!upper) {
          prow[d] = m * sl2;
          prow[d + 1] = l;
        }
        continue;
      }
      const float inv = 1.0f / l;
      float alpha = p.alpha, beta = p.beta;
      if (linfuse) {
        // exact eta: the linear block's mass q . z + eps against the softmax mass sum_t exp(s_t) = 2^(m sl2) l
        if (p.exact_eta) {
          alpha = linv / (linv + exp2f(m * sl2) * l);
          beta = 1.0f - alpha;
        }
        if (p.lin_den_out && !upper) p.lin_den_out[((size_t)b * Nq + qrow) * p.heads + h] = linv;
      } else if (bbase && lbase) {
        alpha = lin / (lin + exp2f(m * sl2) * l);
        beta = 1.0f - alpha;
      }
      const float ilin = 1.0f / linv;
      bf16* orow = obase + (size_t)qrow * ldo + 4 * hh;
#pragma unroll
      for (int o = 0; o < OT; ++o)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (32 * o + 8 * j + 4 * hh < d) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[o][4 * j + r] * inv;
            if constexpr (G::LIN) {
              if (linfuse) {
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = alpha * (yl[o][4 * j + r] * ilin) + beta * v[r];
              }
            }
            if (bbase) {
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] = alpha * (float)bb[o][j][r] + beta * v[r];
            }
            store4(orow + 32 * o + 8 * j, v);
          }
        }
    }
    u = ue;
  }
}

// Blocks one CU holds at once for each key geometry, times the CU count, per device.
constexpr int kMaxDev = 64;
std::atomic<int> g_slots[kMaxDev][9];

template <int DT>
hipError_t launch_dt(const SdpaArgs<bf16>* a, int njobs, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  int slots = dev < kMaxDev ? g_slots[dev][DT].load(std::memory_order_relaxed) : 0;
  if (slots <= 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return hipErrorInvalidDevice;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, sdpa_staged_kernel<DT>, kThreads, 0);
    if (e != hipSuccess) return e;
    slots = cus * std::max(1, occ);
    if (dev < kMaxDev) g_slots[dev][DT].store(slots, std::memory_order_relaxed);
  }
  StagedJobs J{};
  long long u[2] = {0, 0};
  double kt[2] = {1.0, 1.0};   // 32-key tiles per unit, averaged over the splits
  for (int j = 0; j < 2; ++j) {
    const SdpaArgs<bf16>& x = a[j < njobs ? j : 0];
    J.job[j] = x;
    J.nqt[j] = std::max(1, (x.Nq + kTileQ - 1) / kTileQ);
    if (j < njobs) {
      u[j] = (long long)((x.Nq + kTileQ - 1) / kTileQ) * x.heads * x.B * x.splits;
      const int keys = x.N1 + x.N2, last = keys - (x.splits - 1) * StagedGeom<DT>::KMAX;
      kt[j] = ((x.splits - 1) * (StagedGeom<DT>::KMAX / 32) + (last + 31) / 32) / (double)x.splits;
    }
  }
  const long long units = u[0] + u[1];
  if (units <= 0) return hipSuccess;
  if (units >= (1LL << 30)) return hipErrorInvalidValue;
  J.units0 = (int)u[0];
  J.units = (int)units;
  // Blocks per job: the split that evens out the longest block, a block's time taken as its busiest wave's
  // key tiles plus a staging (about kStageTiles key tiles) per segment it starts.
  auto cost = [&](int j, long long per) {
    const long long segs = (per - 1) / J.nqt[j] + 2;
    return (double)((per + kWaves - 1) / kWaves) * kt[j] + (double)segs * kStageTiles;
  };
  long long b0 = u[0] > 0 ? slots : 0;
  if (u[0] > 0 && u[1] > 0) {
    double best = 1e300;
    for (long long c = 1; c < slots; ++c) {
      const long long p0 = (u[0] + c - 1) / c, p1 = (u[1] + (slots - c) - 1) / (slots - c);
      const double t = std::max(cost(0, p0), cost(1, p1));
      if (t < best) { best = t; b0 = c; }
    }
  }
  J.per[0] = u[0] > 0 ? (int)((u[0] + b0 - 1) / b0) : 1;
  J.per[1] = u[1] > 0 ? (int)((u[1] + (slots - b0) - 1) / std::max(1LL, slots - b0)) : 1;
  J.blocks0 = u[0] > 0 ? (int)((u[0] + J.per[0] - 1) / J.per[0]) : 0;
  const long long blocks = J.blocks0 + (u[1] > 0 ? (u[1] + J.per[1] - 1) / J.per[1] : 0);
  hipLaunchKernelGGL((sdpa_staged_kernel<DT>), dim3((unsigned)blocks), dim3(kThreads), 0, s, J);
  return hipGetLastError();
}

}  // namespace

int sdpa_staged_keys(int d) { return (d + 15) / 16 <= 5 ? StagedGeom<5>::KMAX : StagedGeom<8>::KMAX; }

bool sdpa_staged_fuses_linear(int d) { return d > 0 && d <= 64 && d % 8 == 0; }

hipError_t launch_sdpa_staged(const SdpaArgs<bf16>* a, int njobs, hipStream_t s) {
  if (a == nullptr || njobs < 1 || njobs > 2) return hipErrorInvalidValue;
  const int d = a[0].d;
  if (d <= 0 || d > 128 || d % 8) return hipErrorInvalidValue;
  const int kmax = sdpa_staged_keys(d);
  for (int j = 0; j < njobs; ++j) {
    const SdpaArgs<bf16>& x = a[j];
    if (x.d != d || x.Nq < 0 || x.N1 < 0 || x.N2 < 0 || x.B <= 0 || x.heads <= 0) return hipErrorInvalidValue;
    if (x.Nq > 0 && x.N1 + x.N2 <= 0) return hipErrorInvalidValue;
    const int need = std::max(1, (x.N1 + x.N2 + kmax - 1) / kmax);
    if (x.splits != need || (need > 1 && x.part == nullptr)) return hipErrorInvalidValue;
    // buffer offsets of a split's rows are 32-bit
    if (((long long)kmax * std::max(x.ldkv1, x.ldkv2) + d) * 2 >= (1LL << 31)) return hipErrorInvalidValue;
    // the fused linear part: head dims up to 64, one pass over the keys (the split merge blends from
    // blend_src), and not beside blend_src
    if (x.lin_st != nullptr &&
        (!sdpa_staged_fuses_linear(d) || x.splits != 1 || x.lin_zp == nullptr || x.blend_src != nullptr))
      return hipErrorInvalidValue;
  }
  switch ((d + 15) / 16) {
    case 1: return launch_dt<1>(a, njobs, s);
    case 2: return launch_dt<2>(a, njobs, s);
    case 3: return launch_dt<3>(a, njobs, s);
    case 4: return launch_dt<4>(a, njobs, s);
    case 5: return launch_dt<5>(a, njobs, s);
    case 6: return launch_dt<6>(a, njobs, s);
    case 7: return launch_dt<7>(a, njobs, s);
    case 8: return launch_dt<8>(a, njobs, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace edit
