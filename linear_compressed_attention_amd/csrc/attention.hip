// Attention cores on the matrix cores of gfx950.
//
// Page "EDiT: Efficient Diffusion Transformers with Linear Compressed
// Attention" (ICCV 2025 notes):
//   section "Linear-attention formula": y_i = Q_i (sum_j K_j^T V_j) / (Q_i sum_j K_j),
//     computed as a per-head state S = K'^T V' (d x d), z = sum_j K'_j
//     (kv_state_*), then y_i = Q_i S / (Q_i . z + eps) (linattn_apply_*);
//   section "MM-EDiT": the blocks of the hybrid matrix that involve text keep
//     scaled dot-product attention (sdpa_kernel), and the image rows blend the
//     linear and the softmax results with eta = N_I / (N_I + N_T).
//
// All three use the 16x16x32 matrix-core step of common.hpp. Head dimension d
// (a multiple of 8, at most 128) is padded to whole 16-row tiles and 32-deep
// K steps with zeros; DT = ceil(d / 16) is a template parameter.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace edit {

constexpr int kKvChunk = 256;   // compressed tokens per state partial

int kv_state_chunks(int Nc) { return (Nc + kKvChunk - 1) / kKvChunk; }

// The fused depthwise + state kernel takes its chunks as tiles of the compressed grid, TH x TW = kKvChunk
// tokens (both powers of two, TW even so that a token pair shares a row): 16 x 16 where the grid allows, so a
// chunk reads (2 TH + 1) x (2 TW + 1) input pixels for 4 TH TW (the halo 6% instead of up to 50% for chunks
// of whole compressed rows); shorter or narrower grids take wider or taller tiles.
DwStateTile dw_state_tile(int Hc, int Wc) {
  auto p2 = [](int v) { int p = 1; while (p < v) p <<= 1; return p; };
  DwStateTile t;
  t.th = std::min(16, p2(std::max(1, Hc)));
  t.tw = kKvChunk / t.th;
  if (t.tw > p2(std::max(2, Wc))) {
    t.tw = p2(std::max(2, Wc));
    t.th = kKvChunk / t.tw;
  }
  t.ncy = (Hc + t.th - 1) / t.th;
  t.ncx = (Wc + t.tw - 1) / t.tw;
  return t;
}
int dw_state_chunks(int Hc, int Wc) {
  const DwStateTile t = dw_state_tile(Hc, Wc);
  return t.ncy * t.ncx;
}
int kv_state_dp(int d) { return 16 * ((d + 15) / 16); }
int kv_state_dk(int d) { return 32 * ((d + 31) / 32); }

// ---------------------------------------------------------------------------
// KV state, partial sums over one chunk of compressed tokens.
// D[n][k] = sum_j A[n][j] * K'_j[k] with A = [V'^T ; w_hi ; w_lo]: rows n < d
// give S^T (S[k][n] = sum_j K'_j[k] V'_j[n]), rows d and d + 1 give
// z[k] = sum_j w_j K'_j[k] with w = 1 (the layer), or per-token weights
// w[b][j][h] (the backward's dz = sum_j c_j q_j, the same kernel forming
// dS = sum_j q_j^T g_j), split into w_hi = T(w) and w_lo = T(w - w_hi) so
// that a bf16 operand carries ~16 mantissa bits of w. Tokens are the
// matrix-core K dimension, so the chunk's K' and V' slices are staged in LDS
// transposed (channel-major). All loads of a slab are issued before the LDS
// writes (one wait); neighbouring lanes load neighbouring 16-byte channel
// chunks of the same tokens (each token's head slice is one contiguous read),
// and each thread writes four tokens of a channel as one LDS word.
// partial[b][h][chunk][16*DR][16*DT] (fp32).
// ---------------------------------------------------------------------------
// Tokens staged per pass: a whole 256-token chunk in bf16 (84 KB of LDS at
// d = 72, one block per CU), half of it where a launch has several rounds
// of blocks (three blocks per CU then overlap one another's loads).
template <typename T, bool HALF> struct KvSlab { static constexpr int n = HALF ? 128 : 256; };
template <bool HALF> struct KvSlab<float, HALF> { static constexpr int n = 64; };

// Column (token) position of element (row, col) of a staged channel-major
// tile: 8-element chunks are XOR-swizzled by row / 8, so that the transposed
// stores, which hit rows 8 apart, fall in different LDS banks (a 528-byte
// row pitch is a multiple of 128 bytes: unswizzled, every lane of such a
// store hit the same bank). Rows need a multiple of 64 columns.
__device__ __forceinline__ int kv_col(int row, int col) { return (((col >> 3) ^ ((row >> 3) & 7)) << 3) | (col & 7); }

// Four tokens' values of one channel, written to LDS as one 8-byte (bf16) or
// 16-byte (f32) word.
__device__ __forceinline__ void store_quad(bf16* dst, bf16 a, bf16 b, bf16 c, bf16 d) {
  bf16x4 v;
  v[0] = a; v[1] = b; v[2] = c; v[3] = d;
  *reinterpret_cast<bf16x4*>(dst) = v;
}
__device__ __forceinline__ void store_quad(float* dst, float a, float b, float c, float d) {
  f32x4 v;
  v[0] = a; v[1] = b; v[2] = c; v[3] = d;
  *reinterpret_cast<f32x4*>(dst) = v;
}

template <typename T, int DC, bool HALF>
__global__ __launch_bounds__(256) void kv_state_partial_kernel(const T* __restrict__ kc, const T* __restrict__ vc,
                                                               int ld, int Nc, int heads, int nchunks,
                                                               const float* __restrict__ wrow,
                                                               float* __restrict__ partial) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  constexpr int d = 8 * DC;
  constexpr int DT = (d + 15) / 16, DR = (d + 16) / 16;
  constexpr int SLAB = KvSlab<T, HALF>::n;   // tokens staged per pass
  constexpr int PITCH = SLAB + 8;          // elements; rows stay 16-byte aligned
  constexpr int NT = DR * DT;
  constexpr int TPW = (NT + 3) / 4;
  constexpr int QUADS = SLAB / 4;          // token quads per slab
  constexpr int ITEMS = 2 * QUADS * DC;    // (K or V, 8-channel chunk, token quad)
  constexpr int NLOAD = (ITEMS + 255) / 256;
  constexpr int EPC = Chunk<T>::n;         // elements per 16 bytes
  static_assert(SLAB % 64 == 0, "kv_col swizzles within groups of 8 chunks of 8 columns");
  __shared__ __attribute__((aligned(16))) T Kt[16 * DT * PITCH];
  __shared__ __attribute__((aligned(16))) T At[16 * DR * PITCH];
  // (sample, chunk, head) order, head fastest, contiguous per XCD: the heads
  // of one chunk share its token rows' cache lines in one L2.
  const int lb = xcd_swizzle((int)blockIdx.x, (int)gridDim.x);
  const int h = lb % heads, chunk = (lb / heads) % nchunks, b = lb / heads / nchunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = chunk * kKvChunk, j1 = min(Nc, j0 + kKvChunk);

  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc_zero(acc[t]);

  // Rows that never receive data stay zero: K' channels d..16*DT-1 and the
  // rows of A past the two weight rows. Only those rows are cleared (16-byte
  // stores), after the first slab's loads are on their way.
  auto clear_pad_rows = [&]() {
    const u32x4v zero = {0u, 0u, 0u, 0u};
    constexpr int W16 = PITCH * (int)sizeof(T) / 16;   // 16-byte words per row
    for (int i = tid; i < (16 * DT - d) * W16; i += 256)
      reinterpret_cast<u32x4v*>(Kt + d * PITCH)[i] = zero;
    for (int i = tid; i < (16 * DR - d - 2) * W16; i += 256)
      reinterpret_cast<u32x4v*>(At + (d + 2) * PITCH)[i] = zero;
  };

  typedef typename Frag<T>::type FragT;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int js = j0; js < j1; js += SLAB) {
    // Item e: 8-channel chunk (fastest), then token quad, then K or V.
    u32x4v raw[NLOAD][4][8 / EPC];
#pragma unroll
    for (int l = 0; l < NLOAD; ++l) {
      const int e = tid + 256 * l;
      const int c8 = (e % DC) * 8, rest = e / DC;
      const int tq = rest % QUADS, which = rest / QUADS;
      const T* src = (which ? vc : kc) + ((size_t)b * Nc + js + 4 * tq) * ld + h * d + c8;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = e < ITEMS && js + 4 * tq + u < j1;
#pragma unroll
        for (int w = 0; w < 8 / EPC; ++w) {
          const u32x4v zero = {0u, 0u, 0u, 0u};
          raw[l][u][w] = ok ? *reinterpret_cast<const u32x4v*>(src + (size_t)u * ld + w * EPC) : zero;
        }
      }
    }
    if (js == j0) clear_pad_rows();
#pragma unroll
    for (int l = 0; l < NLOAD; ++l) {
      const int e = tid + 256 * l;
      if (e < ITEMS) {
        const int c8 = (e % DC) * 8, rest = e / DC;
        const int tq = rest % QUADS, which = rest / QUADS;
        T* dst = which ? At : Kt;
        const T* v0 = reinterpret_cast<const T*>(&raw[l][0][0]);
        const T* v1 = reinterpret_cast<const T*>(&raw[l][1][0]);
        const T* v2 = reinterpret_cast<const T*>(&raw[l][2][0]);
        const T* v3 = reinterpret_cast<const T*>(&raw[l][3][0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = c8 + i;
          store_quad(dst + row * PITCH + kv_col(row, 4 * tq), v0[i], v1[i], v2[i], v3[i]);
        }
      }
    }
    for (int t = tid; t < SLAB; t += 256) {
      const float wv = js + t < j1 ? (wrow ? wrow[((size_t)b * Nc + js + t) * heads + h] : 1.0f) : 0.0f;
      const T hi = from_f32<T>(wv);
      At[d * PITCH + kv_col(d, t)] = hi;
      At[(d + 1) * PITCH + kv_col(d + 1, t)] = from_f32<T>(wv - to_f32(hi));
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < SLAB / 32; ++ks) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int tile = wave + 4 * t;
        if (tile < NT) {
          const int tr = tile / DT, tc = tile % DT;
          FragT a, bb;
          const int ra = tr * 16 + fr, rk = tc * 16 + fr;
          frag_load(a, At + ra * PITCH + kv_col(ra, ks * 32 + fk));
          frag_load(bb, Kt + rk * PITCH + kv_col(rk, ks * 32 + fk));
          mma16(acc[t], a, bb);
        }
      }
    }
    __syncthreads();
  }

  float* out = partial + (((size_t)b * heads + h) * nchunks + chunk) * (16 * DR) * (16 * DT);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = wave + 4 * t;
    if (tile < NT) {
      const int tr = tile / DT, tc = tile % DT;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out[(tr * 16 + (lane >> 4) * 4 + r) * (16 * DT) + tc * 16 + (lane & 15)] = acc[t][r];
    }
  }
}

// ---------------------------------------------------------------------------
// The Spatial Compressor's depthwise 3x3 stride-2 convs and the state
// partials in one kernel (sections "Spatial Compressor" and
// "Linear-attention formula"): a block makes the compressed keys and values
// of one head over one chunk of 256 compressed tokens, K' = ReLU(DW(k0) +
// b_k) and V' = DW(v0) + b_v, writes them (kc, vc: the backward and the
// hybrid read them), and, with the values still on chip, their chunk
// partial of S^T = V'^T K' and z = sum K' on the matrix cores, in the layout
// kv_state_partial_kernel writes (so kv_state_finalize_kernel merges them
// unchanged). A chunk is a th x tw tile of the compressed grid
// (dw_state_tile: 16 x 16 where the grid allows), so that the input rows and
// columns it shares with its neighbours (the taps' one-pixel border) are a
// small part of what it reads. The compressed tensors are not read back.
// Item e of a block: channel chunk c8 (fastest, so a token's head slice is
// one contiguous run across lanes), token pair (two neighbours in a tile
// row), K or V; an item convolves its two tokens (each from its nine taps,
// loads at clamped in-image positions, taps outside the image adding zero;
// a token outside the grid is computed at a clamped position and zeroed)
// and writes them to LDS as one two-token word per channel, channel-major
// with the kv_col swizzle, the token's place in the tile as its column.
// ---------------------------------------------------------------------------
constexpr int kDwStateThreads = 512;   // 8 waves: two per SIMD overlap one another's loads
constexpr uint32_t kDwOob = 0x80000000u;   // past a block's buffer resource: the load returns zeros

typedef __bf16 dw_bf16x2 __attribute__((ext_vector_type(2)));

// c + a.lo * b.lo + a.hi * b.hi for two bf16 pairs held in 32-bit words.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dw_bf16x2, a), __builtin_bit_cast(dw_bf16x2, b), c, false);
}

// Two tokens' values of one channel, written to LDS as one 4-byte word.
__device__ __forceinline__ void store_pair(bf16* dst, bf16 a, bf16 b) {
  bf16 v[2] = {a, b};
  *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(v);
}

template <typename T, int DC>
__global__ __launch_bounds__(kDwStateThreads) void dwconv_kv_state_kernel(
    const T* __restrict__ kv0, int H, int W, int heads, int nchunks, const T* __restrict__ dwk,
    const T* __restrict__ dbk, const T* __restrict__ dwv, const T* __restrict__ dbv, T* __restrict__ kc,
    T* __restrict__ vc, float* __restrict__ partial, int twl, int ncx) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  constexpr int NTH = kDwStateThreads;
  constexpr int d = 8 * DC;
  constexpr int DT = (d + 15) / 16, DR = (d + 16) / 16;
  constexpr int SLAB = kKvChunk;
  constexpr int PITCH = SLAB + 8;
  constexpr int NT = DR * DT;
  constexpr int NW = NTH / 64;
  constexpr int TPW = (NT + NW - 1) / NW;
  constexpr int PAIRS = SLAB / 2;
  constexpr int ITEMS = 2 * PAIRS * DC;
  static_assert(SLAB % 64 == 0, "kv_col swizzles within groups of 8 chunks of 8 columns");
  __shared__ __attribute__((aligned(16))) T Kt[16 * DT * PITCH];
  __shared__ __attribute__((aligned(16))) T At[16 * DR * PITCH];
  const int Hc = (H + 1) / 2, Wc = (W + 1) / 2, Nc = Hc * Wc, C = heads * d;
  const int lb = xcd_swizzle((int)blockIdx.x, (int)gridDim.x);
  const int h = lb % heads, chunk = (lb / heads) % nchunks, b = lb / heads / nchunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the chunk's tile: compressed rows y0 .., columns x0 .. x0 + tw - 1 (tw = 2^twl); token t of the tile at
  // (y0 + t / tw, x0 + t % tw)
  const int tw = 1 << twl, cy = chunk / ncx;
  const int y0 = cy * (SLAB >> twl), x0 = (chunk - cy * ncx) * tw;   // SLAB >> twl: the tile's rows
  auto in_grid = [&](int t) { return y0 + (t >> twl) < Hc && x0 + (t & (tw - 1)) < Wc; };
  // the input rows the tile's taps reach, [r0, r1), as a buffer resource over the sample's [k0 | v0] rows
  // (the launch checks that 2 th + 1 rows stay below kDwOob bytes)
  const int th = SLAB >> twl;
  const int r0 = max(2 * y0 - 1, 0), r1 = min(2 * (min(y0 + th, Hc) - 1) + 2, H);
  const T* img = kv0 + ((size_t)b * H + r0) * W * 2 * C;
  const uint32_t pixb = 4u * (uint32_t)C;   // bytes per pixel of kv0 (2C bf16)
  const __amdgpu_buffer_rsrc_t rsI = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(img), (short)0, (int)((uint32_t)(r1 - r0) * (uint32_t)W * pixb), 0x00020000);
  // byte step of tap (ky, kx) from the top-left tap, uniform (held as scalars, added as they are)
  uint32_t tapo[9];
#pragma unroll
  for (int t = 0; t < 9; ++t) tapo[t] = __builtin_amdgcn_readfirstlane((uint32_t)((t / 3) * W + t % 3) * pixb);

  // rows that receive no token data: K' channels d .. 16 DT - 1, and the rows
  // of A past V'^T and the two weight rows (ones, zeros: z = sum K')
  {
    const u32x4v zero = {0u, 0u, 0u, 0u};
    constexpr int W16 = PITCH * (int)sizeof(T) / 16;
    for (int i = tid; i < (16 * DT - d) * W16; i += NTH) reinterpret_cast<u32x4v*>(Kt + d * PITCH)[i] = zero;
    for (int i = tid; i < (16 * DR - d - 2) * W16; i += NTH) reinterpret_cast<u32x4v*>(At + (d + 2) * PITCH)[i] = zero;
    for (int t = tid; t < SLAB; t += NTH) {
      At[d * PITCH + kv_col(d, t)] = from_f32<T>(in_grid(t) ? 1.0f : 0.0f);
      At[(d + 1) * PITCH + kv_col(d + 1, t)] = from_f32<T>(0.0f);
    }
  }

  for (int e = tid; e < ITEMS; e += NTH) {
    const int c8 = (e % DC) * 8, rest = e / DC;
    const int tp = rest % PAIRS, which = rest / PAIRS;   // which: 0 keys, 1 values
    const int cin = which * C + h * d + c8;              // channel in kv0's [k0 | v0] row
    const T* wt = (which ? dwv : dwk) + h * d + c8;
    // Every load of the item (nine taps of two tokens, the taps' weights and the bias) is issued before any is
    // used. A tap outside the image reads at an offset past the sample's resource, which returns zeros.
    u32x4v raw[2][9], wr[9];
    int yo[2], xo[2];
    const int ty = y0 + ((2 * tp) >> twl), tx = x0 + ((2 * tp) & (tw - 1));
    bool ok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      ok[u] = ty < Hc && tx + u < Wc;                    // tokens outside the grid: clamped, then zeroed
      yo[u] = min(ty, Hc - 1);
      xo[u] = min(tx + u, Wc - 1);
      // tap (ky, kx) reads pixel (2 yo + ky - 1, 2 xo + kx - 1): the top-left tap's byte offset (wrapping
      // below zero for a border token, whose border taps are masked) plus the tap's fixed step; only the
      // border rows and columns can fall outside the image
      const uint32_t base = (uint32_t)((2 * yo[u] - 1 - r0) * W + 2 * xo[u] - 1) * pixb + 2u * (uint32_t)cin;
      const bool top = yo[u] > 0, bot = 2 * yo[u] + 1 < H, lef = xo[u] > 0, rig = 2 * xo[u] + 1 < W;
#pragma unroll
      for (int t = 0; t < 9; ++t) {
        const int ky = t / 3, kx = t % 3;
        bool in = true;
        if (ky == 0) in = in & top;
        if (ky == 2) in = in & bot;
        if (kx == 0) in = in & lef;
        if (kx == 2) in = in & rig;
        const uint32_t off = in ? base + tapo[t] : kDwOob;
        raw[u][t] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(rsI, (int)off, 0, 0));
      }
    }
#pragma unroll
    for (int t = 0; t < 9; ++t) wr[t] = *reinterpret_cast<const u32x4v*>(wt + t * C);
    float o[2][8];
    load8((which ? dbv : dbk) + h * d + c8, o[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[1][i] = o[0][i];
    // Taps in pairs (0,1) (2,3) (4,5) (6,7) on v_dot2: word k of a tap holds channels 2k and 2k+1; the pair's
    // lo halves (channel 2k of both taps) and hi halves (channel 2k+1) are regrouped into one word each, the
    // weights once per item. Tap 8 alone, by fma.
    uint32_t wp[4][4][2];
#pragma unroll
    for (int pr = 0; pr < 4; ++pr)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t a = wr[2 * pr][k], bw = wr[2 * pr + 1][k];
        wp[pr][k][0] = (a & 0xFFFFu) | (bw << 16);
        wp[pr][k][1] = (a >> 16) | (bw & 0xFFFF0000u);
      }
    float w8[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w8[2 * k] = __builtin_bit_cast(float, wr[8][k] << 16);
      w8[2 * k + 1] = __builtin_bit_cast(float, wr[8][k] & 0xFFFF0000u);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int pr = 0; pr < 4; ++pr)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t a = raw[u][2 * pr][k], bx = raw[u][2 * pr + 1][k];
          o[u][2 * k] = dot2_bf16((a & 0xFFFFu) | (bx << 16), wp[pr][k][0], o[u][2 * k]);
          o[u][2 * k + 1] = dot2_bf16((a >> 16) | (bx & 0xFFFF0000u), wp[pr][k][1], o[u][2 * k + 1]);
        }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[u][2 * k] = __builtin_fmaf(w8[2 * k], __builtin_bit_cast(float, raw[u][8][k] << 16), o[u][2 * k]);
        o[u][2 * k + 1] =
            __builtin_fmaf(w8[2 * k + 1], __builtin_bit_cast(float, raw[u][8][k] & 0xFFFF0000u), o[u][2 * k + 1]);
      }
      if (!which) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[u][i] = o[u][i] > 0.0f ? o[u][i] : 0.0f;
      }
      if (ok[u]) {
        store8((which ? vc : kc) + ((size_t)b * Nc + (size_t)yo[u] * Wc + xo[u]) * C + h * d + c8, o[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[u][i] = 0.0f;
      }
    }
    // the state uses the values as stored
    T* dst = which ? At : Kt;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = c8 + i;
      store_pair(dst + row * PITCH + kv_col(row, 2 * tp), from_f32<T>(o[0][i]), from_f32<T>(o[1][i]));
    }
  }
  __syncthreads();

  typedef typename Frag<T>::type FragT;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc_zero(acc[t]);
#pragma unroll
  for (int ks = 0; ks < SLAB / 32; ++ks) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int tile = wave + NW * t;
      if (tile < NT) {
        const int tr = tile / DT, tc = tile % DT;
        FragT a, bb;
        const int ra = tr * 16 + fr, rk = tc * 16 + fr;
        frag_load(a, At + ra * PITCH + kv_col(ra, ks * 32 + fk));
        frag_load(bb, Kt + rk * PITCH + kv_col(rk, ks * 32 + fk));
        mma16(acc[t], a, bb);
      }
    }
  }
  float* out = partial + (((size_t)b * heads + h) * nchunks + chunk) * (16 * DR) * (16 * DT);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = wave + NW * t;
    if (tile < NT) {
      const int tr = tile / DT, tc = tile % DT;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out[(tr * 16 + (lane >> 4) * 4 + r) * (16 * DT) + tc * 16 + (lane & 15)] = acc[t][r];
    }
  }
}

// Sum the chunk partials in chunk order and emit S (f32, [d][d] as S[k][n]),
// z (f32), the apply kernel's operand st[2][DP][DK] (rows n, K = k: S^T,
// padded with zeros; bf16 keeps a hi and a lo part so hi + lo carries ~16
// mantissa bits of the fp32 sum) and zp[DK]. One thread per output element.
template <typename T>
__global__ __launch_bounds__(256) void kv_state_finalize_kernel(const float* __restrict__ partial, int heads,
                                                                int d, int DR, int DT, int nchunks,
                                                                float* __restrict__ S, float* __restrict__ z,
                                                                T* __restrict__ st, float* __restrict__ zp) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int DP = 16 * DT, DK = 32 * ((DT + 1) / 2);
  const int RW = 16 * DR, CW = 16 * DT;
  const size_t bh = (size_t)b * heads + h;
  const float* part = partial + bh * nchunks * RW * CW;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < DP * DK) {
    const int n = e / DK, k = e % DK;
    float v = 0.0f;
    if (n < d && k < d) {
      const float* p = part + n * CW + k;
#pragma unroll 8
      for (int c = 0; c < nchunks; ++c) v += p[(size_t)c * RW * CW];
      S[(bh * d + k) * d + n] = v;
    }
    T* sthi = st + bh * 2 * DP * DK;
    const T hi = from_f32<T>(v);
    sthi[e] = hi;
    sthi[DP * DK + e] = from_f32<T>(v - to_f32(hi));
  } else if (e < DP * DK + DK) {
    const int k = e - DP * DK;
    float v = 0.0f;
    if (k < d) {
      const float* p = part + d * CW + k;   // rows d (w_hi) and d + 1 (w_lo)
#pragma unroll 8
      for (int c = 0; c < nchunks; ++c) v += p[(size_t)c * RW * CW] + p[(size_t)c * RW * CW + CW];
      z[bh * d + k] = v;
    }
    zp[bh * DK + k] = v;
  }
}

template <typename T>
hipError_t launch_kv_state_finalize(const float* partial, int B, int heads, int d, int nchunks, float* S, float* z,
                                    T* st, float* zp, hipStream_t s) {
  const int DT = (d + 15) / 16, DR = (d + 16) / 16;
  const int DP = 16 * DT, DK = 32 * ((DT + 1) / 2);
  dim3 fgrid((DP * DK + DK + 255) / 256, heads, B);
  hipLaunchKernelGGL((kv_state_finalize_kernel<T>), fgrid, dim3(256), 0, s, partial, heads, d, DR, DT, nchunks, S,
                     z, st, zp);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_kv_state(const T* kc, const T* vc, int ld, int B, int Nc, int heads, int d, float* partial,
                           int nchunks, float* S, float* z, T* st, float* zp, hipStream_t s, const float* wrow) {
  const int DT = (d + 15) / 16, DR = (d + 16) / 16;
  if ((long long)nchunks * heads * B >= (1LL << 31)) return hipErrorInvalidValue;
  dim3 grid(nchunks * heads * B);
  // more blocks than one round on an MI355X (256 CUs): half slabs
  const bool half = (long long)nchunks * heads * B > 256;
  switch (d / 8) {
#define EDIT_KV_CASE(DCV)                                                                              \
  case DCV:                                                                                            \
    if (half)                                                                                          \
      hipLaunchKernelGGL((kv_state_partial_kernel<T, DCV, true>), grid, dim3(256), 0, s, kc, vc, ld, Nc, \
                         heads, nchunks, wrow, partial);                                               \
    else                                                                                               \
      hipLaunchKernelGGL((kv_state_partial_kernel<T, DCV, false>), grid, dim3(256), 0, s, kc, vc, ld, Nc, \
                         heads, nchunks, wrow, partial);                                               \
    break;
    EDIT_KV_CASE(1) EDIT_KV_CASE(2) EDIT_KV_CASE(3) EDIT_KV_CASE(4) EDIT_KV_CASE(5) EDIT_KV_CASE(6)
    EDIT_KV_CASE(7) EDIT_KV_CASE(8) EDIT_KV_CASE(9) EDIT_KV_CASE(10) EDIT_KV_CASE(11) EDIT_KV_CASE(12)
    EDIT_KV_CASE(13) EDIT_KV_CASE(14) EDIT_KV_CASE(15) EDIT_KV_CASE(16)
#undef EDIT_KV_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_kv_state_finalize<T>(partial, B, heads, d, nchunks, S, z, st, zp, s);
}

template <typename T>
hipError_t launch_dwconv_kv_state(const T* kv0, int B, int H, int W, int C, int heads, int d, const T* dwk,
                                  const T* dbk, const T* dwv, const T* dbv, T* kc, T* vc, float* partial,
                                  int nchunks, hipStream_t s) {
  if constexpr (sizeof(T) != 2) {
    return hipErrorNotSupported;   // fp32 keeps the two-kernel form (slabs of 64 tokens)
  } else {
    if (C != heads * d) return hipErrorInvalidValue;
    const DwStateTile tile = dw_state_tile((H + 1) / 2, (W + 1) / 2);
    if (nchunks != tile.ncy * tile.ncx) return hipErrorInvalidValue;
    // a block's input rows (at most 2 th + 1) are addressed by 32-bit offsets below the out-of-range marker
    if ((size_t)(2 * tile.th + 1) * W * 4 * C >= kDwOob) return hipErrorNotSupported;
    if ((long long)nchunks * heads * B >= (1LL << 31)) return hipErrorInvalidValue;
    int twl = 0;
    while ((1 << twl) < tile.tw) ++twl;
    dim3 grid(nchunks * heads * B);
    switch (d / 8) {
#define EDIT_DKV_CASE(DCV)                                                                                   \
  case DCV:                                                                                                  \
    hipLaunchKernelGGL((dwconv_kv_state_kernel<T, DCV>), grid, dim3(kDwStateThreads), 0, s, kv0, H, W, heads, \
                       nchunks, dwk, dbk, dwv, dbv, kc, vc, partial, twl, tile.ncx);                         \
    break;
      EDIT_DKV_CASE(1) EDIT_DKV_CASE(2) EDIT_DKV_CASE(3) EDIT_DKV_CASE(4) EDIT_DKV_CASE(5) EDIT_DKV_CASE(6)
      EDIT_DKV_CASE(7) EDIT_DKV_CASE(8) EDIT_DKV_CASE(9) EDIT_DKV_CASE(10) EDIT_DKV_CASE(11) EDIT_DKV_CASE(12)
      EDIT_DKV_CASE(13) EDIT_DKV_CASE(14) EDIT_DKV_CASE(15) EDIT_DKV_CASE(16)
#undef EDIT_DKV_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
}

// ---------------------------------------------------------------------------
// Apply: y_i = (Q_i S) / (Q_i . z + eps) per head. A block owns one head and
// kApplyTokens tokens; it stages the head's operand st (S^T, hi and lo parts)
// and z in LDS once, and each wave keeps the fragments in registers while it
// walks 16-token tiles: Y^T = S^T Q^T with B = 16 queries read straight from
// memory as 16-byte fragments (the next tile's are requested before the
// current tile's matrix work). Lane l ends with 4 consecutive output channels
// of token l % 16 per 16-channel tile; at bf16 lanes l and l ^ 16 swap halves
// of two tiles so that each stores 8 consecutive channels (16 bytes). The
// denominator is a VALU dot of the lane's query slice with z, summed over the
// four lanes that share a token.
// ---------------------------------------------------------------------------
constexpr int kApplyTokens = 512;   // tokens per block (32 tiles, 8 per wave)

template <typename T, int DT>
__global__ __launch_bounds__(256) void linattn_apply_kernel(const T* __restrict__ q, int ldq,
                                                            const T* __restrict__ st, const float* __restrict__ zp,
                                                            int N, int heads, int d, float eps,
                                                            T* __restrict__ y, int ldy,
                                                            float* __restrict__ den_out) {
  constexpr int KS = (DT + 1) / 2;
  constexpr int DP = 16 * DT, DK = 32 * KS;
  constexpr int PITCH = DK + 8;                      // 16 rows of one fragment read hit distinct banks
  constexpr bool SPLIT = std::is_same<T, bf16>::value;
  constexpr int NPART = SPLIT ? 2 : 1;
  constexpr int TPW = kApplyTokens / 16 / 4;         // tiles per wave
  typedef typename Frag<T>::type FragT;
  __shared__ __attribute__((aligned(16))) T sst[NPART * DP * PITCH];
  __shared__ float szp[DK];
  // Blocks in (sample, token range, head) order, head fastest, each XCD
  // taking a contiguous range: the heads of one token range run together on
  // one XCD, whose L2 then merges their partial-line reads of q and writes
  // of y (a head's slice of a token row is d elements, not whole lines).
  const int ntb = (N + kApplyTokens - 1) / kApplyTokens;
  const int lb = xcd_swizzle((int)blockIdx.x, (int)gridDim.x);
  const int h = lb % heads, tb = (lb / heads) % ntb, b = lb / heads / ntb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  const size_t bh = (size_t)b * heads + h;
  const T* gst = st + bh * 2 * DP * DK;

  // Stage the operand: NPART x DP rows of DK elements, 8 elements per thread step.
  for (int e = tid; e < NPART * DP * (DK / 8); e += 256) {
    const int part = e / (DP * (DK / 8));
    const int r = e % (DP * (DK / 8));
    const int row = r / (DK / 8), c8 = (r % (DK / 8)) * 8;
    float v[8];
    load8(gst + (size_t)part * DP * DK + row * DK + c8, v);
    store8(sst + (part * DP + row) * PITCH + c8, v);
  }
  for (int k = tid; k < DK; k += 256) szp[k] = zp[bh * DK + k];
  __syncthreads();

  FragT ahi[DT][KS], alo[DT][KS];
#pragma unroll
  for (int tn = 0; tn < DT; ++tn)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      frag_load(ahi[tn][s], sst + (tn * 16 + fr) * PITCH + s * 32 + g * 8);
      if (SPLIT) frag_load(alo[tn][s], sst + (DP + tn * 16 + fr) * PITCH + s * 32 + g * 8);
    }
  float zr[KS][8];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) zr[s][i] = szp[s * 32 + g * 8 + i];

  const int tile0 = (tb * 4 + wave) * TPW;
  // Query fragments run PD tiles ahead of the matrix work (a ring of PD
  // register sets, about 48 registers), so PD - 1 memory latencies overlap.
  constexpr int QREG = KS * (int)sizeof(FragT) / 4;
  constexpr int PD = 48 / QREG < 2 ? 2 : (48 / QREG > TPW ? TPW : 48 / QREG);
  FragT bq[PD][KS];
  auto load_q = [&](FragT (&dst)[KS], int tile) {
    const int tok = tile * 16 + fr;
    const bool tv = tok < N;
    const T* qrow = q + ((size_t)b * N + (tv ? tok : 0)) * ldq + h * d;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int k = s * 32 + g * 8;
      if (tv && k < d) frag_load(dst[s], qrow + k);
      else frag_zero(dst[s]);
    }
  };
#pragma unroll
  for (int tt = 0; tt < PD - 1; ++tt) load_q(bq[tt], tile0 + tt);
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile = tile0 + tt;
    const int c = tt % PD;
    if (tt + PD - 1 < TPW) load_q(bq[(tt + PD - 1) % PD], tile + PD - 1);
    const int tok = tile * 16 + fr;
    float den = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) den += to_f32(bq[c][s][i]) * zr[s][i];
    den += __shfl_xor(den, 16, 64);
    den += __shfl_xor(den, 32, 64);
    const float inv = 1.0f / (den + eps);
    // The normaliser q . z + eps, kept for the hybrid's exact eta.
    if (den_out && g == 0 && tok < N) den_out[((size_t)b * N + tok) * heads + h] = den + eps;
    f32x4 acc[DT];
#pragma unroll
    for (int tn = 0; tn < DT; ++tn) {
      acc_zero(acc[tn]);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (SPLIT) mma16(acc[tn], alo[tn][s], bq[c][s]);
        mma16(acc[tn], ahi[tn][s], bq[c][s]);
      }
    }
    T* yrow = y + ((size_t)b * N + min(tok, N - 1)) * ldy + h * d;
    if constexpr (SPLIT) {
      // Lanes l and l ^ 16 (g and g ^ 1) hold channels 4g .. 4g+3 of each 16-channel tile. For the tiles tn,
      // tb of a pair, even g keeps tn's four and takes its partner's four of tn, odd g keeps tb's and takes
      // its partner's of tb: every lane then stores 8 consecutive channels (16 bytes; a lone last tile pairs
      // with itself and only even g store).
      uint32_t pk[DT][2];
#pragma unroll
      for (int tn = 0; tn < DT; ++tn) {
        bf16x4 t4;
#pragma unroll
        for (int r = 0; r < 4; ++r) t4[r] = (bf16)(acc[tn][r] * inv);
        pk[tn][0] = reinterpret_cast<const uint32_t*>(&t4)[0];
        pk[tn][1] = reinterpret_cast<const uint32_t*>(&t4)[1];
      }
      const bool odd = (lane & 16) != 0;
      auto from_partner = [&](uint32_t v) {
        const auto pr = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return odd ? pr[0] : pr[1];
      };
#pragma unroll
      for (int tn = 0; tn < DT; tn += 2) {
        const int tb = tn + 1 < DT ? tn + 1 : tn;
        const uint32_t r0 = from_partner(odd ? pk[tn][0] : pk[tb][0]);
        const uint32_t r1 = from_partner(odd ? pk[tn][1] : pk[tb][1]);
        const int n = odd ? tb * 16 + (g - 1) * 4 : tn * 16 + g * 4;
        const uint4 w = odd ? make_uint4(r0, r1, pk[tb][0], pk[tb][1]) : make_uint4(pk[tn][0], pk[tn][1], r0, r1);
        if (tok < N && n < d && !(odd && tb == tn)) *reinterpret_cast<uint4*>(yrow + n) = w;
      }
    } else {
      if (tok < N) {
#pragma unroll
        for (int tn = 0; tn < DT; ++tn) {
          const int n = tn * 16 + g * 4;
          if (n < d) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = acc[tn][r] * inv;
            store4(yrow + n, o);
          }
        }
      }
    }
  }
}

template <typename T>
hipError_t launch_linattn_apply(const T* q, int ldq, const T* st, const float* zp, int B, int N, int heads,
                                int d, float eps, T* y, int ldy, float* den_out, hipStream_t s) {
  const int blocks = (N + kApplyTokens - 1) / kApplyTokens;
  if ((long long)blocks * heads * B >= (1LL << 31)) return hipErrorInvalidValue;
  dim3 grid(blocks * heads * B), block(256);
  switch ((d + 15) / 16) {
#define EDIT_APPLY_CASE(DTV)                                                                        \
  case DTV:                                                                                         \
    hipLaunchKernelGGL((linattn_apply_kernel<T, DTV>), grid, block, 0, s, q, ldq, st, zp, N, heads, d, \
                       eps, y, ldy, den_out);                                                       \
    break;
    EDIT_APPLY_CASE(1) EDIT_APPLY_CASE(2) EDIT_APPLY_CASE(3) EDIT_APPLY_CASE(4)
    EDIT_APPLY_CASE(5) EDIT_APPLY_CASE(6) EDIT_APPLY_CASE(7) EDIT_APPLY_CASE(8)
#undef EDIT_APPLY_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Softmax attention over up to two key/value segments (the hybrid's
// image->text and text->[image;text] blocks), scale 1/sqrt(d), online
// softmax over 32-key slabs. Each wave owns 16 queries. S^T = K Q^T comes out
// with lane l holding 8 key scores of query l % 16, which is exactly the B
// fragment of O^T = V^T P^T when V^T is read with the same key order
// (keys 4g..4g+3 and 16+4g..16+4g+3 for lane group g), so P never leaves
// registers.
// ---------------------------------------------------------------------------
// Position of key k in row `row` (a channel) of the transposed value slab:
// groups of 4 keys are XOR-swizzled by row / 8, so that the staging writes
// (8 channels of one key per thread, 8 rows apart across a wave's lanes) and
// the fragment reads (4 keys of 16 rows) fall in distinct LDS banks.
__device__ __forceinline__ int vt_key(int row, int k) { return ((((k >> 2) ^ (row >> 3)) & 7) << 2) | (k & 3); }

template <typename T, int DT>
__global__ __launch_bounds__(256) void sdpa_kernel(SdpaArgs<T> p) {
  constexpr int KS = (DT + 1) / 2;
  constexpr int DK = 32 * KS;
  constexpr int KPITCH = DK + 8;            // elements; 16 B multiple
  constexpr int VPITCH = 40;
  typedef typename Frag<T>::type FragT;
  __shared__ __attribute__((aligned(16))) T Ks[32 * KPITCH];
  __shared__ __attribute__((aligned(16))) T Vt[16 * DT * VPITCH];
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g = lane >> 4;
  const int d = p.d;
  const float sl2 = 1.4426950408889634f / sqrtf((float)d);   // log2(e) / sqrt(d)

  for (int i = tid; i < 32 * KPITCH; i += 256) Ks[i] = from_f32<T>(0.0f);
  for (int i = tid; i < 16 * DT * VPITCH; i += 256) Vt[i] = from_f32<T>(0.0f);

  // blockIdx.x = split * query blocks + query block; the split takes slabs [jlo, jhi).
  const int nqb = (p.Nq + 63) / 64, sp = (int)blockIdx.x / nqb, qb = (int)blockIdx.x % nqb;
  const int qi = qb * 64 + wave * 16 + fr;
  const bool qv = qi < p.Nq;
  const T* qrow = p.q + ((size_t)b * p.Nq + (qv ? qi : 0)) * p.ldq + h * d;
  FragT bq[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int k = s * 32 + g * 8;
    if (qv && k < d) frag_load(bq[s], qrow + k);
    else frag_zero(bq[s]);
  }
  f32x4 acc[DT];
#pragma unroll
  for (int tn = 0; tn < DT; ++tn) acc_zero(acc[tn]);
  float mrun = -INFINITY, lrun = 0.0f;
  const int dc = d / 8;
  const int Ntot = p.N1 + p.N2;
  __syncthreads();

  // Key/value slabs of 32 keys. A thread's share of a slab (item e: K or V,
  // key, 8-channel chunk) is loaded into registers PF slabs ahead, so that
  // PF slabs' loads are in flight while one is staged in LDS and used; the
  // loop is unrolled by PF so that every ring slot is a compile-time index.
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  constexpr int EPC = 16 / (int)sizeof(T);         // elements per 16 bytes
  constexpr int NIT = (DT + 1) / 2;                // items per thread (2 x 32 keys x d/8 chunks <= 256 NIT)
  constexpr int PF = sizeof(T) == 2 ? 4 : 2;       // slabs in flight
  const int nitems = 2 * 32 * dc;
  const int nslab_all = (Ntot + 31) / 32, spl = (nslab_all + p.splits - 1) / p.splits;
  const int jlo = sp * spl, nslab = max(0, min(nslab_all, jlo + spl) - jlo);
  u32x4v raw[PF][NIT][8 / EPC];
  // A thread's items, the same in every slab: K or V, key within the slab,
  // channel chunk (the divisions by d / 8 done once).
  int it_key[NIT], it_c8[NIT];
  bool it_v[NIT], it_ok[NIT];
#pragma unroll
  for (int u = 0; u < NIT; ++u) {
    const int e = tid + 256 * u, r = e % (32 * dc);
    it_ok[u] = e < nitems;
    it_v[u] = e >= 32 * dc;
    it_key[u] = r / dc;
    it_c8[u] = (r % dc) * 8;
  }
  auto issue = [&](u32x4v (&dst)[NIT][8 / EPC], int k0) {
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
      const bool which = it_v[u];
      const int kk = k0 + it_key[u], c8 = it_c8[u];
      const u32x4v zero = {0u, 0u, 0u, 0u};
      if (it_ok[u] && kk < Ntot) {
        const bool first = kk < p.N1;
        const T* base = first ? (which ? p.v1 : p.k1) : (which ? p.v2 : p.k2);
        const int ld = first ? p.ldkv1 : p.ldkv2;
        const int nseg = first ? p.N1 : p.N2;
        const int j = first ? kk : kk - p.N1;
        const T* src = base + ((size_t)b * nseg + j) * ld + h * d + c8;
#pragma unroll
        for (int w = 0; w < 8 / EPC; ++w) dst[u][w] = *reinterpret_cast<const u32x4v*>(src + w * EPC);
      } else {
#pragma unroll
        for (int w = 0; w < 8 / EPC; ++w) dst[u][w] = zero;
      }
    }
  };
  auto stage = [&](const u32x4v (&src)[NIT][8 / EPC]) {
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
      if (it_ok[u]) {
        const int key = it_key[u], c8 = it_c8[u];
        if (!it_v[u]) {
#pragma unroll
          for (int w = 0; w < 8 / EPC; ++w) *reinterpret_cast<u32x4v*>(Ks + key * KPITCH + c8 + w * EPC) = src[u][w];
        } else {
          const T* v = reinterpret_cast<const T*>(&src[u][0]);
#pragma unroll
          for (int i = 0; i < 8; ++i) Vt[(c8 + i) * VPITCH + vt_key(c8 + i, key)] = v[i];
        }
      }
    }
  };
#pragma unroll
  for (int i = 0; i < PF - 1; ++i)
    if (i < nslab) issue(raw[i], 32 * (jlo + i));

  for (int js0 = 0; js0 < nslab; js0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int js = js0 + u;
      if (js >= nslab) break;
      const int k0 = 32 * (jlo + js);
      if (js + PF - 1 < nslab) issue(raw[(u + PF - 1) % PF], 32 * (jlo + js + PF - 1));
      stage(raw[u]);
      __syncthreads();
      // Scores of keys 16*kt + 4g + r for query fr.
      f32x4 sc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        acc_zero(sc[kt]);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          FragT ak;
          frag_load(ak, Ks + (kt * 16 + fr) * KPITCH + s * 32 + g * 8);
          mma16(sc[kt], ak, bq[s]);
        }
      }
      float pv[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = k0 + kt * 16 + g * 4 + r;
          const float v = kk < Ntot ? sc[kt][r] * sl2 : -INFINITY;
          pv[kt * 4 + r] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(mrun, tmax);
      const float corr = exp2f(mrun - mnew);
      mrun = mnew;
      float psum = 0.0f;
      float pf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pf[i] = exp2f(pv[i] - mnew);
        psum += pf[i];
      }
      lrun = lrun * corr + psum;
      FragT bp;
      frag_from_f32(bp, pf);
#pragma unroll
      for (int tn = 0; tn < DT; ++tn) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[tn][r] *= corr;
        const int row = tn * 16 + fr;
        const T* vrow = Vt + row * VPITCH;
        FragT av;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          av[i] = vrow[vt_key(row, g * 4) + i];
          av[4 + i] = vrow[vt_key(row, 16 + g * 4) + i];
        }
        mma16(acc[tn], av, bp);
      }
      __syncthreads();
    }
  }

  lrun += __shfl_xor(lrun, 16, 64);
  lrun += __shfl_xor(lrun, 32, 64);
  if (p.splits > 1) {
    // This split's partial: unnormalised output, running max (log2 units), running sum.
    if (qv) {
      float* prow = p.part + ((((size_t)sp * p.B + b) * p.heads + h) * p.Nq + qi) * (d + 2);
#pragma unroll
      for (int tn = 0; tn < DT; ++tn) {
        const int n = tn * 16 + g * 4;
        if (n < d) {
#pragma unroll
          for (int r = 0; r < 4; ++r) prow[n + r] = acc[tn][r];
        }
      }
      if (g == 0) {
        prow[d] = mrun;
        prow[d + 1] = lrun;
      }
    }
    return;
  }
  const float inv = 1.0f / lrun;
  if (qv) {
    T* orow = p.out + ((size_t)b * p.Nq + qi) * p.ldo + h * d;
    const T* brow = p.blend_src ? p.blend_src + ((size_t)b * p.Nq + qi) * p.ldbs + h * d : nullptr;
    float alpha = p.alpha, beta = p.beta;
    if (brow && p.lin_den) {
      // Exact eta: the linear block's mass q . z + eps against the softmax
      // block's sum_t exp(s_t) = 2^mrun * lrun (scores are kept in log2 units).
      const float lin = p.lin_den[((size_t)b * p.Nq + qi) * p.heads + h];
      const float soft = exp2f(mrun) * lrun;
      alpha = lin / (lin + soft);
      beta = 1.0f - alpha;
    }
#pragma unroll
    for (int tn = 0; tn < DT; ++tn) {
      const int n = tn * 16 + g * 4;
      if (n < d) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = acc[tn][r] * inv;
        if (brow) {
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = alpha * to_f32(brow[n + r]) + beta * o[r];
        }
        store4(orow + n, o);
      }
    }
  }
}

// Merge of the key splits, one thread per four consecutive outputs of a row:
// with M the largest running max, the output is
// sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, then the same blend as the
// one-pass kernel (the exact eta's softmax mass is 2^M times that
// denominator). Up to kCombineMax splits are read in one round trip (every
// load issued before the first use); more take further passes of the loop.
constexpr int kCombineMax = 8;
template <typename T>
__global__ __launch_bounds__(256) void sdpa_combine_kernel(SdpaArgs<T> p) {
  // grid: (Nq d / 4 / 256, heads, B); thread i of a (sample, head) takes query i / (d / 4), dims 4 (i % (d / 4))
  const int d = p.d, d4 = d / 4, h = blockIdx.y, b = blockIdx.z;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= p.Nq * d4) return;
  const int qi = i / d4, n = (i - qi * d4) * 4;
  const size_t sstride = (size_t)p.B * p.heads * p.Nq * (d + 2);
  // rows of d + 2 floats (d a multiple of 8): the 4 outputs sit 8-byte aligned
  const float* base = p.part + (((size_t)b * p.heads + h) * p.Nq + qi) * (d + 2);
  float M = -INFINITY, L = 0.0f, O[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < p.splits; s0 += kCombineMax) {
    float ms[kCombineMax], ls[kCombineMax];
    float2 oa[kCombineMax], ob[kCombineMax];
#pragma unroll
    for (int j = 0; j < kCombineMax; ++j) {
      ms[j] = -INFINITY;
      ls[j] = 0.0f;
      oa[j] = ob[j] = make_float2(0.0f, 0.0f);
      if (s0 + j < p.splits) {
        const float* ps = base + (s0 + j) * sstride;
        ms[j] = ps[d];
        ls[j] = ps[d + 1];
        oa[j] = *reinterpret_cast<const float2*>(ps + n);
        ob[j] = *reinterpret_cast<const float2*>(ps + n + 2);
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kCombineMax; ++j) Mn = fmaxf(Mn, ms[j]);
    const float c = exp2f(M - Mn);   // 0 on the first pass (M = -inf)
    L *= c;
#pragma unroll
    for (int k = 0; k < 4; ++k) O[k] *= c;
#pragma unroll
    for (int j = 0; j < kCombineMax; ++j) {
      if (s0 + j < p.splits) {
        const float w = exp2f(ms[j] - Mn);
        L += w * ls[j];
        O[0] += w * oa[j].x;
        O[1] += w * oa[j].y;
        O[2] += w * ob[j].x;
        O[3] += w * ob[j].y;
      }
    }
    M = Mn;
  }
  const float inv = 1.0f / L;
  float o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = O[k] * inv;
  if (p.blend_src) {
    float alpha = p.alpha, beta = p.beta;
    if (p.lin_den) {
      const float lin = p.lin_den[((size_t)b * p.Nq + qi) * p.heads + h];
      alpha = lin / (lin + exp2f(M) * L);
      beta = 1.0f - alpha;
    }
    const T* brow = p.blend_src + ((size_t)b * p.Nq + qi) * p.ldbs + h * d + n;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = alpha * to_f32(brow[k]) + beta * o[k];
  }
  store4(p.out + ((size_t)b * p.Nq + qi) * p.ldo + h * d + n, o);
}

int sdpa_splits(int Nq, int Nkeys, int heads, int B, int d, bool staged) {
  if (staged) return std::max(1, (Nkeys + sdpa_staged_keys(d) - 1) / sdpa_staged_keys(d));
  const long long base = (long long)((Nq + 63) / 64) * heads * B;
  const int nslab = (Nkeys + 31) / 32;
  if (base <= 0 || nslab <= 0) return 1;
  long long s = (2048 + base - 1) / base;
  s = std::min<long long>(s, (nslab + 3) / 4);
  return (int)std::max<long long>(1, std::min<long long>(s, 32));
}

template <typename T>
hipError_t launch_sdpa_combine(const SdpaArgs<T>& a, hipStream_t s) {
  const long long per_head = (long long)a.Nq * (a.d / 4);
  if (a.d % 8 || per_head >= (1LL << 31) - 256 || a.heads > 65535 || a.B > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((sdpa_combine_kernel<T>), dim3((unsigned)((per_head + 255) / 256), a.heads, a.B), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_sdpa(const SdpaArgs<T>& a0, hipStream_t s) {
  if (a0.Nq <= 0) return hipSuccess;
  SdpaArgs<T> a = a0;
  if constexpr (std::is_same<T, bf16>::value) {
    // the staged kernel: splits of at most sdpa_staged_keys(d) keys
    hipError_t e = launch_sdpa_staged(&a, 1, s);
    if (e != hipSuccess || a.splits == 1) return e;
    return launch_sdpa_combine(a, s);
  }
  if (a.splits < 1 || a.part == nullptr) a.splits = 1;
  const long long gx = (long long)((a.Nq + 63) / 64) * a.splits;
  if (gx >= (1LL << 31)) return hipErrorInvalidValue;
  dim3 grid((unsigned)gx, a.heads, a.B), block(256);
  switch ((a.d + 15) / 16) {
#define EDIT_SDPA_CASE(DTV) \
  case DTV: hipLaunchKernelGGL((sdpa_kernel<T, DTV>), grid, block, 0, s, a); break;
    EDIT_SDPA_CASE(1) EDIT_SDPA_CASE(2) EDIT_SDPA_CASE(3) EDIT_SDPA_CASE(4)
    EDIT_SDPA_CASE(5) EDIT_SDPA_CASE(6) EDIT_SDPA_CASE(7) EDIT_SDPA_CASE(8)
#undef EDIT_SDPA_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_sdpa_combine(a, s);
}

template <typename T>
hipError_t launch_sdpa_pair(const SdpaArgs<T>& a, const SdpaArgs<T>& b, hipStream_t s) {
  if constexpr (std::is_same<T, bf16>::value) {
    // one staged launch over both problems, then the merge of each one's key splits
    SdpaArgs<T> j[2] = {a, b};
    int n = 0;
    if (a.Nq > 0) j[n++] = a;
    if (b.Nq > 0) j[n++] = b;
    if (n == 0) return hipSuccess;
    hipError_t e = launch_sdpa_staged(j, n, s);
    for (int i = 0; i < n && e == hipSuccess; ++i)
      if (j[i].splits > 1) e = launch_sdpa_combine(j[i], s);
    return e;
  }
  hipError_t e = launch_sdpa<T>(a, s);
  return e != hipSuccess ? e : launch_sdpa<T>(b, s);
}

#define EDIT_INST(T)                                                                                     \
  template hipError_t launch_kv_state<T>(const T*, const T*, int, int, int, int, int, float*, int, float*, \
                                         float*, T*, float*, hipStream_t, const float*);                              \
  template hipError_t launch_dwconv_kv_state<T>(const T*, int, int, int, int, int, int, const T*, const T*,       \
                                                const T*, const T*, T*, T*, float*, int, hipStream_t);            \
  template hipError_t launch_kv_state_finalize<T>(const float*, int, int, int, int, float*, float*, T*, float*,   \
                                                  hipStream_t);                                                   \
  template hipError_t launch_linattn_apply<T>(const T*, int, const T*, const float*, int, int, int, int, \
                                              float, T*, int, float*, hipStream_t);                     \
  template hipError_t launch_sdpa<T>(const SdpaArgs<T>&, hipStream_t);                                      \
  template hipError_t launch_sdpa_pair<T>(const SdpaArgs<T>&, const SdpaArgs<T>&, hipStream_t);
EDIT_INST(bf16)
EDIT_INST(float)
#undef EDIT_INST

}  // namespace edit
