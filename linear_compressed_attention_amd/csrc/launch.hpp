// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>

#include "fold.hpp"

namespace edit {

typedef __bf16 bf16;

// How the GEMM's A operand is produced from memory.
enum AMode {
  A_PLAIN = 0,   // A[m][k] = a[m*lda + k]
  A_CONV3 = 1,   // implicit 3x3 stride-1 pad-1 convolution: k = tap*Cin + cin over an image [B][H][W][Cin]
  A_CAT2 = 2     // two row sources side by side: A[m][k] = a[m*lda + k] for k < K1, else a2[m*lda2 + k - K1]
};
// What the epilogue adds before the store.
enum EMode {
  E_BIAS = 0,       // C = acc + bias
  E_BIAS_RELU = 1,  // C = max(acc + bias, 0)
  E_F32 = 2,        // Cf[split][m][n] = acc (fp32, no bias): one K slice of a split-K product
  E_RES = 3,        // C = acc + bias + R (launch_gemm picks it for E_BIAS when GemmArgs::R is set)
  E_BIAS_GN = 4     // C = acc + bias, and GroupNorm partial statistics of the stored tile into gnp
};

// C[M][N] = A[M][K] * B[N][K]^T + epilogue. B and the bias may come in up
// to three row segments of seg_rows rows each (segment s covers rows
// s*seg_rows .. (s+1)*seg_rows-1), so [W_k; W_v] or [W_q; W_k; W_v] need no
// concatenated copy.
template <typename T>
struct GemmArgs {
  int M, N, K;
  const T* A;
  int lda;
  int H, W, Cin;               // A_CONV3 geometry (M = B*H*W, K = 9*Cin)
  const T* A2;                 // A_CAT2: second source, columns K1 .. K-1
  int lda2;
  int K1;
  const T* Bseg[3];
  const T* bias[3];
  int seg_rows;
  int ldb;
  T* C;
  int ldc;
  int spread;                  // 1: one block per tile, so that the hardware hands tiles to CUs as
                               // they free up (for GEMMs that share the chip with another stream)
  // E_F32: K is cut into slices of kchunk (a multiple of 64); slice s writes Cf + s * split_stride
  // with row stride ldc (register-staged kernel: one grid row per slice; DMA kernel: tile index
  // = slice * output tiles + output tile).
  float* Cf;
  long long split_stride;
  int kchunk;
  // E_BIAS with R set (run as E_RES): C = A B^T + bias + R (R [M][ldr], the same type as C).
  const T* R;
  int ldr;
  // E_BIAS_GN (the direct-load conv only): per output tile of gn_rows rows and every column n,
  // gnp[(m0 / gn_rows) * N + n] = (mean, sum of squared deviations) of the stored values.
  float* gnp;
  int gn_rows;
  // bf16 A_CONV3 with fold.W set: the restore fold (fold.hpp) is also computed, by extra blocks of the
  // conv's launch where its tiles leave CUs idle, else by the fold's own kernel after it.
  FoldArgs fold;
  int fold_blocks;             // set by the launcher
};

template <typename T>
hipError_t launch_gemm(const GemmArgs<T>& a, AMode am, EMode em, hipStream_t s);

// The bf16 3x3 conv (A_CONV3, E_BIAS or E_BIAS_GN with 256-row statistics
// tiles) on the halo-staged implicit GEMM (conv_halo.hip): H*W a multiple of
// 256, W in {32, 64, 128} or a multiple of 256, C a multiple of 16, N of 96.
// Returns hipErrorNotSupported, launching nothing, for other shapes.
hipError_t launch_conv3x3_halo(const GemmArgs<bf16>& a, EMode em, hipStream_t s);

// The bf16 GEMM with direct global-to-LDS loads (plain or 3x3-conv A, bias or
// bias + ReLU epilogue). Returns hipErrorNotSupported, launching nothing, for
// shapes it does not cover.
hipError_t launch_gemm_dma(const GemmArgs<bf16>& a, AMode am, EMode em, hipStream_t s);

// GroupNorm statistics of x [B][HW][C] (G groups of C/G consecutive
// channels): per (b, group) mean and rstd, and the per-channel affine folded
// into scale/shift [B][C]. partial holds [B][nchunks][G][2] floats.
template <typename T>
hipError_t launch_groupnorm_stats(const T* x, int B, int HW, int C, int G, const T* gamma,
                                  const T* beta, float eps, float* partial, int nchunks,
                                  float* stat, float* scale, float* shift, hipStream_t s);
int groupnorm_chunks(int HW, int C);
// GroupNorm statistics from per-(tile, channel) partials (mean, M2) of tiles of `rows` rows
// (partial [B * HW / rows][C][2]; HW a multiple of rows): stat, scale and shift as launch_groupnorm_stats.
template <typename T>
hipError_t launch_groupnorm_finalize_channels(const float* partial, int B, int HW, int C, int G, int rows,
                                              const T* gamma, const T* beta, float eps, float* stat, float* scale,
                                              float* shift, hipStream_t s);

// The ConvFusion 1x1 restore (W2 [C][Cr], b2 [C]) folded into a Linear
// (W [C][C], b [C]) that reads X + act W2^T + b2: wcat [C][C + Cr] = [W | W W2],
// bcat [C] = b + W b2, for an A_CAT2 GEMM over [X | act].
template <typename T>
hipError_t launch_restore_fold(const T* W, const T* b, const T* W2, const T* b2, int C, int Cr, T* wcat, T* bcat,
                               hipStream_t s);

// a = LeakyReLU(x * scale[b] + shift[b], 0.01) elementwise over x [B][HW][C].
template <typename T>
hipError_t launch_groupnorm_apply(const T* x, int B, int HW, int C, const float* scale, const float* shift, T* a,
                                  hipStream_t s);

// Depthwise 3x3 stride-2 pad-1 conv of two channel groups side by side in
// kv0 [B][H][W][2C]: keys (channels 0..C-1, then ReLU) and values (C..2C-1).
template <typename T>
hipError_t launch_dwconv_s2(const T* kv0, int B, int H, int W, int C, const T* dwk, const T* dbk,
                            const T* dwv, const T* dbv, T* kc, T* vc, hipStream_t s);

// Per-head state of the compressed keys/values: S = K'^T V', z = sum K'.
// kc and vc rows (tokens) are ld elements apart.
// Writes f32 S [B][h][d][d], z [B][h][d] and the apply kernel's operand:
// st [B][h][2][DP][DK] of T (S transposed, split hi/lo for bf16), zp [B][h][DK] f32.
// wrow (optional, [B][Nc][heads] f32) weights each token's term of z.
template <typename T>
hipError_t launch_kv_state(const T* kc, const T* vc, int ld, int B, int Nc, int heads, int d, float* partial,
                           int nchunks, float* S, float* z, T* st, float* zp, hipStream_t s,
                           const float* wrow = nullptr);
int kv_state_chunks(int Nc);
// Chunks of the fused depthwise + state kernel: th x tw compressed tokens (th * tw = 256), ncy x ncx of them
// over an Hc x Wc grid.
struct DwStateTile { int th, tw, ncy, ncx; };
DwStateTile dw_state_tile(int Hc, int Wc);
int dw_state_chunks(int Hc, int Wc);
// The depthwise stride-2 convs (as launch_dwconv_s2) and the per-head state partials (one per chunk, as
// launch_kv_state's first kernel forms them from kc, vc, but over dw_state_tile's 2-D chunks of the
// compressed grid) in one pass over kv0: kc, vc are written and the partials [B][h][nchunks][..] formed from
// the values on chip; launch_kv_state_finalize then merges them. nchunks must be dw_state_chunks(Hc, Wc)
// (else hipErrorInvalidValue). bf16 only (hipErrorNotSupported, nothing launched, for fp32).
template <typename T>
hipError_t launch_dwconv_kv_state(const T* kv0, int B, int H, int W, int C, int heads, int d, const T* dwk,
                                  const T* dbk, const T* dwv, const T* dbv, T* kc, T* vc, float* partial,
                                  int nchunks, hipStream_t s);
// S, z, st, zp of launch_kv_state from its chunk partials (summed in chunk order).
template <typename T>
hipError_t launch_kv_state_finalize(const float* partial, int B, int heads, int d, int nchunks, float* S, float* z,
                                    T* st, float* zp, hipStream_t s);

// ---- backward (backward.hip) ----
// out[c][r] = in[r][c] (row strides ldi, ldo), for z < batch at in + z * zin, out + z * zout.
// Output columns rows .. rows_pad - 1 are written as zeros. colsum (optional,
// fp32): per 64-row tile t = 0 .. ceil(rows_pad / 64) - 1, the sum of that
// tile's rows of in, at colsum[(z * cols + c) * tiles + t]. in2 (optional): the input of z = 1
// instead of in + zin.
template <typename T>
hipError_t launch_transpose(const T* in, int rows, int cols, int ldi, T* out, int ldo, hipStream_t s,
                            int rows_pad = 0, int batch = 1, long zin = 0, long zout = 0, float* colsum = nullptr,
                            const T* in2 = nullptr);
// For every tap t = 3 ky + kx of the 3x3 conv: out[t][c][m'] = in[m' - off][c],
// zero where that tap does not connect the two pixels (and in the padding up
// to ldo); in is [B*H*W][ldi], out [9][cols][ldo]. colsum as for launch_transpose
// (tap t as z, ceil(ldo / 64) tiles).
template <typename T>
hipError_t launch_shift_transpose9(const T* in, int B, int H, int W, int cols, int ldi, T* out, int ldo,
                                   hipStream_t s, float* colsum = nullptr);
// out[r] = sum_t part[r * n + t] for t < n (the per-tile sums a transpose wrote), fixed order; out32 optional.
// Rows from rsplit on (when out2 is given) go to out2[r - rsplit], without the fp32 copy.
template <typename T>
hipError_t launch_colsum_finalize(const float* part, int rows, int n, T* out, hipStream_t s, float* out32 = nullptr,
                                  T* out2 = nullptr, int rsplit = 0);
template <typename T>
hipError_t launch_zero(T* p, long n, hipStream_t s);
// out[(r % rpg) * ldo + (r / rpg) * gstride + c] = sum_s part[s * stride + r * cols + c] (rpg 0: rows).
// With out2, rows r >= rsplit go to out2 at row r - rsplit instead (rpg 0: rsplit). With bias, bias[c] is
// added to every row's sum.
template <typename O, typename O2 = O>
hipError_t launch_splitk_reduce(const float* part, int S, long long stride, int rows, int cols, O* out, int ldo,
                                hipStream_t s, int rpg = 0, int gstride = 0, O2* out2 = nullptr, int rsplit = 0,
                                const O* bias = nullptr);
// Linear-attention backward, query side: g = dy / den, c = -(dy . y) / den, dq_pre = (g S^T + c z) where q > 0.
template <typename T>
hipError_t launch_attn_bwd_q(const T* dy, const T* q, const float* S, const float* z, int B, int N, int heads, int d,
                             float eps, T* g, float* c, T* dq_pre, hipStream_t s);
// dkv [B][Nc][2C] (fp32) = [ (V' dS^T + dz) where K' > 0 | K' dS ].
template <typename T>
hipError_t launch_kv_bwd(const T* kc, const T* vc, const float* dS, const float* dz, int B, int Nc, int heads,
                         int d, float* dkv, hipStream_t s);
// Depthwise 3x3 stride-2 backward over 2C channels (dout fp32): input gradient, and weight / bias
// gradients; bk / bv also receive the input gradient's sums over pixels (the key / value Linears'
// bias gradients), formed from the fp32 dout.
template <typename T>
hipError_t launch_dw_bwd_input(const float* dout, int B, int H, int W, int C, const T* dwk, const T* dwv, T* din,
                               hipStream_t s);
int dw_bwd_chunks(int B, int H, int W);
template <typename T>
hipError_t launch_dw_bwd_weight(const float* dout, const T* in, const T* wk, const T* wv, int B, int H, int W, int C,
                                float* partial, T* dwk, T* dbk, T* dwv, T* dbv, T* bk, T* bv, hipStream_t s);
// GroupNorm + LeakyReLU backward: dgamma, dbeta and dxc from dact (partial: B x gn_bwd_chunks(N) x C x 2 floats).
int gn_bwd_chunks(int N);
template <typename T>
hipError_t launch_gn_bwd(const T* dact, const T* act, const T* xc, const float* stat, const T* gamma, int B, int N,
                         int C, int G, float* partial, float* m12, T* dgamma, T* dbeta, T* dxc, int lddxc,
                         hipStream_t s);
// out[i][j] = add[i][j] + ru[i] rv[j] + sum_k A[i][k] B[j][k] (A fp32 [M][lda], B [N][ldb]; add, ru optional).
template <typename TB, typename TO>
hipError_t launch_small_nt(int M, int N, int K, const float* A, int lda, const TB* Bm, int ldb, const float* add,
                           int ldadd, TO* out, int ldo, hipStream_t s, const float* ru = nullptr,
                           const TB* rv = nullptr);
int kv_state_dp(int d);   // padded rows of the state operand
int kv_state_dk(int d);   // padded K of the state operand

// y[b][n][h*d + j] = (q S)_j / (q . z + eps) per head. If den_out is given it
// receives q . z + eps as [B][N][heads] floats.
template <typename T>
hipError_t launch_linattn_apply(const T* q, int ldq, const T* st, const float* zp, int B, int N,
                                int heads, int d, float eps, T* y, int ldy, float* den_out, hipStream_t s);

// Softmax attention of queries q over up to two key/value segments, per head,
// scale 1/sqrt(d). If blend_src is given: out = alpha * blend_src + beta * attn.
template <typename T>
struct SdpaArgs {
  const T* q; int ldq; int Nq;
  const T* k1; const T* v1; int ldkv1; int N1;
  const T* k2; const T* v2; int ldkv2; int N2;
  int B, heads, d;
  T* out; int ldo;
  const T* blend_src; int ldbs; float alpha, beta;
  // If set (with blend_src): alpha = L / (L + sum_t exp(s_t)) per query and
  // head, L = lin_den[b][query][head], beta = 1 - alpha.
  const float* lin_den;
  // If set (bf16, staged kernel, d <= 64): the blend's linear part is formed
  // in the kernel from the head's state instead of read from blend_src:
  // lin_st[B][heads][2][DP][DK] (S^T as bf16 hi + lo, as the apply kernel
  // reads it), lin_zp[B][heads][DK] (z), y_lin = q S / (q . z + lin_eps);
  // with exact_eta, L = q . z + lin_eps in the formula above.
  const T* lin_st;
  const float* lin_zp;
  float lin_eps;
  int exact_eta;
  float* lin_den_out;   // if set (with lin_st): q . z + lin_eps per [b][query][head]
  // Key splits (1: one pass over all keys). With splits > 1 each block takes
  // one split's slabs and writes fp32 partials [split][B][heads][Nq][d + 2]
  // (unnormalised output, running max, running sum) to part, and a second
  // kernel merges them in split order, then normalises and blends.
  int splits;
  float* part;
};
template <typename T>
hipError_t launch_sdpa(const SdpaArgs<T>& a, hipStream_t s);
// Key splits for Nq queries over Nkeys keys: enough blocks for the chip
// (about 2048) with at least four 32-key slabs per split, at most 32.
// bf16 (staged): one split per sdpa_staged_keys(d) keys (the keys a block stages at once).
int sdpa_splits(int Nq, int Nkeys, int heads, int B, int d, bool staged);
int sdpa_staged_keys(int d);
// Whether the staged kernel forms the image rows' linear part itself (lin_st): bf16 with d <= 64.
bool sdpa_staged_fuses_linear(int d);
// Two softmax problems of one head geometry: bf16 runs both in one staged
// launch (their blocks share the chip), then merges each one's key splits;
// fp32 runs them one after the other. Each problem's partials need a buffer
// of its own.
template <typename T>
hipError_t launch_sdpa_pair(const SdpaArgs<T>& a, const SdpaArgs<T>& b, hipStream_t s);
// The bf16 softmax kernel with the keys staged in LDS (sdpa_staged.hip), over
// one or two problems with the same d: one pass each, or with splits > 1 the
// fp32 partials for sdpa_combine_kernel.
hipError_t launch_sdpa_staged(const SdpaArgs<bf16>* jobs, int njobs, hipStream_t s);

}  // namespace edit
