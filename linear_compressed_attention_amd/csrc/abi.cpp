// C ABI of the EDiT layer and the MM-EDiT hybrid: argument checks, workspace
// layout and the launch sequence. Declared in include/edit_attn.h.
//
// Launch sequence of one EDiT layer (page "EDiT: Efficient Diffusion
// Transformers with Linear Compressed Attention", ICCV 2025 notes):
//   section "ConvFusion":
//     1 gemm A_CONV3      xc  = Conv3x3(x) + b_cf1               (C -> C/r)
//     2 groupnorm stats   per (b, group) mean / rstd -> scale, shift
//     3 gn apply, fold    act = LeakyReLU(GN(xc)); wcat = [W_q | W_q W_cf2],
//                         bcat = b_q + W_q b_cf2 (the 1x1 restore folded into W_q)
//     4 gemm A_CAT2 relu  q   = ReLU([x | act] wcat^T + bcat)
//                             = ReLU((x + act W_cf2^T + b_cf2) W_q^T + b_q)
//   section "Spatial Compressor":
//     5 gemm (2 segments) kv0 = [x W_k^T + b_k | x W_v^T + b_v]
//     6 dwconv_s2         kc  = ReLU(DW(k0)), vc = DW(v0)
//   section "Linear-attention formula":
//     7 kv_state          S = kc^T vc, z = sum kc (per head)
//     8 linattn_apply     y = q S / (q . z + eps)
//   output Linear:
//     9 gemm              out = y W_o^T + b_o
// The hybrid (section "MM-EDiT") adds the text Q/K/V Linears (one gemm with
// three segments), image rows eta * y + (1 - eta) * softmax(q K_T^T) V_T,
// text rows over [kc ; K_T], and the text output Linear.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>

#include "../../include/edit_attn.h"
#include "launch.hpp"

using edit::bf16;

// Scratch of edit_attn_forward_noalloc: one array per device, in the code object, so that the call
// itself allocates nothing. On the host the array's name is a stand-in, not device memory: host code
// uses only the address static_scratch() looks up. Every no-allocation call on a device shares the
// array, so such calls that overlap in time on one device race.
static __device__ __align__(256) unsigned char scratch[EDIT_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

edit_status_t fail(edit_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// The bits of an enum field as an int (the C ABI's enums are int-sized).
template <typename E>
int enum_int(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

struct Geometry {
  int B, H, W, C, heads, d, r, G, Cr, N, M, Hc, Wc, Nc, nt;
  int qmode, kvmode;   // edit_query_mode_t, edit_kv_mode_t (the layer itself: 0, 0)
  int Nkv;             // tokens the per-head sums run over (Nc, or N for uncompressed keys)
  int gn_chunks, kv_chunks, DT, DR, DP, DK;
  size_t es;
  float eps;
  edit_dtype_t dtype;
};

// Output Linears with few 128-row tiles (the hybrid's text rows) leave most CUs idle: bf16 cuts K = C into
// S slices (multiples of 64) whose fp32 partials a second kernel sums with the bias; S keeps the tiles of
// all slices within one per CU. 1: no split.
int out_splits(int M, int C, int es) {
  if (es != 2 || C % 192 != 0) return 1;
  const long tiles = (long)((M + 127) / 128) * (C / 192);
  int S = 1;
  for (int k = 2; k <= 8; ++k)
    if ((C / 64) % k == 0 && tiles * k <= 256) S = k;
  return S;
}

struct Layout {
  size_t xc, gn_part, gn_stat, gn_scale, gn_shift, cf_act, q_fold_w, q_fold_b, q, kv0, kc, vc, kv_part, S, z, st,
      zp, y;
  size_t qkv_t, y_img, y_txt, lin_den, sdpa_part_img, sdpa_part_txt, out_part_txt;
  size_t xc_k, gn_part_k, gn_stat_k, gn_scale_k, gn_shift_k, cf_act_k, k_fold_w, k_fold_b;   // key ConvFusion branch
  size_t total;
};

// State partials per (sample, head): the bf16 compressed path forms them in the depthwise kernel over 2-D
// tiles of the compressed grid, every other path over runs of consecutive key/value tokens.
int state_chunks(const Geometry& g) {
  if (g.kvmode == EDIT_KV_COMPRESSED && g.es == 2) return edit::dw_state_chunks(g.Hc, g.Wc);
  return edit::kv_state_chunks(g.Nkv);
}

edit_status_t check_shape(const edit_shape_t* s, int n_text, Geometry* g) {
  if (!s) return fail(EDIT_ERR_ARG, "shape is NULL");
  if (s->B <= 0 || s->H <= 0 || s->W <= 0 || s->C <= 0 || s->heads <= 0 || s->head_dim <= 0 ||
      s->reduction <= 0 || s->gn_groups <= 0)
    return fail(EDIT_ERR_ARG, "every size must be positive (B=%d H=%d W=%d C=%d heads=%d head_dim=%d r=%d G=%d)",
                s->B, s->H, s->W, s->C, s->heads, s->head_dim, s->reduction, s->gn_groups);
  if ((long)s->heads * s->head_dim != s->C)
    return fail(EDIT_ERR_ARG, "C (%d) must equal heads (%d) * head_dim (%d)", s->C, s->heads, s->head_dim);
  if (s->C % s->reduction != 0)
    return fail(EDIT_ERR_ARG, "reduction %d does not divide C %d", s->reduction, s->C);
  const int Cr = s->C / s->reduction;
  if (Cr % s->gn_groups != 0)
    return fail(EDIT_ERR_ARG, "gn_groups %d does not divide C/r %d", s->gn_groups, Cr);
  if (!(s->eps >= 0.0f) || !std::isfinite(s->eps)) return fail(EDIT_ERR_ARG, "eps must be finite and >= 0");
  // A C caller may put any int in an enum field: read it as an int, since a C++ load of an enum
  // value outside the enumerators' range is undefined.
  const int dt = enum_int(s->dtype);
  if (dt != EDIT_F32 && dt != EDIT_BF16) return fail(EDIT_ERR_ARG, "unknown dtype %d", dt);
  if (n_text < 0) return fail(EDIT_ERR_ARG, "n_text must be >= 0 (got %d)", n_text);
  if (s->C % 8 || Cr % 8 || s->head_dim % 8)
    return fail(EDIT_ERR_UNSUPPORTED, "C (%d), C/r (%d) and head_dim (%d) must be multiples of 8", s->C, Cr,
                s->head_dim);
  if (s->head_dim > 128) return fail(EDIT_ERR_UNSUPPORTED, "head_dim %d > 128", s->head_dim);
  if (Cr > 2048) return fail(EDIT_ERR_UNSUPPORTED, "C/r %d > 2048", Cr);
  const long N = (long)s->H * s->W, M = N * s->B;
  if (M * 2L * s->C >= (1L << 31) || (long)s->B * n_text * 3L * s->C >= (1L << 31))
    return fail(EDIT_ERR_UNSUPPORTED, "tensor too large for 32-bit row indexing");
  g->B = s->B; g->H = s->H; g->W = s->W; g->C = s->C; g->heads = s->heads; g->d = s->head_dim;
  g->r = s->reduction; g->G = s->gn_groups; g->Cr = Cr; g->N = (int)N; g->M = (int)M;
  g->Hc = (s->H + 1) / 2; g->Wc = (s->W + 1) / 2; g->Nc = g->Hc * g->Wc; g->nt = n_text;
  g->qmode = EDIT_QUERY_CONVFUSION; g->kvmode = EDIT_KV_COMPRESSED; g->Nkv = g->Nc;
  g->gn_chunks = edit::groupnorm_chunks(g->N, Cr);
  g->DT = (g->d + 15) / 16; g->DR = (g->d + 16) / 16;
  g->DP = edit::kv_state_dp(g->d); g->DK = edit::kv_state_dk(g->d);
  g->es = s->dtype == EDIT_BF16 ? 2 : 4;
  g->kv_chunks = state_chunks(*g);
  g->eps = s->eps;
  g->dtype = s->dtype;
  return EDIT_OK;
}

// The query / key-value processing of the ablation variants.
edit_status_t apply_variant(const edit_variant_t* v, Geometry* g) {
  if (!v) return fail(EDIT_ERR_ARG, "variant is NULL");
  const int qm = enum_int(v->query), kvm = enum_int(v->kv);
  if (qm != EDIT_QUERY_CONVFUSION && qm != EDIT_QUERY_LINEAR)
    return fail(EDIT_ERR_ARG, "unknown query mode %d", qm);
  if (kvm != EDIT_KV_COMPRESSED && kvm != EDIT_KV_FULL && kvm != EDIT_KV_KEY_CONVFUSION)
    return fail(EDIT_ERR_ARG, "unknown key/value mode %d", kvm);
  g->qmode = qm;
  g->kvmode = kvm;
  g->Nkv = kvm == EDIT_KV_COMPRESSED ? g->Nc : g->N;
  g->kv_chunks = state_chunks(*g);
  return EDIT_OK;
}

// The bf16 conv computes the GroupNorm partial statistics in its epilogue when its row tiles never
// straddle two samples (H*W a multiple of the tile height) and it runs on the direct-load kernel (C a
// multiple of 64, C/r of 96); otherwise a separate pass over xc does. Tiles are 256 rows on the
// kernel-row conv; on the tap-streaming conv 256, or 128 where 256-row tiles (x C/r / 96 column tiles)
// would fill fewer than half of an MI355X's 256 CUs.
int gn_tile_rows(const Geometry& g) {
  // the kernel-row conv (conv_halo.hip) takes 256-row tiles of whole image rows or row segments
  const bool rows_conv = g.es == 2 && g.N % 256 == 0 && g.C % 64 == 0 && g.Cr % 96 == 0 &&
                         (g.W == 32 || g.W == 64 || g.W == 128 || g.W % 256 == 0);
  if (rows_conv) return 256;
  const long tiles256 = (long)(g.M / 256) * (g.Cr / 96);
  return tiles256 < 128 && g.N % 128 == 0 ? 128 : 256;
}
bool gn_in_conv(const Geometry& g) {
  return g.es == 2 && g.N % gn_tile_rows(g) == 0 && g.C % 64 == 0 && g.Cr % 96 == 0 &&
         (size_t)g.M * g.C * 2 < 0x80000000ull && (size_t)g.Cr * 9 * g.C * 2 < 0x80000000ull;
}
size_t gn_part_bytes(const Geometry& g) {
  const size_t sep = (size_t)g.B * g.gn_chunks * g.G * 2 * 4;
  const size_t fused = gn_in_conv(g) ? (size_t)g.M / gn_tile_rows(g) * g.Cr * 2 * 4 : 0;
  return sep > fused ? sep : fused;
}

Layout make_layout(const Geometry& g) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t M = g.M, es = g.es, BH = (size_t)g.B * g.heads;
  if (g.qmode == EDIT_QUERY_CONVFUSION) {
    L.xc = take(M * g.Cr * es);
    L.gn_part = take(gn_part_bytes(g));
    L.gn_stat = take((size_t)g.B * g.G * 2 * 4);
    L.gn_scale = take((size_t)g.B * g.Cr * 4);
    L.gn_shift = take((size_t)g.B * g.Cr * 4);
    L.cf_act = take(M * g.Cr * es);
    L.q_fold_w = take((size_t)g.C * (g.C + g.Cr) * es);
    L.q_fold_b = take((size_t)g.C * es);
  }
  L.q = take(M * g.C * es);
  L.kv0 = take(M * 2 * g.C * es);
  if (g.kvmode == EDIT_KV_COMPRESSED) {
    L.kc = take((size_t)g.B * g.Nc * g.C * es);
    L.vc = take((size_t)g.B * g.Nc * g.C * es);
  }
  if (g.kvmode == EDIT_KV_KEY_CONVFUSION) {
    L.xc_k = take(M * g.Cr * es);
    L.gn_part_k = take(gn_part_bytes(g));
    L.gn_stat_k = take((size_t)g.B * g.G * 2 * 4);
    L.gn_scale_k = take((size_t)g.B * g.Cr * 4);
    L.gn_shift_k = take((size_t)g.B * g.Cr * 4);
    L.cf_act_k = take(M * g.Cr * es);
    L.k_fold_w = take((size_t)g.C * (g.C + g.Cr) * es);
    L.k_fold_b = take((size_t)g.C * es);
  }
  L.kv_part = take(BH * g.kv_chunks * (16 * g.DR) * (16 * g.DT) * 4);
  L.S = take(BH * g.d * g.d * 4);
  L.z = take(BH * g.d * 4);
  L.st = take(BH * 2 * g.DP * g.DK * es);
  L.zp = take(BH * g.DK * 4);
  L.y = take(M * g.C * es);
  if (g.nt > 0) {
    L.qkv_t = take((size_t)g.B * g.nt * 3 * g.C * es);
    L.y_img = take(M * g.C * es);
    L.y_txt = take((size_t)g.B * g.nt * g.C * es);
    L.lin_den = take((size_t)g.B * g.N * g.heads * 4);
    // the softmax blocks' key-split partials, image rows and text rows apart (bf16 runs both at once); none
    // for a block that takes all its keys in one split
    const bool staged = g.es == 2;
    const int si = edit::sdpa_splits(g.N, g.nt, g.heads, g.B, g.d, staged);
    const int st = edit::sdpa_splits(g.nt, g.Nc + g.nt, g.heads, g.B, g.d, staged);
    L.sdpa_part_img = take(si > 1 ? (size_t)si * g.B * g.heads * g.N * (g.d + 2) * 4 : 0);
    L.sdpa_part_txt = take(st > 1 ? (size_t)st * g.B * g.heads * g.nt * (g.d + 2) * 4 : 0);
    const int so = out_splits(g.B * g.nt, g.C, g.es);
    L.out_part_txt = take(so > 1 ? (size_t)so * g.B * g.nt * g.C * 4 : 0);
  }
  L.total = off;
  return L;
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

edit_status_t check_ptr(const void* p, const char* name) {
  if (!p) return fail(EDIT_ERR_ARG, "%s is NULL", name);
  if (misaligned(p, 16)) return fail(EDIT_ERR_ARG, "%s is not 16-byte aligned", name);
  return EDIT_OK;
}

// The parameters a geometry's variant reads: the ConvFusion set only with a
// ConvFusion query, the depthwise set only with compressed keys and values.
edit_status_t check_weights(const edit_weights_t* w, const Geometry& g) {
  if (!w) return fail(EDIT_ERR_ARG, "weights struct is NULL");
  const void* p[] = {w->w_q, w->b_q, w->w_k, w->b_k, w->w_v, w->b_v, w->w_o, w->b_o, w->w_cf1, w->b_cf1,
                     w->gn_gamma, w->gn_beta, w->w_cf2, w->b_cf2, w->dw_k, w->db_k, w->dw_v, w->db_v};
  const char* n[] = {"w_q", "b_q", "w_k", "b_k", "w_v", "b_v", "w_o", "b_o", "w_cf1", "b_cf1",
                     "gn_gamma", "gn_beta", "w_cf2", "b_cf2", "dw_k", "db_k", "dw_v", "db_v"};
  for (int i = 0; i < 18; ++i) {
    if (i >= 8 && i < 14 && g.qmode != EDIT_QUERY_CONVFUSION) continue;
    if (i >= 14 && g.kvmode != EDIT_KV_COMPRESSED) continue;
    edit_status_t st = check_ptr(p[i], n[i]);
    if (st != EDIT_OK) return st;
  }
  return EDIT_OK;
}

// Elements of each edit_weights_t member, in its declaration order.
void weight_elems(const Geometry& g, size_t (&ne)[18]) {
  const size_t C = g.C, Cr = g.Cr;
  const size_t v[18] = {Cr * 9 * C, Cr, Cr, Cr, C * Cr, C, C * C, C, C * C, C, C * C, C, 9 * C, C, 9 * C, C,
                        C * C, C};
  for (int i = 0; i < 18; ++i) ne[i] = v[i];
}
void weight_ptrs(const edit_weights_t* w, const void* (&p)[18]) {
  const void* v[18] = {w->w_cf1, w->b_cf1, w->gn_gamma, w->gn_beta, w->w_cf2, w->b_cf2, w->w_q, w->b_q, w->w_k,
                       w->b_k, w->w_v, w->b_v, w->dw_k, w->db_k, w->dw_v, w->db_v, w->w_o, w->b_o};
  for (int i = 0; i < 18; ++i) p[i] = v[i];
}
// Whether [p, p + bytes) overlaps any parameter the geometry's variant reads.
bool overlaps_weight(const void* p, size_t bytes, const edit_weights_t* w, const Geometry& g) {
  size_t ne[18];
  const void* wp[18];
  weight_elems(g, ne);
  weight_ptrs(w, wp);
  for (int i = 0; i < 18; ++i)
    if (overlap(p, bytes, wp[i], ne[i] * g.es)) return true;
  return false;
}

edit_status_t check_convfusion_weights(const edit_convfusion_weights_t* w) {
  if (!w) return fail(EDIT_ERR_ARG, "key ConvFusion weights struct is NULL");
  const void* p[] = {w->w_cf1, w->b_cf1, w->gn_gamma, w->gn_beta, w->w_cf2, w->b_cf2};
  const char* n[] = {"key.w_cf1", "key.b_cf1", "key.gn_gamma", "key.gn_beta", "key.w_cf2", "key.b_cf2"};
  for (int i = 0; i < 6; ++i) {
    edit_status_t st = check_ptr(p[i], n[i]);
    if (st != EDIT_OK) return st;
  }
  return EDIT_OK;
}

edit_status_t check_text_weights(const edit_text_weights_t* w) {
  if (!w) return fail(EDIT_ERR_ARG, "text weights struct is NULL");
  const void* p[] = {w->w_q, w->b_q, w->w_k, w->b_k, w->w_v, w->b_v, w->w_o, w->b_o};
  const char* n[] = {"txt.w_q", "txt.b_q", "txt.w_k", "txt.b_k", "txt.w_v", "txt.b_v", "txt.w_o", "txt.b_o"};
  for (int i = 0; i < 8; ++i) {
    edit_status_t st = check_ptr(p[i], n[i]);
    if (st != EDIT_OK) return st;
  }
  return EDIT_OK;
}

// The library carries gfx950 code only; confirm the current device is one.
edit_status_t check_device() {
  int dev = -1, count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0)
    return fail(EDIT_ERR_HIP, "no HIP device available (%s)", hipGetErrorString(e));
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(EDIT_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  static thread_local int checked_dev = -1;
  if (checked_dev == dev) return EDIT_OK;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(EDIT_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(EDIT_ERR_HIP, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
  checked_dev = dev;
  return EDIT_OK;
}

#define EDIT_LAUNCH(call)                                                                  \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) return fail(EDIT_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// Records events[i] on the stream when per-step timing was asked for.
// serial: every step on the caller's stream even without events (no second stream).
struct Marks {
  void* const* ev;
  hipStream_t s;
  bool serial = false;
  hipError_t mark(int i) const {
    return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess;
  }
};

// ConvFusion of x up to the restore: act = LeakyReLU(GN(Conv3x3(x))). The 1x1
// restore is folded into the Linear (w_lin, b_lin) that reads the restored
// stream x + act W_cf2^T + b_cf2: wcat = [w_lin | w_lin W_cf2],
// bcat = b_lin + w_lin b_cf2, for one GEMM over [x | act] (cat_linear).
// parts selects the 3x3 conv, the GroupNorm + LeakyReLU, and the fold (which
// reads weights only, so it may run on another stream).
enum { CF_CONV = 1, CF_NORM = 2, CF_FOLD = 4, CF_ALL = 7 };
template <typename T>
edit_status_t convfusion(const Geometry& g, const T* x, const void* w_cf1, const void* b_cf1, const void* gamma,
                         const void* beta, const void* w_cf2, const void* b_cf2, const void* w_lin,
                         const void* b_lin, T* xc, float* gn_part, float* gn_stat, float* gn_scale, float* gn_shift,
                         T* act, T* wcat, T* bcat, hipStream_t s, const Marks& mk, int parts = CF_ALL) {
  using namespace edit;
  // bf16: the restore fold goes with the conv's launch (see GemmArgs::fold)
  const bool fold_with_conv = (parts & CF_CONV) && (parts & CF_FOLD) && std::is_same<T, bf16>::value &&
                              g.C % 64 == 0 && g.Cr % 32 == 0;
  if (parts & CF_CONV) {
    // xc = Conv3x3(x) + b_cf1
    EDIT_LAUNCH(mk.mark(EDIT_STEP_CF_CONV3X3));
    GemmArgs<T> a{};
    a.M = g.M; a.N = g.Cr; a.K = 9 * g.C; a.A = x; a.lda = g.C; a.H = g.H; a.W = g.W; a.Cin = g.C;
    a.Bseg[0] = a.Bseg[1] = a.Bseg[2] = static_cast<const T*>(w_cf1);
    a.bias[0] = a.bias[1] = a.bias[2] = static_cast<const T*>(b_cf1);
    a.seg_rows = g.Cr; a.ldb = 9 * g.C; a.C = xc; a.ldc = g.Cr;
    if constexpr (std::is_same<T, bf16>::value) {
      if (fold_with_conv)
        a.fold = FoldArgs{static_cast<const bf16*>(w_lin), static_cast<const bf16*>(b_lin),
                          static_cast<const bf16*>(w_cf2), static_cast<const bf16*>(b_cf2), wcat, bcat, g.C, g.Cr};
    }
    if (gn_in_conv(g)) {
      a.gnp = gn_part; a.gn_rows = gn_tile_rows(g);
      EDIT_LAUNCH(launch_gemm<T>(a, A_CONV3, E_BIAS_GN, s));
    } else {
      EDIT_LAUNCH(launch_gemm<T>(a, A_CONV3, E_BIAS, s));
    }
  }
  if (parts & CF_NORM) {
    // GroupNorm statistics -> per-channel scale / shift; act = LeakyReLU(GN(xc))
    EDIT_LAUNCH(mk.mark(EDIT_STEP_GN_STATS));
    if (gn_in_conv(g)) {
      EDIT_LAUNCH(launch_groupnorm_finalize_channels<T>(gn_part, g.B, g.N, g.Cr, g.G, gn_tile_rows(g),
                                                        static_cast<const T*>(gamma), static_cast<const T*>(beta),
                                                        1e-5f, gn_stat, gn_scale, gn_shift, s));
    } else {
      EDIT_LAUNCH(launch_groupnorm_stats<T>(xc, g.B, g.N, g.Cr, g.G, static_cast<const T*>(gamma),
                                            static_cast<const T*>(beta), 1e-5f, gn_part, g.gn_chunks, gn_stat,
                                            gn_scale, gn_shift, s));
    }
    EDIT_LAUNCH(mk.mark(EDIT_STEP_CF_ACT));
    EDIT_LAUNCH(launch_groupnorm_apply<T>(xc, g.B, g.N, g.Cr, gn_scale, gn_shift, act, s));
  }
  if ((parts & CF_FOLD) && !fold_with_conv) {
    // the restore folded into the Linear's weights
    EDIT_LAUNCH(launch_restore_fold<T>(static_cast<const T*>(w_lin), static_cast<const T*>(b_lin),
                                       static_cast<const T*>(w_cf2), static_cast<const T*>(b_cf2), g.C, g.Cr, wcat,
                                       bcat, s));
  }
  return EDIT_OK;
}

// out = [x | act] wcat^T + bcat (+ ReLU), row stride ldc: the Linear of the
// restored stream x + ConvFusion(x) with the restore folded in.
template <typename T>
edit_status_t cat_linear(const Geometry& g, const T* x, const T* act, const T* wcat, const T* bcat, T* out, int ldc,
                         bool spread, hipStream_t s) {
  using namespace edit;
  GemmArgs<T> a{};
  a.spread = spread;
  a.M = g.M; a.N = g.C; a.K = g.C + g.Cr; a.A = x; a.lda = g.C; a.A2 = act; a.lda2 = g.Cr; a.K1 = g.C;
  a.Bseg[0] = a.Bseg[1] = a.Bseg[2] = wcat;
  a.bias[0] = a.bias[1] = a.bias[2] = bcat;
  a.seg_rows = g.C; a.ldb = g.C + g.Cr; a.C = out; a.ldc = ldc;
  EDIT_LAUNCH(launch_gemm<T>(a, A_CAT2, E_BIAS_RELU, s));
  return EDIT_OK;
}

// out[m][0..C) = epilogue(a[m] W^T + b) with row stride ldc.
template <typename T>
edit_status_t linear_cc(const Geometry& g, const T* a_in, const void* w, const void* b, T* out, int ldc, bool relu,
                        bool spread, hipStream_t s) {
  using namespace edit;
  GemmArgs<T> a{};
  a.spread = spread;
  a.M = g.M; a.N = g.C; a.K = g.C; a.A = a_in; a.lda = g.C;
  a.Bseg[0] = a.Bseg[1] = a.Bseg[2] = static_cast<const T*>(w);
  a.bias[0] = a.bias[1] = a.bias[2] = static_cast<const T*>(b);
  a.seg_rows = g.C; a.ldb = g.C; a.C = out; a.ldc = ldc;
  EDIT_LAUNCH(launch_gemm<T>(a, A_PLAIN, relu ? E_BIAS_RELU : E_BIAS, s));
  return EDIT_OK;
}

// A second stream per device for the key/value branch, and the events that
// fork it from the caller's stream and join it back. Created on first use,
// kept for the life of the process; g_side_mu serialises the enqueue of a
// fork .. join section, so that concurrent callers do not interleave records
// of the shared events.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[64];

edit_status_t side_stream(SideStream** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) return fail(EDIT_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    // Both streams run on this device: a device-scope release is enough. All
    // three objects are created before any is kept, so a failure leaves the
    // slot empty for the next call to retry.
    const unsigned fl = hipEventDisableTiming | hipEventReleaseToDevice;
    SideStream n;
    if ((e = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&n.fork, fl)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&n.join, fl)) != hipSuccess) {
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.s) (void)hipStreamDestroy(n.s);
      return fail(EDIT_ERR_HIP, "creating the key/value stream failed: %s", hipGetErrorString(e));
    }
    ss = n;
  }
  *out = &ss;
  return EDIT_OK;
}

// The device address of the static scratch (above), looked up once per device (hipGetSymbolAddress
// with that device current) and kept; host code passes only that address, never the array's name.
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

edit_status_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) return fail(EDIT_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(EDIT_ERR_HIP, "looking up the static scratch on device %d failed: %s", dev, hipGetErrorString(e));
    if (misaligned(p, 256)) return fail(EDIT_ERR_HIP, "the static scratch is not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EDIT_OK;
}

// The image stream up to the linear-attention output y (steps 1-8 of the
// layer; the ablation variants swap the query or the key/value processing).
// The query branch (steps 1-4) and the key/value branch (steps 5-7) only
// meet at step 8. Without per-step events the key/value branch runs on a
// second stream, so its kernels take the CUs the query branch leaves idle
// (the 3x3 conv has C/r / 96 x M / 256 tiles, 192 at 16384 tokens, fewer
// than the CUs); at bf16 that stream carries only the key/value GEMM and the
// depthwise + state pass follows the join on the caller's stream. With
// per-step events every step runs in order on the caller's stream. Each
// cross-stream event costs 5-10 us on MI355X, so there are only the fork
// and the join.
template <typename T>
edit_status_t run_image(const Geometry& g, const Layout& L, const edit_weights_t* w, const T* x, char* ws,
                        hipStream_t s, const Marks& mk, float* lin_den = nullptr,
                        const edit_convfusion_weights_t* kcf = nullptr, bool apply = true,
                        const std::function<edit_status_t(hipStream_t)>* side_work = nullptr) {
  using namespace edit;
  auto P = [&](size_t off) { return reinterpret_cast<T*>(ws + off); };
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const bool fork = mk.ev == nullptr && !mk.serial;

  // 1-4. queries: q = ReLU((x + ConvFusion(x)) W_q^T + b_q), or ReLU(x W_q^T + b_q).
  // parts: which ConvFusion parts to queue; q_proj waits for `folded` on qs when it is given.
  const bool cf = g.qmode == EDIT_QUERY_CONVFUSION;
  auto q_convfusion = [&](hipStream_t qs, int parts) -> edit_status_t {
    return convfusion<T>(g, x, w->w_cf1, w->b_cf1, w->gn_gamma, w->gn_beta, w->w_cf2, w->b_cf2, w->w_q, w->b_q,
                         P(L.xc), F(L.gn_part), F(L.gn_stat), F(L.gn_scale), F(L.gn_shift), P(L.cf_act),
                         P(L.q_fold_w), P(L.q_fold_b), qs, mk, parts);
  };
  auto q_proj = [&](hipStream_t qs) -> edit_status_t {
    EDIT_LAUNCH(mk.mark(EDIT_STEP_Q_PROJ));
    if (cf) return cat_linear<T>(g, x, P(L.cf_act), P(L.q_fold_w), P(L.q_fold_b), P(L.q), g.C, fork, qs);
    return linear_cc<T>(g, x, w->w_q, w->b_q, P(L.q), g.C, true, fork, qs);
  };
  // 6-7 at bf16 with compressed keys / values: the depthwise convs with the state partials in one pass, then
  // their merge into S, z
  auto dw_state = [&](hipStream_t ks) -> edit_status_t {
    if constexpr (std::is_same<T, bf16>::value) {
      EDIT_LAUNCH(launch_dwconv_kv_state<T>(P(L.kv0), g.B, g.H, g.W, g.C, g.heads, g.d,
                                            static_cast<const T*>(w->dw_k), static_cast<const T*>(w->db_k),
                                            static_cast<const T*>(w->dw_v), static_cast<const T*>(w->db_v),
                                            P(L.kc), P(L.vc), F(L.kv_part), g.kv_chunks, ks));
      EDIT_LAUNCH(mk.mark(EDIT_STEP_KV_STATE));
      EDIT_LAUNCH(launch_kv_state_finalize<T>(F(L.kv_part), g.B, g.heads, g.d, g.kv_chunks, F(L.S), F(L.z),
                                              P(L.st), F(L.zp), ks));
    }
    return EDIT_OK;
  };
  const bool fused_dw = std::is_same<T, bf16>::value && g.kvmode == EDIT_KV_COMPRESSED;
  // 5-7. keys, values and the per-head state S, z (with_dw false: the bf16 compressed path stops after the
  // key/value GEMM and leaves dw_state to the caller)
  auto kv_branch = [&](hipStream_t ks, bool with_dw) -> edit_status_t {
    edit_status_t st;
    EDIT_LAUNCH(mk.mark(EDIT_STEP_KV_PROJ));
    const T *kk, *vv;
    int ldkv;
    if (g.kvmode == EDIT_KV_COMPRESSED) {
      // 5. kv0 = [x W_k^T + b_k | x W_v^T + b_v]
      GemmArgs<T> a{};
      a.M = g.M; a.N = 2 * g.C; a.K = g.C; a.A = x; a.lda = g.C;
      a.Bseg[0] = static_cast<const T*>(w->w_k); a.Bseg[1] = a.Bseg[2] = static_cast<const T*>(w->w_v);
      a.bias[0] = static_cast<const T*>(w->b_k); a.bias[1] = a.bias[2] = static_cast<const T*>(w->b_v);
      a.seg_rows = g.C; a.ldb = g.C; a.C = P(L.kv0); a.ldc = 2 * g.C; a.spread = fork;
      EDIT_LAUNCH(launch_gemm<T>(a, A_PLAIN, E_BIAS, ks));
      EDIT_LAUNCH(mk.mark(EDIT_STEP_SC_DWCONV));
      // 6. compressed keys / values (bf16: with the state partials of step 7 in the same pass)
      if (fused_dw) return with_dw ? dw_state(ks) : EDIT_OK;
      EDIT_LAUNCH(launch_dwconv_s2<T>(P(L.kv0), g.B, g.H, g.W, g.C, static_cast<const T*>(w->dw_k),
                                      static_cast<const T*>(w->db_k), static_cast<const T*>(w->dw_v),
                                      static_cast<const T*>(w->db_v), P(L.kc), P(L.vc), ks));
      kk = P(L.kc); vv = P(L.vc); ldkv = g.C;
    } else {
      // Uncompressed keys and values side by side in kv0: K = ReLU(kin W_k^T + b_k), V = x W_v^T + b_v,
      // with kin = x or, for ConvFusion keys, x + ConvFusion_K(x) (its restore folded into W_k).
      if (g.kvmode == EDIT_KV_KEY_CONVFUSION) {
        st = convfusion<T>(g, x, kcf->w_cf1, kcf->b_cf1, kcf->gn_gamma, kcf->gn_beta, kcf->w_cf2, kcf->b_cf2,
                           w->w_k, w->b_k, P(L.xc_k), F(L.gn_part_k), F(L.gn_stat_k), F(L.gn_scale_k),
                           F(L.gn_shift_k), P(L.cf_act_k), P(L.k_fold_w), P(L.k_fold_b), ks, Marks{nullptr, ks});
        if (st != EDIT_OK) return st;
        st = cat_linear<T>(g, x, P(L.cf_act_k), P(L.k_fold_w), P(L.k_fold_b), P(L.kv0), 2 * g.C, fork, ks);
      } else {
        st = linear_cc<T>(g, x, w->w_k, w->b_k, P(L.kv0), 2 * g.C, true, fork, ks);
      }
      if (st != EDIT_OK) return st;
      if ((st = linear_cc<T>(g, x, w->w_v, w->b_v, P(L.kv0) + g.C, 2 * g.C, false, fork, ks)) != EDIT_OK) return st;
      EDIT_LAUNCH(mk.mark(EDIT_STEP_SC_DWCONV));
      kk = P(L.kv0); vv = P(L.kv0) + g.C; ldkv = 2 * g.C;
    }
    EDIT_LAUNCH(mk.mark(EDIT_STEP_KV_STATE));
    // 7. per-head state
    EDIT_LAUNCH(launch_kv_state<T>(kk, vv, ldkv, g.B, g.Nkv, g.heads, g.d, F(L.kv_part), g.kv_chunks, F(L.S),
                                   F(L.z), P(L.st), F(L.zp), ks));
    return EDIT_OK;
  };

  edit_status_t st;
  if (!fork) {
    if (cf && (st = q_convfusion(s, CF_ALL)) != EDIT_OK) return st;
    if ((st = q_proj(s)) != EDIT_OK) return st;
    if ((st = kv_branch(s, true)) != EDIT_OK) return st;
    if (side_work && (st = (*side_work)(s)) != EDIT_OK) return st;
  } else {
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* side;
    if ((st = side_stream(&side)) != EDIT_OK) return st;
    EDIT_LAUNCH(hipEventRecord(side->fork, s));
    EDIT_LAUNCH(hipStreamWaitEvent(side->s, side->fork, 0));
    // The query branch is the longer chain and is queued first, so its conv
    // takes its CUs before the key/value GEMM's blocks fill the rest. (Any
    // kernel queued ahead of the conv lets those blocks take every CU first.)
    st = cf ? q_convfusion(s, CF_ALL) : EDIT_OK;
    if (st == EDIT_OK) st = q_proj(s);
    // work of the caller's that depends on neither branch (the hybrid's text Q|K|V) goes first on the side
    // stream, beside the conv (measured at SD3.5M: queued after the key/value GEMM instead, that GEMM starts
    // ~60 us earlier but the text GEMM then runs beside the query GEMM, and the join comes ~20 us later)
    if (st == EDIT_OK && side_work) st = (*side_work)(side->s);
    // The bf16 compressed path joins after its key/value GEMM, which ends well before the query GEMM, so the
    // caller's stream finds the join already satisfied; the depthwise + state pass then follows the query GEMM
    // on the caller's stream with the whole chip (a join behind a still-running side stream leaves the chip
    // idle ~11 us on MI355X).
    if (st == EDIT_OK) st = kv_branch(side->s, !fused_dw);
    // Join even after a failed launch, so the caller's stream never runs ahead of queued side work.
    const hipError_t e1 = hipEventRecord(side->join, side->s);
    const hipError_t e2 = e1 == hipSuccess ? hipStreamWaitEvent(s, side->join, 0) : e1;
    if (st != EDIT_OK) return st;
    if (e2 != hipSuccess) return fail(EDIT_ERR_HIP, "joining the key/value stream failed: %s", hipGetErrorString(e2));
    if (fused_dw && (st = dw_state(s)) != EDIT_OK) return st;
  }
  EDIT_LAUNCH(mk.mark(EDIT_STEP_APPLY));
  // 8. y = q S / (q . z + eps) (the hybrid may form it inside its image-row softmax instead)
  if (apply)
    EDIT_LAUNCH(launch_linattn_apply<T>(P(L.q), g.C, P(L.st), F(L.zp), g.B, g.N, g.heads, g.d, g.eps, P(L.y), g.C,
                                        lin_den, s));
  return EDIT_OK;
}

template <typename T>
edit_status_t out_linear(int M, int C, const void* wo, const void* bo, const T* y, T* out, hipStream_t s,
                         float* part = nullptr, int S = 1) {
  using namespace edit;
  GemmArgs<T> a{};
  a.M = M; a.N = C; a.K = C; a.A = y; a.lda = C;
  a.Bseg[0] = a.Bseg[1] = a.Bseg[2] = static_cast<const T*>(wo);
  a.bias[0] = a.bias[1] = a.bias[2] = static_cast<const T*>(bo);
  a.seg_rows = C; a.ldb = C; a.C = out; a.ldc = C;
  if (part != nullptr && S > 1) {
    // S slices of K into fp32 partials [S][M][C], then their sum plus the bias
    a.Cf = part; a.split_stride = (long long)M * C; a.kchunk = C / S;
    EDIT_LAUNCH(launch_gemm<T>(a, A_PLAIN, E_F32, s));
    EDIT_LAUNCH(launch_splitk_reduce<T>(part, S, (long long)M * C, M, C, out, C, s, 0, 0, (T*)nullptr, 0,
                                        static_cast<const T*>(bo)));
    return EDIT_OK;
  }
  EDIT_LAUNCH(launch_gemm<T>(a, A_PLAIN, E_BIAS, s));
  return EDIT_OK;
}

template <typename T>
edit_status_t run_edit(const Geometry& g, const Layout& L, const edit_weights_t* w, const void* x, void* y,
                       void* ws, hipStream_t s, const Marks& mk, const edit_convfusion_weights_t* kcf = nullptr) {
  char* wsb = static_cast<char*>(ws);
  edit_status_t st = run_image<T>(g, L, w, static_cast<const T*>(x), wsb, s, mk, nullptr, kcf);
  if (st != EDIT_OK) return st;
  EDIT_LAUNCH(mk.mark(EDIT_STEP_OUT_PROJ));
  st = out_linear<T>(g.M, g.C, w->w_o, w->b_o, reinterpret_cast<const T*>(wsb + L.y), static_cast<T*>(y), s);
  if (st != EDIT_OK) return st;
  EDIT_LAUNCH(mk.mark(EDIT_NUM_STEPS));
  return EDIT_OK;
}

template <typename T>
edit_status_t run_hybrid(const Geometry& g, const Layout& L, const edit_weights_t* w,
                         const edit_text_weights_t* wt, const void* x_img, const void* x_txt, void* y_img,
                         void* y_txt, void* ws, hipStream_t s, bool exact_eta) {
  using namespace edit;
  char* wsb = static_cast<char*>(ws);
  auto P = [&](size_t off) { return reinterpret_cast<T*>(wsb + off); };
  float* lin_den = exact_eta && g.nt > 0 ? reinterpret_cast<float*>(wsb + L.lin_den) : nullptr;
  // bf16 with head dims up to 64 and the text keys in one split: the image rows' softmax kernel forms the
  // linear part itself from the head's state (the apply step and y_lin's round trip through memory drop out)
  const bool fuse = g.es == 2 && g.nt > 0 && edit::sdpa_staged_fuses_linear(g.d) &&
                    edit::sdpa_splits(g.N, g.nt, g.heads, g.B, g.d, true) == 1;
  const int C = g.C, MT = g.B * g.nt;
  // Text Q | K | V in one GEMM with three weight segments; it reads only x_txt, so it runs on the image
  // path's side stream beside the conv (the image path joins that stream before it returns).
  const std::function<edit_status_t(hipStream_t)> text_qkv = [&](hipStream_t ts) -> edit_status_t {
    GemmArgs<T> a{};
    a.M = MT; a.N = 3 * C; a.K = C; a.A = static_cast<const T*>(x_txt); a.lda = C;
    a.Bseg[0] = static_cast<const T*>(wt->w_q); a.Bseg[1] = static_cast<const T*>(wt->w_k);
    a.Bseg[2] = static_cast<const T*>(wt->w_v);
    a.bias[0] = static_cast<const T*>(wt->b_q); a.bias[1] = static_cast<const T*>(wt->b_k);
    a.bias[2] = static_cast<const T*>(wt->b_v);
    a.seg_rows = C; a.ldb = C; a.C = P(L.qkv_t); a.ldc = 3 * C;
    EDIT_LAUNCH(launch_gemm<T>(a, A_PLAIN, E_BIAS, ts));
    return EDIT_OK;
  };
  edit_status_t st = run_image<T>(g, L, w, static_cast<const T*>(x_img), wsb, s, Marks{nullptr, s},
                                  fuse ? nullptr : lin_den, nullptr, !fuse, g.nt > 0 ? &text_qkv : nullptr);
  if (st != EDIT_OK) return st;
  if (g.nt == 0) return out_linear<T>(g.M, g.C, w->w_o, w->b_o, P(L.y), static_cast<T*>(y_img), s);

  const T* qkv = P(L.qkv_t);
  const float eta = (float)((double)g.N / ((double)g.N + (double)g.nt));
  // Image rows: eta * y_lin + (1 - eta) * softmax(Q_I K_T^T / sqrt(d)) V_T, with eta the token ratio
  // or, exactly, (q.z + eps) / (q.z + eps + sum_t exp(s_t)) per row and head.
  SdpaArgs<T> sa{};
  sa.q = P(L.q); sa.ldq = C; sa.Nq = g.N;
  sa.k1 = qkv + C; sa.v1 = qkv + 2 * C; sa.ldkv1 = 3 * C; sa.N1 = g.nt;
  sa.k2 = nullptr; sa.v2 = nullptr; sa.ldkv2 = 0; sa.N2 = 0;
  sa.B = g.B; sa.heads = g.heads; sa.d = g.d;
  sa.out = P(L.y_img); sa.ldo = C;
  sa.blend_src = P(L.y); sa.ldbs = C; sa.alpha = eta; sa.beta = 1.0f - eta; sa.lin_den = lin_den;
  if (fuse) {
    // y_lin from the state in the kernel; the exact eta's q . z + eps is written to lin_den
    sa.blend_src = nullptr; sa.ldbs = 0;
    sa.lin_st = P(L.st); sa.lin_zp = reinterpret_cast<const float*>(wsb + L.zp); sa.lin_eps = g.eps;
    sa.exact_eta = exact_eta ? 1 : 0;
    sa.lin_den = nullptr; sa.lin_den_out = lin_den;
  }
  sa.splits = sdpa_splits(g.N, g.nt, g.heads, g.B, g.d, g.es == 2);
  sa.part = sa.splits > 1 ? reinterpret_cast<float*>(wsb + L.sdpa_part_img) : nullptr;
  // Text rows: softmax over [K'_I ; K_T] with values [V'_I ; V_T].
  SdpaArgs<T> ta{};
  ta.q = qkv; ta.ldq = 3 * C; ta.Nq = g.nt;
  ta.k1 = P(L.kc); ta.v1 = P(L.vc); ta.ldkv1 = C; ta.N1 = g.Nc;
  ta.k2 = qkv + C; ta.v2 = qkv + 2 * C; ta.ldkv2 = 3 * C; ta.N2 = g.nt;
  ta.B = g.B; ta.heads = g.heads; ta.d = g.d;
  ta.out = P(L.y_txt); ta.ldo = C;
  ta.blend_src = nullptr; ta.ldbs = 0; ta.alpha = 0.0f; ta.beta = 1.0f; ta.lin_den = nullptr;
  ta.splits = sdpa_splits(g.nt, g.Nc + g.nt, g.heads, g.B, g.d, g.es == 2);
  ta.part = ta.splits > 1 ? reinterpret_cast<float*>(wsb + L.sdpa_part_txt) : nullptr;
  // text rows first: their key splits are the longer blocks of work, started before the image tiles
  EDIT_LAUNCH(launch_sdpa_pair<T>(ta, sa, s));

  st = out_linear<T>(g.M, C, w->w_o, w->b_o, P(L.y_img), static_cast<T*>(y_img), s);
  if (st != EDIT_OK) return st;
  const int so = out_splits(MT, C, g.es);
  return out_linear<T>(MT, C, wt->w_o, wt->b_o, P(L.y_txt), static_cast<T*>(y_txt), s,
                       so > 1 ? reinterpret_cast<float*>(wsb + L.out_part_txt) : nullptr, so);
}

// ---------------------------------------------------------------------------
// Backward (the chain rule through the forward steps; see edit_attn_backward
// in the header). Scratch layout, byte offsets into the backward workspace.
// Tensors contracted over tokens (the weight gradients) are transposed to
// [channels][tokens] rows of Mp = M rounded up to 8 elements, so that the
// GEMM reads both operands K-contiguous; those products are cut into K slices
// (split-K) written as fp32 partials and added in slice order.
// ---------------------------------------------------------------------------
struct BwdLayout {
  size_t zeros, w_oT, wqT, wkvT, wflip, dy, g, cvec, dq_pre, dS, dz, st, zp, kvpart, dkv, dk0v0, dXq, dXkv;
  size_t dact, dxc, doutT, yT, xT, dqT, actT, dkvT, dxcT9, colsum, skpart, dWx, dWa, dbq32, dwpart, gnpart, m12;
  size_t total;
  int Mp, Crp;   // tokens rounded up to 8; C/r rounded up to 64 (the conv input gradient's channel stride)
};

struct SplitK {
  int S, kchunk;
};

// K slices for a [rows][cols] weight gradient over M tokens, slices a multiple of 64 tokens. The output tile is
// the one the GEMM will pick: bf16 128 x 192 (cols a multiple of 192) or 128 x 96 (of 96) on the DMA kernel, else
// 128 x 128. The slice count minimises an estimate of the time in 64-token K steps: rounds of 512 blocks (two per
// CU on 256 CUs) times the K steps of one slice, plus each slice's fp32 partial written and read back (~1 K step
// per million output elements). A count just past a whole round (540 units on 512 slots) would leave a second
// round of a few blocks running a whole slice on an almost idle chip.
SplitK splitk(int rows, int cols, int M, bool bf) {
  const int bn = bf && cols % 192 == 0 ? 192 : (bf && cols % 96 == 0 ? 96 : 128);
  const long tiles = ((long)(rows + 127) / 128) * ((cols + bn - 1) / bn);
  const double slice_cost = (double)rows * cols * 1e-6;
  long best_k = 64;
  double best = 1e300;
  for (long S = 1; S <= 32; ++S) {
    long kchunk = ((M + S - 1) / S + 63) / 64 * 64;
    if (kchunk < 64) kchunk = 64;
    const long se = (M + kchunk - 1) / kchunk;
    const long rounds = (tiles * se + 511) / 512;
    const double t = (double)rounds * (double)(kchunk / 64) + (se > 1 ? (double)se * slice_cost : 0.0);
    if (t < best) { best = t; best_k = kchunk; }
  }
  SplitK r;
  r.kchunk = (int)best_k;
  r.S = (int)((M + best_k - 1) / best_k);
  return r;
}

BwdLayout make_bwd_layout(const Geometry& g) {
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t M = g.M, Mc = (size_t)g.B * g.Nc, C = g.C, Cr = g.Cr, es = g.es, BH = (size_t)g.B * g.heads;
  L.Mp = (int)((M + 7) / 8 * 8);
  L.Crp = (int)((Cr + 63) / 64 * 64);
  const size_t Mp = L.Mp, Crp = L.Crp;
  L.zeros = take(2 * C * es);
  L.w_oT = take(C * C * es);
  L.wqT = take((C + Cr) * C * es);
  L.wkvT = take(C * 2 * C * es);
  L.wflip = take(C * 9 * Crp * es);
  L.dy = take(M * C * es);
  L.g = take(M * C * es);
  L.cvec = take(M * g.heads * 4);
  L.dq_pre = take(M * C * es);
  L.dXq = take(M * C * es);   // transposed together with dq_pre (one batched launch)
  L.dS = take(BH * g.d * g.d * 4);
  L.dz = take(BH * g.d * 4);
  L.st = take(BH * 2 * g.DP * g.DK * es);
  L.zp = take(BH * g.DK * 4);
  L.kvpart = take(BH * edit::kv_state_chunks(g.N) * (16 * g.DR) * (16 * g.DT) * 4);
  L.dkv = take(Mc * 2 * C * 4);   // fp32: its sums over tokens cancel (see kv_bwd_kernel)
  L.dk0v0 = take(M * 2 * C * es);
  L.dXkv = take(M * C * es);
  L.dact = take(M * Cr * es);
  L.dxc = take(M * Crp * es);
  L.doutT = take(C * Mp * es);
  L.yT = take(C * Mp * es);
  L.xT = take(C * Mp * es);
  L.dqT = take(2 * C * Mp * es);
  L.actT = take(Cr * Mp * es);
  L.dkvT = take(2 * C * Mp * es);
  L.dxcT9 = take(9 * Cr * Mp * es);
  // the transposes' per-64-token-tile channel sums, for the bias gradients
  L.colsum = take((2 * C > 9 * Cr ? 2 * C : 9 * Cr) * ((Mp + 63) / 64) * 4);
  size_t sk = 0;
  const int shapes[4][2] = {{g.C, g.C}, {2 * g.C, g.C}, {2 * g.C, g.Cr}, {9 * g.Cr, g.C}};
  for (auto& sh : shapes) {
    const SplitK k = splitk(sh[0], sh[1], L.Mp, g.es == 2);
    const size_t b = (size_t)k.S * sh[0] * sh[1] * 4;
    if (b > sk) sk = b;
  }
  L.skpart = take(sk);
  L.dWx = take(C * C * 4);
  L.dWa = take(C * Cr * 4);
  L.dbq32 = take(C * 4);
  L.dwpart = take((size_t)edit::dw_bwd_chunks(g.B, g.H, g.W) * 11 * 2 * C * 4);
  L.gnpart = take((size_t)g.B * edit::gn_bwd_chunks(g.N) * Cr * 2 * 4);
  L.m12 = take((size_t)g.B * g.G * 2 * 4);
  L.total = off;
  return L;
}

template <typename T>
edit_status_t run_backward(const Geometry& g, const Layout& F, const BwdLayout& L, const edit_weights_t* w,
                           const T* x, const T* dout, const char* fws, T* dx, const edit_grads_t* gr, char* ws,
                           hipStream_t s) {
  using namespace edit;
  auto P = [&](size_t off) { return reinterpret_cast<T*>(ws + off); };
  auto Q = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  auto FP = [&](size_t off) { return reinterpret_cast<const T*>(fws + off); };
  auto FF = [&](size_t off) { return reinterpret_cast<const float*>(fws + off); };
  auto W = [](const void* p) { return static_cast<const T*>(p); };
  auto G = [](void* p) { return static_cast<T*>(p); };
  const int M = g.M, C = g.C, Cr = g.Cr, Mp = L.Mp, Crp = L.Crp;
  const T* zeros = P(L.zeros);
  // bias gradients: the transposes of the output gradients also write per-tile channel sums (nrt tiles)
  float* cs = Q(L.colsum);
  const int nrt = (Mp + 63) / 64;

  // C[M'][N'] = A B^T (+ R), both operands K-contiguous.
  auto gemm = [&](int Mr, int Nr, int K, const T* A, int lda, const T* B, int ldb, T* out, int ldc,
                  const T* R = nullptr) -> edit_status_t {
    GemmArgs<T> a{};
    a.M = Mr; a.N = Nr; a.K = K; a.A = A; a.lda = lda;
    a.Bseg[0] = a.Bseg[1] = a.Bseg[2] = B;
    a.bias[0] = a.bias[1] = a.bias[2] = zeros;
    a.seg_rows = Nr; a.ldb = ldb; a.C = out; a.ldc = ldc; a.R = R; a.ldr = ldc;
    EDIT_LAUNCH(launch_gemm<T>(a, A_PLAIN, E_BIAS, s));
    return EDIT_OK;
  };
  // P[r][c] = sum_m At[r][m] Bt[c][m] over the tokens (transposed operands, row stride Mp, zero
  // padding past M) as split-K fp32 partials; wsum then adds the slices of rows [r0, r0 + n) into out
  // (rows in groups of rpg interleave in the output row, see launch_splitk_reduce).
  int wrows = 0, wcols = 0, wS = 0;
  auto wprod = [&](int rows, int cols, const T* At, const T* Bt) -> edit_status_t {
    const SplitK k = splitk(rows, cols, Mp, sizeof(T) == 2);
    GemmArgs<T> a{};
    a.M = rows; a.N = cols; a.K = Mp; a.A = At; a.lda = Mp;
    a.Bseg[0] = a.Bseg[1] = a.Bseg[2] = Bt;
    a.bias[0] = a.bias[1] = a.bias[2] = zeros;
    a.seg_rows = cols; a.ldb = Mp; a.ldc = cols;
    a.Cf = Q(L.skpart); a.split_stride = (long long)rows * cols; a.kchunk = k.kchunk;
    EDIT_LAUNCH(launch_gemm<T>(a, A_PLAIN, E_F32, s));
    wrows = rows; wcols = cols; wS = k.S;
    return EDIT_OK;
  };
  auto wsum = [&](int r0, int n, auto* out, int ldo, int rpg = 0, int gstride = 0) -> edit_status_t {
    EDIT_LAUNCH(launch_splitk_reduce(Q(L.skpart) + (size_t)r0 * wcols, wS, (long long)wrows * wcols, n, wcols, out,
                                     ldo, s, rpg, gstride));
    return EDIT_OK;
  };
  // rows 0 .. n1 - 1 of the product to out1, rows n1 .. n - 1 to out2 (one launch)
  auto wsum2 = [&](int n, int n1, T* out1, T* out2, int ldo) -> edit_status_t {
    EDIT_LAUNCH(launch_splitk_reduce(Q(L.skpart), wS, (long long)wrows * wcols, n, wcols, out1, ldo, s, 0, 0, out2,
                                     n1));
    return EDIT_OK;
  };
  auto wgrad = [&](int rows, int cols, const T* At, const T* Bt, auto* out, int ldo, int rpg = 0,
                   int gstride = 0) -> edit_status_t {
    edit_status_t e = wprod(rows, cols, At, Bt);
    return e != EDIT_OK ? e : wsum(0, rows, out, ldo, rpg, gstride);
  };
  edit_status_t st;

  // weights arranged as the GEMMs' B operands
  EDIT_LAUNCH(launch_zero<T>(P(L.zeros), 2L * C, s));
  EDIT_LAUNCH(launch_transpose<T>(W(w->w_o), C, C, C, P(L.w_oT), C, s));
  EDIT_LAUNCH(launch_transpose<T>(FP(F.q_fold_w), C, C + Cr, C + Cr, P(L.wqT), C, s));
  // W_k^T and W_v^T side by side, one launch (z = 1 reads W_v)
  EDIT_LAUNCH(launch_transpose<T>(W(w->w_k), C, C, C, P(L.wkvT), 2 * C, s, 0, 2, 0, (long)C, nullptr, W(w->w_v)));
  // the 3x3 conv's input gradient is a 3x3 conv of dxc with the taps mirrored and the channel roles
  // swapped: wflip[ci][t * Cr + co] = w_cf1[co][8 - t][ci], one transpose per tap
  // (channel slots Cr .. Crp - 1 of every tap zero)
  EDIT_LAUNCH(launch_transpose<T>(W(w->w_cf1) + 8 * C, Cr, C, 9 * C, P(L.wflip), 9 * Crp, s, Crp, 9, -(long)C, Crp));
  EDIT_LAUNCH(launch_transpose<T>(x, M, C, C, P(L.xT), Mp, s, Mp));

  // output Linear: dy = dout W_o, dW_o = dout^T y, db_o = sum dout
  if ((st = gemm(M, C, C, dout, C, P(L.w_oT), C, P(L.dy), C)) != EDIT_OK) return st;
  EDIT_LAUNCH(launch_transpose<T>(dout, M, C, C, P(L.doutT), Mp, s, Mp, 1, 0, 0, cs));
  EDIT_LAUNCH(launch_colsum_finalize<T>(cs, C, nrt, G(gr->b_o), s));
  EDIT_LAUNCH(launch_transpose<T>(FP(F.y), M, C, C, P(L.yT), Mp, s, Mp));
  if ((st = wgrad(C, C, P(L.doutT), P(L.yT), G(gr->w_o), C)) != EDIT_OK) return st;

  // linear attention: g, c, dq_pre; dS = sum q^T g and dz = sum c q (the state kernel with per-token weights c)
  EDIT_LAUNCH(launch_attn_bwd_q<T>(P(L.dy), FP(F.q), FF(F.S), FF(F.z), g.B, g.N, g.heads, g.d, g.eps, P(L.g),
                                   Q(L.cvec), P(L.dq_pre), s));
  // query Linear over [x | act] with the restore folded in (W' = [W_q | W_q W_cf2], b' = b_q + W_q b_cf2):
  // dXq = dq_pre W_q (the restored stream's gradient dxt, which also reaches x), dact = dq_pre W_q W_cf2
  if ((st = gemm(M, C, C, P(L.dq_pre), C, P(L.wqT), C, P(L.dXq), C)) != EDIT_OK) return st;
  if ((st = gemm(M, Cr, C, P(L.dq_pre), C, P(L.wqT) + (size_t)C * C, C, P(L.dact), Cr)) != EDIT_OK) return st;
  EDIT_LAUNCH(launch_kv_state<T>(FP(F.q), P(L.g), C, g.B, g.N, g.heads, g.d, Q(L.kvpart), kv_state_chunks(g.N),
                                 Q(L.dS), Q(L.dz), P(L.st), Q(L.zp), s, Q(L.cvec)));
  // dK' (through the keys' ReLU), dV'
  EDIT_LAUNCH(launch_kv_bwd<T>(FP(F.kc), FP(F.vc), Q(L.dS), Q(L.dz), g.B, g.Nc, g.heads, g.d, Q(L.dkv), s));

  // Spatial Compressor: depthwise convs, then the key / value Linears
  EDIT_LAUNCH(launch_dw_bwd_input<T>(Q(L.dkv), g.B, g.H, g.W, C, W(w->dw_k), W(w->dw_v), P(L.dk0v0), s));
  // ... and with them the key / value Linears' bias gradients (sums of dk0, dv0 over tokens)
  EDIT_LAUNCH(launch_dw_bwd_weight<T>(Q(L.dkv), FP(F.kv0), W(w->dw_k), W(w->dw_v), g.B, g.H, g.W, C, Q(L.dwpart),
                                      G(gr->dw_k), G(gr->db_k), G(gr->dw_v), G(gr->db_v), G(gr->b_k), G(gr->b_v), s));
  // dXkv = [dk0 | dv0] [W_k; W_v] + dXq (the two input-gradient terms so far)
  if ((st = gemm(M, C, 2 * C, P(L.dk0v0), 2 * C, P(L.wkvT), 2 * C, P(L.dXkv), C, P(L.dXq))) != EDIT_OK) return st;
  EDIT_LAUNCH(launch_transpose<T>(P(L.dk0v0), M, 2 * C, 2 * C, P(L.dkvT), Mp, s, Mp));
  // dW_k and dW_v: one product over [dk0 | dv0]^T
  if ((st = wprod(2 * C, C, P(L.dkvT), P(L.xT))) != EDIT_OK) return st;
  if ((st = wsum2(2 * C, C, G(gr->w_k), G(gr->w_v), C)) != EDIT_OK) return st;

  // the query Linear's weights: dW' = dq_pre^T [x | act], then
  // dW_q = dW'_x + dW'_act W_cf2^T + db_q b_cf2^T, db_q = sum dq_pre
  // and the restore's 1x1 conv: dxt = dq_pre W_q (= dXq), dW_cf2 = dxt^T act, db_cf2 = sum dxt.
  // dqT = [dq_pre | dxt]^T (one batched transpose over the two buffers).
  EDIT_LAUNCH(launch_transpose<T>(P(L.dq_pre), M, C, C, P(L.dqT), Mp, s, Mp, 2, (long)((L.dXq - L.dq_pre) / sizeof(T)),
                                  (long)C * Mp, cs));
  EDIT_LAUNCH(launch_colsum_finalize<T>(cs, 2 * C, nrt, G(gr->b_q), s, Q(L.dbq32), G(gr->b_cf2), C));
  EDIT_LAUNCH(launch_transpose<T>(FP(F.cf_act), M, Cr, Cr, P(L.actT), Mp, s, Mp));
  if ((st = wgrad(C, C, P(L.dqT), P(L.xT), Q(L.dWx), C)) != EDIT_OK) return st;
  if ((st = wprod(2 * C, Cr, P(L.dqT), P(L.actT))) != EDIT_OK) return st;   // [dW'_act | dW_cf2]
  // dW'_act (fp32, rows 0 .. C - 1) and dW_cf2 (rows C .. 2C - 1), one launch
  EDIT_LAUNCH(launch_splitk_reduce(Q(L.skpart), wS, (long long)wrows * wcols, 2 * C, wcols, Q(L.dWa), Cr, s, 0, 0,
                                   G(gr->w_cf2), C));
  EDIT_LAUNCH((launch_small_nt<T, T>(C, C, Cr, Q(L.dWa), Cr, W(w->w_cf2), Cr, Q(L.dWx), C, G(gr->w_q), C, s,
                                     Q(L.dbq32), W(w->b_cf2))));

  // LeakyReLU + GroupNorm, then the 3x3 conv: dx += conv(dxc, mirrored taps), dW_cf1 per tap
  EDIT_LAUNCH(launch_gn_bwd<T>(P(L.dact), FP(F.cf_act), FP(F.xc), FF(F.gn_stat), W(w->gn_gamma), g.B, g.N, Cr, g.G,
                               Q(L.gnpart), Q(L.m12), G(gr->gn_gamma), G(gr->gn_beta), P(L.dxc), Crp, s));
  {
    GemmArgs<T> a{};
    // dx = conv(dxc, mirrored taps) + dXkv; dxc's channels padded to Crp (zeros) for 64-wide K steps
    a.M = M; a.N = C; a.K = 9 * Crp; a.A = P(L.dxc); a.lda = Crp; a.H = g.H; a.W = g.W; a.Cin = Crp;
    a.Bseg[0] = a.Bseg[1] = a.Bseg[2] = P(L.wflip);
    a.bias[0] = a.bias[1] = a.bias[2] = zeros;
    a.seg_rows = C; a.ldb = 9 * Crp; a.C = dx; a.ldc = C; a.R = P(L.dXkv); a.ldr = C;
    EDIT_LAUNCH(launch_gemm<T>(a, A_CONV3, E_BIAS, s));
  }
  // dW_cf1[co][t][ci] = sum_m dxc[m + off_t][co] x[m][ci]: the nine shifted copies of dxc stacked as
  // [9 Cr][tokens], one product whose row t * Cr + co lands at w_cf1 + co * 9C + t * C
  EDIT_LAUNCH(launch_shift_transpose9<T>(P(L.dxc), g.B, g.H, g.W, Cr, Crp, P(L.dxcT9), Mp, s, cs));
  EDIT_LAUNCH(launch_colsum_finalize<T>(cs + (size_t)4 * Cr * nrt, Cr, nrt, G(gr->b_cf1), s));   // centre tap
  if ((st = wgrad(9 * Cr, C, P(L.dxcT9), P(L.xT), G(gr->w_cf1), 9 * C, Cr, C)) != EDIT_OK) return st;
  return EDIT_OK;
}

}  // namespace

extern "C" {

size_t edit_attn_workspace_size(const edit_shape_t* shape) {
  Geometry g;
  if (check_shape(shape, 0, &g) != EDIT_OK) return 0;
  return make_layout(g).total;
}

size_t mmedit_hybrid_workspace_size(const edit_shape_t* shape, int n_text) {
  Geometry g;
  if (check_shape(shape, n_text, &g) != EDIT_OK) return 0;
  return make_layout(g).total;
}

static void export_layout(const Layout& L, edit_ws_layout_t* out) {
  out->xc = L.xc; out->gn_stat = L.gn_stat; out->cf_act = L.cf_act; out->q_fold_w = L.q_fold_w;
  out->q_fold_b = L.q_fold_b; out->q = L.q; out->kv0 = L.kv0;
  out->kc = L.kc; out->vc = L.vc; out->S = L.S; out->z = L.z; out->y = L.y;
  out->qkv_t = L.qkv_t; out->y_img = L.y_img; out->y_txt = L.y_txt; out->lin_den = L.lin_den;
  out->xc_k = L.xc_k; out->gn_stat_k = L.gn_stat_k; out->cf_act_k = L.cf_act_k; out->k_fold_w = L.k_fold_w;
  out->k_fold_b = L.k_fold_b;
  out->total = L.total;
}

edit_status_t edit_attn_workspace_layout(const edit_shape_t* shape, int n_text, edit_ws_layout_t* out) {
  Geometry g;
  edit_status_t st = check_shape(shape, n_text, &g);
  if (st != EDIT_OK) return st;
  if (!out) return fail(EDIT_ERR_ARG, "layout is NULL");
  export_layout(make_layout(g), out);
  return EDIT_OK;
}

size_t edit_attn_variant_workspace_size(const edit_shape_t* shape, const edit_variant_t* variant) {
  Geometry g;
  if (check_shape(shape, 0, &g) != EDIT_OK || apply_variant(variant, &g) != EDIT_OK) return 0;
  return make_layout(g).total;
}

edit_status_t edit_attn_variant_workspace_layout(const edit_shape_t* shape, const edit_variant_t* variant,
                                                 edit_ws_layout_t* out) {
  Geometry g;
  edit_status_t st = check_shape(shape, 0, &g);
  if (st != EDIT_OK) return st;
  if ((st = apply_variant(variant, &g)) != EDIT_OK) return st;
  if (!out) return fail(EDIT_ERR_ARG, "layout is NULL");
  export_layout(make_layout(g), out);
  return EDIT_OK;
}

// workspace == nullptr with scratch_ws set: the static scratch (edit_attn_forward_noalloc), whose
// device address is looked up only once the arguments have passed every check.
static edit_status_t forward_impl(const edit_shape_t* shape, const edit_weights_t* w, const void* x, void* y,
                                  void* workspace, size_t ws_bytes, void* hip_stream, void* const* events,
                                  const edit_variant_t* variant = nullptr,
                                  const edit_convfusion_weights_t* kcf = nullptr, bool scratch_ws = false) {
  Geometry g;
  edit_status_t st = check_shape(shape, 0, &g);
  if (st != EDIT_OK) return st;
  if (variant && (st = apply_variant(variant, &g)) != EDIT_OK) return st;
  if ((st = check_weights(w, g)) != EDIT_OK) return st;
  if (g.kvmode == EDIT_KV_KEY_CONVFUSION && (st = check_convfusion_weights(kcf)) != EDIT_OK) return st;
  if ((st = check_ptr(x, "x")) != EDIT_OK) return st;
  if ((st = check_ptr(y, "y")) != EDIT_OK) return st;
  const Layout L = make_layout(g);
  const size_t act = (size_t)g.M * g.C * g.es;
  if (overlap(y, act, x, act)) return fail(EDIT_ERR_ARG, "y overlaps x");
  if (overlaps_weight(y, act, w, g)) return fail(EDIT_ERR_ARG, "y overlaps a weight");
  if (scratch_ws) {
    if (L.total > EDIT_NOALLOC_SCRATCH_BYTES)
      return fail(EDIT_ERR_WORKSPACE, "this shape needs %zu bytes of scratch; the static scratch holds %zu", L.total,
                  (size_t)EDIT_NOALLOC_SCRATCH_BYTES);
    if ((st = check_device()) != EDIT_OK) return st;
    if ((st = static_scratch(&workspace)) != EDIT_OK) return st;
    ws_bytes = EDIT_NOALLOC_SCRATCH_BYTES;
  } else {
    if (!workspace) return fail(EDIT_ERR_ARG, "workspace is NULL");
    if (misaligned(workspace, 256)) return fail(EDIT_ERR_ARG, "workspace is not 256-byte aligned");
    if (ws_bytes < L.total)
      return fail(EDIT_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
    if ((st = check_device()) != EDIT_OK) return st;
  }
  if (overlap(y, act, workspace, ws_bytes)) return fail(EDIT_ERR_ARG, "y overlaps the workspace");
  if (overlap(x, act, workspace, ws_bytes)) return fail(EDIT_ERR_ARG, "x overlaps the workspace");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  Marks mk{events, s};
  mk.serial = scratch_ws;
  return g.dtype == EDIT_BF16 ? run_edit<bf16>(g, L, w, x, y, workspace, s, mk, kcf)
                              : run_edit<float>(g, L, w, x, y, workspace, s, mk, kcf);
}

edit_status_t edit_attn_forward(const edit_shape_t* shape, const edit_weights_t* w, const void* x, void* y,
                                void* workspace, size_t ws_bytes, void* hip_stream) {
  return forward_impl(shape, w, x, y, workspace, ws_bytes, hip_stream, nullptr);
}

edit_status_t edit_attn_forward_noalloc(const edit_shape_t* shape, const edit_weights_t* w, const void* x, void* y,
                                        void* hip_stream) {
  return forward_impl(shape, w, x, y, nullptr, 0, hip_stream, nullptr, nullptr, nullptr, true);
}

edit_status_t edit_attn_variant_forward(const edit_shape_t* shape, const edit_variant_t* variant,
                                        const edit_weights_t* w, const edit_convfusion_weights_t* key_cf,
                                        const void* x, void* y, void* workspace, size_t ws_bytes,
                                        void* hip_stream) {
  if (!variant) return fail(EDIT_ERR_ARG, "variant is NULL");
  return forward_impl(shape, w, x, y, workspace, ws_bytes, hip_stream, nullptr, variant, key_cf);
}

edit_status_t edit_attn_forward_timed(const edit_shape_t* shape, const edit_weights_t* w, const void* x, void* y,
                                      void* workspace, size_t ws_bytes, void* hip_stream, void* const* events) {
  if (!events) return fail(EDIT_ERR_ARG, "events is NULL");
  for (int i = 0; i <= EDIT_NUM_STEPS; ++i)
    if (!events[i]) return fail(EDIT_ERR_ARG, "events[%d] is NULL", i);
  return forward_impl(shape, w, x, y, workspace, ws_bytes, hip_stream, events);
}

size_t edit_attn_backward_workspace_size(const edit_shape_t* shape) {
  Geometry g;
  if (check_shape(shape, 0, &g) != EDIT_OK) return 0;
  return make_bwd_layout(g).total;
}

edit_status_t edit_attn_backward_workspace_layout(const edit_shape_t* shape, edit_bwd_layout_t* out) {
  Geometry g;
  edit_status_t st = check_shape(shape, 0, &g);
  if (st != EDIT_OK) return st;
  if (!out) return fail(EDIT_ERR_ARG, "layout is NULL");
  const BwdLayout L = make_bwd_layout(g);
  out->dy = L.dy; out->dq_pre = L.dq_pre; out->dS = L.dS; out->dz = L.dz; out->dkv = L.dkv;
  out->dk0v0 = L.dk0v0; out->dxq = L.dXq; out->dxkv = L.dXkv; out->dact = L.dact; out->dxc = L.dxc;
  out->dxc_ld = (size_t)L.Crp;
  out->total = L.total;
  return EDIT_OK;
}

edit_status_t edit_attn_backward(const edit_shape_t* shape, const edit_weights_t* w, const void* x, const void* dy,
                                 const void* fwd_workspace, size_t fwd_ws_bytes, void* dx, const edit_grads_t* grads,
                                 void* workspace, size_t ws_bytes, void* hip_stream) {
  Geometry g;
  edit_status_t st = check_shape(shape, 0, &g);
  if (st != EDIT_OK) return st;
  if ((st = check_weights(w, g)) != EDIT_OK) return st;
  if ((st = check_ptr(x, "x")) != EDIT_OK) return st;
  if ((st = check_ptr(dy, "dy")) != EDIT_OK) return st;
  if ((st = check_ptr(dx, "dx")) != EDIT_OK) return st;
  if (!grads) return fail(EDIT_ERR_ARG, "grads struct is NULL");
  {
    const void* p[] = {grads->w_cf1, grads->b_cf1, grads->gn_gamma, grads->gn_beta, grads->w_cf2, grads->b_cf2,
                       grads->w_q, grads->b_q, grads->w_k, grads->b_k, grads->w_v, grads->b_v,
                       grads->dw_k, grads->db_k, grads->dw_v, grads->db_v, grads->w_o, grads->b_o};
    const char* n[] = {"grads.w_cf1", "grads.b_cf1", "grads.gn_gamma", "grads.gn_beta", "grads.w_cf2",
                       "grads.b_cf2", "grads.w_q", "grads.b_q", "grads.w_k", "grads.b_k", "grads.w_v", "grads.b_v",
                       "grads.dw_k", "grads.db_k", "grads.dw_v", "grads.db_v", "grads.w_o", "grads.b_o"};
    for (int i = 0; i < 18; ++i)
      if ((st = check_ptr(p[i], n[i])) != EDIT_OK) return st;
    // Every gradient is an output: it may overlap no input (x, dy, a weight), no other output
    // (dx, another gradient) and neither workspace. Sizes in edit_weights_t / edit_grads_t order.
    size_t ne[18];
    weight_elems(g, ne);
    const size_t act = (size_t)g.M * g.C * g.es;
    for (int i = 0; i < 18; ++i) {
      const size_t bi = ne[i] * g.es;
      if (overlap(p[i], bi, x, act) || overlap(p[i], bi, dy, act) || overlap(p[i], bi, dx, act))
        return fail(EDIT_ERR_ARG, "%s overlaps x, dy or dx", n[i]);
      if (overlap(p[i], bi, workspace, ws_bytes) || overlap(p[i], bi, fwd_workspace, fwd_ws_bytes))
        return fail(EDIT_ERR_ARG, "%s overlaps a workspace", n[i]);
      if (overlaps_weight(p[i], bi, w, g)) return fail(EDIT_ERR_ARG, "%s overlaps a weight", n[i]);
      for (int j = 0; j < 18; ++j)
        if (j != i && overlap(p[i], bi, p[j], ne[j] * g.es))
          return fail(EDIT_ERR_ARG, "%s overlaps another gradient", n[i]);
    }
    if (overlaps_weight(dx, act, w, g)) return fail(EDIT_ERR_ARG, "dx overlaps a weight");
  }
  if (!fwd_workspace) return fail(EDIT_ERR_ARG, "forward workspace is NULL");
  if (misaligned(fwd_workspace, 256)) return fail(EDIT_ERR_ARG, "forward workspace is not 256-byte aligned");
  const Layout F = make_layout(g);
  if (fwd_ws_bytes < F.total)
    return fail(EDIT_ERR_WORKSPACE, "forward workspace has %zu bytes, needs %zu", fwd_ws_bytes, F.total);
  if (!workspace) return fail(EDIT_ERR_ARG, "workspace is NULL");
  if (misaligned(workspace, 256)) return fail(EDIT_ERR_ARG, "workspace is not 256-byte aligned");
  const BwdLayout L = make_bwd_layout(g);
  if (ws_bytes < L.total) return fail(EDIT_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  const size_t act = (size_t)g.M * g.C * g.es;
  if (overlap(dx, act, x, act) || overlap(dx, act, dy, act)) return fail(EDIT_ERR_ARG, "dx overlaps x or dy");
  if (overlap(dx, act, workspace, ws_bytes) || overlap(dx, act, fwd_workspace, fwd_ws_bytes))
    return fail(EDIT_ERR_ARG, "dx overlaps a workspace");
  if (overlap(workspace, ws_bytes, fwd_workspace, fwd_ws_bytes))
    return fail(EDIT_ERR_ARG, "the two workspaces overlap");
  if ((st = check_device()) != EDIT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const char* fws = static_cast<const char*>(fwd_workspace);
  char* wsb = static_cast<char*>(workspace);
  return g.dtype == EDIT_BF16
             ? run_backward<bf16>(g, F, L, w, static_cast<const bf16*>(x), static_cast<const bf16*>(dy), fws,
                                  static_cast<bf16*>(dx), grads, wsb, s)
             : run_backward<float>(g, F, L, w, static_cast<const float*>(x), static_cast<const float*>(dy), fws,
                                   static_cast<float*>(dx), grads, wsb, s);
}

static edit_status_t hybrid_impl(const edit_shape_t* shape, int n_text, const edit_weights_t* img,
                                 const edit_text_weights_t* txt, const void* x_img, const void* x_txt,
                                 void* y_img, void* y_txt, void* workspace, size_t ws_bytes, void* hip_stream,
                                 bool exact_eta) {
  Geometry g;
  edit_status_t st = check_shape(shape, n_text, &g);
  if (st != EDIT_OK) return st;
  if ((st = check_weights(img, g)) != EDIT_OK) return st;
  if ((st = check_ptr(x_img, "x_img")) != EDIT_OK) return st;
  if ((st = check_ptr(y_img, "y_img")) != EDIT_OK) return st;
  if (n_text > 0) {
    if ((st = check_text_weights(txt)) != EDIT_OK) return st;
    if ((st = check_ptr(x_txt, "x_txt")) != EDIT_OK) return st;
    if ((st = check_ptr(y_txt, "y_txt")) != EDIT_OK) return st;
  }
  if (!workspace) return fail(EDIT_ERR_ARG, "workspace is NULL");
  if (misaligned(workspace, 256)) return fail(EDIT_ERR_ARG, "workspace is not 256-byte aligned");
  const Layout L = make_layout(g);
  if (ws_bytes < L.total)
    return fail(EDIT_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  const size_t ai = (size_t)g.M * g.C * g.es, at = (size_t)g.B * n_text * g.C * g.es;
  const void* ins[] = {x_img, x_txt, workspace};
  const size_t ins_n[] = {ai, n_text > 0 ? at : 0, ws_bytes};
  for (int i = 0; i < 3; ++i) {
    if (overlap(y_img, ai, ins[i], ins_n[i])) return fail(EDIT_ERR_ARG, "y_img overlaps an input or the workspace");
    if (n_text > 0 && overlap(y_txt, at, ins[i], ins_n[i]))
      return fail(EDIT_ERR_ARG, "y_txt overlaps an input or the workspace");
  }
  if (n_text > 0 && overlap(y_img, ai, y_txt, at)) return fail(EDIT_ERR_ARG, "y_img overlaps y_txt");
  if (overlaps_weight(y_img, ai, img, g) || (n_text > 0 && overlaps_weight(y_txt, at, img, g)))
    return fail(EDIT_ERR_ARG, "an output overlaps an image-stream weight");
  if (overlap(x_img, ai, workspace, ws_bytes) || (n_text > 0 && overlap(x_txt, at, workspace, ws_bytes)))
    return fail(EDIT_ERR_ARG, "an input overlaps the workspace");
  if ((st = check_device()) != EDIT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  return g.dtype == EDIT_BF16
             ? run_hybrid<bf16>(g, L, img, txt, x_img, x_txt, y_img, y_txt, workspace, s, exact_eta)
             : run_hybrid<float>(g, L, img, txt, x_img, x_txt, y_img, y_txt, workspace, s, exact_eta);
}

edit_status_t mmedit_hybrid_forward(const edit_shape_t* shape, int n_text, const edit_weights_t* img,
                                    const edit_text_weights_t* txt, const void* x_img, const void* x_txt,
                                    void* y_img, void* y_txt, void* workspace, size_t ws_bytes,
                                    void* hip_stream) {
  return hybrid_impl(shape, n_text, img, txt, x_img, x_txt, y_img, y_txt, workspace, ws_bytes, hip_stream, false);
}

edit_status_t mmedit_hybrid_exact_forward(const edit_shape_t* shape, int n_text, const edit_weights_t* img,
                                          const edit_text_weights_t* txt, const void* x_img, const void* x_txt,
                                          void* y_img, void* y_txt, void* workspace, size_t ws_bytes,
                                          void* hip_stream) {
  return hybrid_impl(shape, n_text, img, txt, x_img, x_txt, y_img, y_txt, workspace, ws_bytes, hip_stream, true);
}

const char* edit_status_string(edit_status_t status) {
  switch (status) {
    case EDIT_OK: return "EDIT_OK";
    case EDIT_ERR_ARG: return "EDIT_ERR_ARG: invalid argument";
    case EDIT_ERR_UNSUPPORTED: return "EDIT_ERR_UNSUPPORTED: outside the kernels' limits";
    case EDIT_ERR_WORKSPACE: return "EDIT_ERR_WORKSPACE: workspace too small";
    case EDIT_ERR_HIP: return "EDIT_ERR_HIP: HIP runtime error";
  }
  return "unknown status";
}

const char* edit_last_error(void) { return g_err; }

}  // extern "C"
