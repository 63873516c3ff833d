/*
 * edit_attn.h -- C ABI of the MI355X (gfx950) EDiT linear compressed
 * attention layer forward and its MM-EDiT hybrid.
 *
 * The operation is defined on the page "EDiT: Efficient Diffusion
 * Transformers with Linear Compressed Attention" (ICCV 2025 paper notes,
 * arXiv 2503.16726):
 *   - section "ConvFusion": Q = ReLU(Linear(X + Conv1x1(LeakyReLU(GN(Conv3x3(X)))))),
 *     the token sequence laid out as an H x W grid before the convolutions;
 *   - section "Spatial Compressor": K = ReLU(Conv(Linear(X))), V = Conv(Linear(X)),
 *     the conv being 3x3 depthwise with stride 2 (four times fewer tokens);
 *   - section "Linear-attention formula": y_i = Q_i (sum_j K_j^T V_j) / (Q_i sum_j K_j);
 *   - section "MM-EDiT": the hybrid matrix that keeps linear attention for
 *     image-image pairs and softmax attention for pairs involving text,
 *     mixed by eta = N_I / (N_I + N_T).
 * The output projection that follows the attention is not written on the
 * page; it is a plain Linear C -> C with bias.
 *
 * Conventions shared by every entry point
 *   Layout   x, y: [B][H*W][C], token n = row * W + col, channels innermost.
 *            x_txt, y_txt: [B][n_text][C]. Heads split the channels
 *            contiguously: channel c belongs to head c / head_dim.
 *            Linear weights are [out][in] row-major (y = x W^T + b).
 *            w_cf1 is [C/r][3][3][C] (input channels innermost), w_cf2 is
 *            [C][C/r], dw_k / dw_v are [3][3][C]; every bias is [out].
 *   Dtype    every tensor, weights and biases included, has the shape's
 *            dtype. EDIT_BF16 keeps bf16 storage with fp32 accumulation
 *            (GroupNorm statistics, the K^T V state, softmax and every
 *            accumulator are fp32); EDIT_F32 is fp32 throughout.
 *   Memory   every pointer is a device pointer owned by the caller; the
 *            library allocates no memory and keeps no data between calls
 *            (on first use on a device it creates one more stream and two
 *            events there, kept for the life of the process).
 *            Tensor pointers must be 16-byte aligned, the workspace
 *            256-byte aligned. Outputs must not overlap inputs or the
 *            workspace.
 *   Stream   work is enqueued on hip_stream (a hipStream_t passed as
 *            void*; NULL = the default stream), which must belong to the
 *            current HIP device, and the call returns without waiting. The
 *            forwards fork part of their work onto the library's second
 *            stream of that device and join it back to hip_stream before
 *            returning. Errors of the asynchronous work surface at the
 *            caller's next synchronisation.
 *   Errors   arguments are checked before anything is enqueued; on any
 *            error nothing is launched and a status other than EDIT_OK is
 *            returned. edit_last_error() gives the detail (thread-local).
 *            No entry point aborts or throws.
 *   Fixed    GroupNorm eps 1e-5, LeakyReLU slope 0.01, softmax scale
 *            1/sqrt(head_dim); eps of the linear branch comes with the shape.
 *   Results  are bit-for-bit reproducible for identical inputs and shape
 *            (no atomics in any reduction).
 */
#ifndef EDIT_ATTN_H
#define EDIT_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { EDIT_F32 = 0, EDIT_BF16 = 1 } edit_dtype_t;

typedef enum {
  EDIT_OK = 0,
  EDIT_ERR_ARG = 1,          /* invalid argument: bad size, null / misaligned / overlapping pointer */
  EDIT_ERR_UNSUPPORTED = 2,  /* valid, but outside the kernels' limits (see edit_shape_t) */
  EDIT_ERR_WORKSPACE = 3,    /* workspace smaller than the *_workspace_size query */
  EDIT_ERR_HIP = 4           /* no usable device, or a launch failed */
} edit_status_t;

/* Problem statement of one layer call.
 *   B          batch
 *   H, W       token grid (N = H*W image tokens)
 *   C          channels, = heads * head_dim
 *   reduction  ConvFusion channel reduction r (the 3x3 conv maps C -> C/r)
 *   gn_groups  GroupNorm groups over the C/r compressed channels
 *   eps        added to the linear-attention denominator Q_i . z (>= 0)
 * Kernel limits (EDIT_ERR_UNSUPPORTED otherwise): C, C/r and head_dim are
 * multiples of 8; head_dim <= 128. */
typedef struct {
  int B, H, W, C, heads, head_dim, reduction, gn_groups;
  float eps;
  edit_dtype_t dtype;
} edit_shape_t;

/* Parameters of the image stream (EDiT layer). */
typedef struct {
  const void *w_cf1, *b_cf1;       /* ConvFusion 3x3, C -> C/r            */
  const void *gn_gamma, *gn_beta;  /* GroupNorm affine, [C/r]             */
  const void *w_cf2, *b_cf2;       /* ConvFusion 1x1, C/r -> C            */
  const void *w_q, *b_q;           /* query Linear (inside ConvFusion)    */
  const void *w_k, *b_k;           /* key Linear (Spatial Compressor)     */
  const void *w_v, *b_v;           /* value Linear (Spatial Compressor)   */
  const void *dw_k, *db_k;         /* key depthwise 3x3 stride 2          */
  const void *dw_v, *db_v;         /* value depthwise 3x3 stride 2        */
  const void *w_o, *b_o;           /* output Linear                       */
} edit_weights_t;

/* Parameters of the text stream of the hybrid: its own Q/K/V/O Linears. */
typedef struct {
  const void *w_q, *b_q, *w_k, *b_k, *w_v, *b_v, *w_o, *b_o;
} edit_text_weights_t;

/* Bytes of workspace edit_attn_forward needs for this shape; 0 if the shape
 * is invalid (edit_last_error() says why). */
size_t edit_attn_workspace_size(const edit_shape_t* shape);

/* EDiT layer forward: y = Out(LinearAttention(Q_CF(x), K_SC(x), V_SC(x))).
 * x [B][H*W][C] in, y [B][H*W][C] out, workspace of at least
 * edit_attn_workspace_size(shape) bytes. */
edit_status_t edit_attn_forward(const edit_shape_t* shape, const edit_weights_t* w,
                                const void* x, void* y,
                                void* workspace, size_t ws_bytes, void* hip_stream);

/* Bytes of the static scratch edit_attn_forward_noalloc works in (256 MiB: the
 * workspace of up to about 22 000 tokens at C = 1152 in bf16, e.g. the
 * 128 x 128 grid). */
#define EDIT_NOALLOC_SCRATCH_BYTES (256u << 20)

/* edit_attn_forward for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument, and the call allocates nothing. Its
 * intermediates live in a static array of EDIT_NOALLOC_SCRATCH_BYTES bytes in
 * the library's code object, one per device, held from the first such call
 * on that device until the process ends (its address is looked up on that
 * first call, with the device current). Shapes whose workspace
 * (edit_attn_workspace_size) exceeds the array return EDIT_ERR_WORKSPACE
 * before anything is launched. Every step runs in order on hip_stream (no
 * second stream, no events); the result equals edit_attn_forward's bit for
 * bit. All calls on one device share the array and its contents after the
 * last call: calls that overlap in time on one device race, so the caller
 * serialises them (e.g. one stream per device). No part of the array needs
 * to start at zero. Other arguments, checks and errors as edit_attn_forward. */
edit_status_t edit_attn_forward_noalloc(const edit_shape_t* shape, const edit_weights_t* w,
                                        const void* x, void* y, void* hip_stream);

/* Bytes of workspace mmedit_hybrid_forward needs; 0 if invalid. */
size_t mmedit_hybrid_workspace_size(const edit_shape_t* shape, int n_text);

/* MM-EDiT hybrid forward.
 *   image rows: eta * LinearAttention(Q_I, K'_I, V'_I) + (1 - eta) * softmax(Q_I K_T^T / sqrt(d)) V_T
 *   text rows:  softmax([Q_T K'_I^T, Q_T K_T^T] / sqrt(d)) [V'_I ; V_T]
 *   eta = H*W / (H*W + n_text); then the image and the text output Linears.
 * Q_I, K'_I, V'_I are the EDiT features of x_img; Q_T, K_T, V_T the text
 * Linears of x_txt. n_text = 0 is legal: x_txt, y_txt, txt may then be NULL
 * and y_img equals edit_attn_forward's y bit for bit. */
edit_status_t mmedit_hybrid_forward(const edit_shape_t* shape, int n_text,
                                    const edit_weights_t* img, const edit_text_weights_t* txt,
                                    const void* x_img, const void* x_txt,
                                    void* y_img, void* y_txt,
                                    void* workspace, size_t ws_bytes, void* hip_stream);

/* MM-EDiT hybrid forward with eta computed exactly per image row and head
 * instead of the token ratio: the notes' hybrid matrix weights the linear
 * block by eta^Lin and the image->text softmax block by 1 - eta^Lin, and
 * approximate eta^Lin by N_I / (N_I + N_T) to avoid a custom kernel ("EDiT"
 * notes, section "MM-EDiT", the hybrid matrix and the remark under it).
 * Computed exactly, both blocks share one normaliser:
 *   image row i: (q_i S + sum_t exp(s_it) V_t) / (q_i . z + eps + sum_t exp(s_it)),
 *   s_it = q_i . K_t / sqrt(d),
 * i.e. eta_i = (q_i . z + eps) / (q_i . z + eps + sum_t exp(s_it)). Text rows
 * and everything else as mmedit_hybrid_forward; same arguments, layout and
 * workspace size (mmedit_hybrid_workspace_size). exp(s) is taken in fp32:
 * scores above ~88 (never reached by unit-scale features) overflow to the
 * softmax block alone. n_text = 0 gives edit_attn_forward's y bit for bit. */
edit_status_t mmedit_hybrid_exact_forward(const edit_shape_t* shape, int n_text,
                                          const edit_weights_t* img, const edit_text_weights_t* txt,
                                          const void* x_img, const void* x_txt,
                                          void* y_img, void* y_txt,
                                          void* workspace, size_t ws_bytes, void* hip_stream);

/* Where each intermediate of the last forward with this shape lives in the
 * workspace (byte offsets; 0 size = not produced for this call). The layout
 * is a pure function of (shape, n_text). Intermediates, with their dtype T
 * (the shape's dtype) or f32:
 *   xc      [B][N][C/r] T      ConvFusion 3x3 output
 *   gn_stat [B][G][2]   f32    GroupNorm mean and 1/sqrt(var + 1e-5)
 *   cf_act  [B][N][C/r] T      LeakyReLU(GN(xc)), the input of the 1x1 restore
 *   q_fold_w [C][C+C/r] T      [W_q | W_q W_cf2]: the 1x1 restore folded into the query
 *   q_fold_b [C]        T      b_q + W_q b_cf2   Linear, so q = ReLU([X | cf_act] q_fold_w^T + q_fold_b)
 *                              equals ReLU(Linear_Q(X + Conv1x1(cf_act))); the restored
 *                              stream itself is never stored
 *   q       [B][N][C]   T      ConvFusion queries (after ReLU)
 *   kv0     [B][N][2C]  T      key Linear | value Linear, side by side per token
 *   kc, vc  [B][N'][C]  T      compressed keys (ReLU'd) and values, N' = ceil(H/2)*ceil(W/2)
 *   S       [B][h][d][d] f32   sum_j K'_j^T V'_j per head
 *   z       [B][h][d]   f32    sum_j K'_j per head
 *   y       [B][N][C]   T      linear-attention output (hybrid: before blending)
 *   qkv_t   [B][N_T][3C] T     text Q | K | V (hybrid only)
 *   y_img   [B][N][C]   T      blended image rows (hybrid with text only)
 *   y_txt   [B][N_T][C] T      text rows before the text output Linear (hybrid only)
 *   lin_den [B][N][h]   f32    q . z + eps per token and head (exact-eta hybrid only)
 *   xc_k, gn_stat_k, cf_act_k, k_fold_w, k_fold_b
 *                              the key branch's ConvFusion, its restore folded into
 *                              W_k (EDIT_KV_KEY_CONVFUSION only)
 * For the ablation variants (edit_attn_variant_forward): q holds the variant's
 * queries; with uncompressed keys kv0 holds ReLU(key Linear) | value Linear
 * and the sums S, z run over all N tokens; kc, vc (and xc, gn_stat, cf_act,
 * q_fold_w, q_fold_b with a plain query) are not produced. */
typedef struct {
  size_t xc, gn_stat, cf_act, q_fold_w, q_fold_b, q, kv0, kc, vc, S, z, y, qkv_t, y_img, y_txt, lin_den;
  size_t xc_k, gn_stat_k, cf_act_k, k_fold_w, k_fold_b;
  size_t total;
} edit_ws_layout_t;

edit_status_t edit_attn_workspace_layout(const edit_shape_t* shape, int n_text,
                                         edit_ws_layout_t* layout);

/* Ablation variants of the query and key/value processing ("EDiT" notes,
 * section "Ablation: Query/Key/Value processing": the table of rows
 * (Q, K, V) = (CF, SC, SC), (CF, CF, -), (-, SC, SC), (CF, -, -)):
 *   query EDIT_QUERY_CONVFUSION  Q = ReLU(Linear_Q(X + ConvFusion(X)))   (CF)
 *         EDIT_QUERY_LINEAR      Q = ReLU(Linear_Q(X))                   (-)
 *   kv    EDIT_KV_COMPRESSED     K' = ReLU(DW(Linear_K X)), V' = DW(Linear_V X)   (SC, SC)
 *         EDIT_KV_FULL           K = ReLU(Linear_K X), V = Linear_V X over all N  (-, -)
 *         EDIT_KV_KEY_CONVFUSION K = ReLU(Linear_K(X + ConvFusion_K(X))) with the
 *                                key branch's own ConvFusion parameters, V = Linear_V X  (CF, -)
 * The table's rows are {CONVFUSION, COMPRESSED} (the layer itself),
 * {CONVFUSION, KEY_CONVFUSION}, {LINEAR, COMPRESSED} and {CONVFUSION, FULL}. */
typedef enum { EDIT_QUERY_CONVFUSION = 0, EDIT_QUERY_LINEAR = 1 } edit_query_mode_t;
typedef enum { EDIT_KV_COMPRESSED = 0, EDIT_KV_FULL = 1, EDIT_KV_KEY_CONVFUSION = 2 } edit_kv_mode_t;
typedef struct {
  edit_query_mode_t query;
  edit_kv_mode_t kv;
} edit_variant_t;

/* The key branch's ConvFusion parameters (shapes as the image stream's
 * w_cf1, b_cf1, gn_gamma, gn_beta, w_cf2, b_cf2). */
typedef struct {
  const void *w_cf1, *b_cf1, *gn_gamma, *gn_beta, *w_cf2, *b_cf2;
} edit_convfusion_weights_t;

/* Workspace bytes and layout of a variant; 0 / an error for an invalid one. */
size_t edit_attn_variant_workspace_size(const edit_shape_t* shape, const edit_variant_t* variant);
edit_status_t edit_attn_variant_workspace_layout(const edit_shape_t* shape, const edit_variant_t* variant,
                                                 edit_ws_layout_t* layout);

/* EDiT layer forward in an ablation variant. Arguments as edit_attn_forward;
 * weights the variant does not read may be NULL (the ConvFusion set with a
 * plain query, the depthwise set with uncompressed keys); key_cf is read (and
 * must be valid) only for EDIT_KV_KEY_CONVFUSION. {CONVFUSION, COMPRESSED}
 * gives edit_attn_forward's y bit for bit. */
edit_status_t edit_attn_variant_forward(const edit_shape_t* shape, const edit_variant_t* variant,
                                        const edit_weights_t* w, const edit_convfusion_weights_t* key_cf,
                                        const void* x, void* y,
                                        void* workspace, size_t ws_bytes, void* hip_stream);

/* Steps of one EDiT forward, in launch order (per-step timing). */
typedef enum {
  EDIT_STEP_CF_CONV3X3 = 0,  /* ConvFusion 3x3 compressing conv             (1 kernel)  */
  EDIT_STEP_GN_STATS = 1,    /* GroupNorm statistics                         (2 kernels) */
  EDIT_STEP_CF_ACT = 2,      /* GN + LeakyReLU; 1x1 restore folded into W_q (2 kernels) */
  EDIT_STEP_Q_PROJ = 3,      /* query Linear over [X | act] + ReLU           (1 kernel)  */
  EDIT_STEP_KV_PROJ = 4,     /* key and value Linears                        (1 kernel)  */
  EDIT_STEP_SC_DWCONV = 5,   /* depthwise 3x3 stride 2, ReLU on keys          (1 kernel)  */
  EDIT_STEP_KV_STATE = 6,    /* S = K'^T V', z = sum K' per head             (2 kernels) */
  EDIT_STEP_APPLY = 7,       /* y = q S / (q . z + eps)                      (1 kernel)  */
  EDIT_STEP_OUT_PROJ = 8,    /* output Linear                                (1 kernel)  */
  EDIT_NUM_STEPS = 9
} edit_step_t;

/* edit_attn_forward that also records events[i] (a hipEvent_t passed as
 * void*) on hip_stream just before step i is enqueued, and
 * events[EDIT_NUM_STEPS] after the last one, so hipEventElapsedTime between
 * neighbours times each step on the stream that runs it. events must hold
 * EDIT_NUM_STEPS + 1 created events; results equal edit_attn_forward's. */
edit_status_t edit_attn_forward_timed(const edit_shape_t* shape, const edit_weights_t* w,
                                      const void* x, void* y, void* workspace, size_t ws_bytes,
                                      void* hip_stream, void* const* events);

/* Gradients of the image-stream parameters: one output per edit_weights_t
 * member, same shape and dtype. */
typedef struct {
  void *w_cf1, *b_cf1, *gn_gamma, *gn_beta, *w_cf2, *b_cf2, *w_q, *b_q, *w_k, *b_k, *w_v, *b_v;
  void *dw_k, *db_k, *dw_v, *db_v, *w_o, *b_o;
} edit_grads_t;

/* Bytes of scratch edit_attn_backward needs for this shape (beyond the
 * forward's workspace); 0 if the shape is invalid. */
size_t edit_attn_backward_workspace_size(const edit_shape_t* shape);

/* EDiT layer backward: the gradients of sum(dy * y) with respect to x and to
 * every parameter, y = edit_attn_forward(x, w). It is the chain rule through
 * the forward steps (the page trains the layer by distillation, section
 * "训练策略" (training strategy), which needs them): the output Linear, the linear-attention
 * formula (dQ, dS, dz, then dK', dV' through S = sum K'^T V' and z = sum K'),
 * the depthwise stride-2 convs and their ReLU, the key / value Linears, and
 * ConvFusion (the query Linear with the 1x1 restore folded in, LeakyReLU,
 * GroupNorm, the 3x3 conv).
 *   fwd_workspace  the workspace of an edit_attn_forward call with the same
 *                  shape, weights and x, not modified since (its
 *                  intermediates are read, never written); fwd_ws_bytes its size
 *   dy             [B][H*W][C], gradient of the layer output
 *   dx             [B][H*W][C] out; grads: every member an output
 *   workspace      scratch of edit_attn_backward_workspace_size(shape) bytes
 * Parameter gradients are sums over the batch and the tokens, accumulated in
 * fp32 in a fixed order and rounded once to the dtype; outputs are
 * overwritten, not accumulated into. */
edit_status_t edit_attn_backward(const edit_shape_t* shape, const edit_weights_t* w,
                                 const void* x, const void* dy,
                                 const void* fwd_workspace, size_t fwd_ws_bytes,
                                 void* dx, const edit_grads_t* grads,
                                 void* workspace, size_t ws_bytes, void* hip_stream);

/* Where the backward's intermediate gradients of the last edit_attn_backward
 * call with this shape live in its workspace (byte offsets; a pure function
 * of the shape), for checking the backward step by step. T is the shape's
 * dtype; chain-rule steps as in edit_attn_backward:
 *   dy      [B][N][C]    T    gradient of the linear-attention output (dout W_o)
 *   dq_pre  [B][N][C]    T    gradient of the queries' pre-activation (the ReLU's mask applied)
 *   dS      [B][h][d][d] f32  gradient of S = sum K'^T V' (same index order as S)
 *   dz      [B][h][d]    f32  gradient of z = sum K'
 *   dkv     [B][N'][2C]  f32  gradients of the keys' pre-activation (ReLU's mask applied) | of V'
 *   dk0v0   [B][N][2C]   T    gradients of the key | value Linears' outputs
 *   dxq     [B][N][C]    T    gradient of the restored stream x + Conv1x1(act) (= dq_pre W_q)
 *   dxkv    [B][N][C]    T    dxq + the key and value Linears' input gradients
 *   dact    [B][N][C/r]  T    gradient of act = LeakyReLU(GN(xc))
 *   dxc     [B][N][.]    T    gradient of xc, rows of dxc_ld elements (C/r used, the rest zero) */
typedef struct {
  size_t dy, dq_pre, dS, dz, dkv, dk0v0, dxq, dxkv, dact, dxc;
  size_t dxc_ld;   /* elements per dxc row */
  size_t total;
} edit_bwd_layout_t;

edit_status_t edit_attn_backward_workspace_layout(const edit_shape_t* shape, edit_bwd_layout_t* layout);

const char* edit_status_string(edit_status_t status);
const char* edit_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EDIT_ATTN_H */
