/*
 * rib.h - C ABI of the MI355X (gfx950) RIB window-attention library (librib.so).
 *
 * Rank-factorized Implicit Neural Bias (RIB) replaces an additive relative
 * positional bias by low-rank positional tokens Q_p, K_p that are generated
 * from normalized in-window coordinates (Fourier features + a small MLP) and
 * appended channel-wise to the content tokens, so the biased score is one
 * dot product:  S = [Q_c, Q_p][K_c, K_p]^T = Q_c K_c^T + Q_p K_p^T.
 * Sources (web pages on the paper "Rank-Factorized Implicit Neural Bias:
 * Scaling Super-Resolution Transformer with FlashAttention", arXiv 2603.06738):
 *   [EN]  gist.science/paper/2603.06738, "Technical Summary"
 *   [DE]  gist.science/de/paper/2603.06738, "Technische Zusammenfassung"
 *   [ES]  gist.science/es/paper/2603.06738, "Resumen tecnico"
 *   [ZH]  gist.science/zh/paper/2603.06738, technical part
 *   [ABS] khansong-paper-with-me.hf.space, the paper's abstract
 *
 * Conventions shared by every entry point
 *  - Pointers marked (device) are HIP device pointers, caller-allocated and
 *    caller-owned; the library never allocates or frees device memory. Pointers
 *    to structs are host. Host-side state: a per-device record of two fixed
 *    facts (compute units, and workgroups per CU of the forward kernel) and of
 *    the address of the allocation-free forward's workspace array, each filled
 *    once under a mutex, and the timing registry below; all are safe to use
 *    from several host threads. Device-side state: that one array per GPU
 *    (rib_window_attn_fwd_noalloc), used by no other entry point.
 *  - Tensors are dense, row-major, innermost dimension last, and 16-byte
 *    aligned. A feature map is [B, H, W, heads, d_c].
 *  - Windows are square, non-overlapping, unshifted and unpadded: H and W
 *    must be multiples of w. Inside a window, token t = iy*w + ix (row-major).
 *    Units (batch, window, head) are ordered: windows row-major per image,
 *    images in batch order, heads innermost.
 *  - Activations are RIB_F32 or RIB_BF16 (bfloat16). MLP weights, LSE and the
 *    positional-token gradients dQ_p, dK_p are always float32.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream): no host or device synchronisation. Outputs are overwritten,
 *    never accumulated into. Calls on different streams are safe when they
 *    use distinct output and workspace buffers.
 *  - Arguments are validated before anything is launched. A failing call
 *    launches nothing and returns a non-zero status; rib_last_error() then
 *    holds a message (per host thread). No C++ exception crosses this ABI.
 *  - Empty inputs (B == 0) are valid and launch nothing.
 *  - Supported today: d_c = 32 or 64; 1 <= r <= 32; 2 <= w <= 256. bfloat16 at
 *    d_c = 32 runs on the matrix-core kernels; float32 runs and d_c = 64 run on
 *    plain per-token kernels sized for correctness, not speed.
 */
#ifndef RIB_H
#define RIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RIB_OK = 0,
  RIB_ERR_INVALID_ARG = 1, /* bad shape, null or misaligned pointer, bad dtype */
  RIB_ERR_UNSUPPORTED = 2, /* valid arguments the library does not implement */
  RIB_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  RIB_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} rib_status_t;

typedef enum { RIB_F32 = 0, RIB_BF16 = 1 } rib_dtype_t;

/* A hipStream_t passed as an opaque handle. */
typedef void* rib_stream_t;

/* Shape of one attention call. */
typedef struct {
  int32_t B, H, W; /* batch and feature-map height / width */
  int32_t heads;   /* attention heads */
  int32_t d_c;     /* content channels per head (Q_c, K_c, V, O) */
  int32_t w;       /* window side; N = w*w tokens per window */
  int32_t r;       /* rank of the positional tokens Q_p, K_p */
} rib_shape_t;

/* Position MLP, nn.Linear layout (out x in), float32 (device). */
typedef struct {
  int32_t n_freq;   /* F: frequencies 2^k * pi, k = 0..F-1, per axis; 4F features */
  int32_t hidden;   /* hidden width */
  int32_t rank;     /* r: the MLP emits 2r values, Q_p first, then K_p */
  const float* w1;  /* [hidden, 4F] */
  const float* b1;  /* [hidden], or NULL for zeros */
  const float* w2;  /* [2r, hidden] */
  const float* b2;  /* [2r], or NULL for zeros */
} rib_mlp_t;

/*
 * rib_posgen - positional tokens of one window size [DE §2.A.1-2], [EN §2.A.1-2].
 *
 * Token t = iy*w + ix gets (x, y) = (c_ix, c_iy) with c_i = (2i - (w-1))/(w-1),
 * i.e. linspace(-1, 1, w) [DE §2.A.1]; features
 * phi = [sin(2^k pi x)]_k ++ [cos(2^k pi x)]_k ++ [sin(2^k pi y)]_k ++ [cos(2^k pi y)]_k;
 * out = W2 GELU(W1 phi + b1) + b2 with the exact (erf) GELU; Q_p[t] = out[0:r],
 * K_p[t] = out[r:2r]. The phase 2^k n/(w-1) is reduced exactly in integers
 * before sin/cos are evaluated. One (Q_p, K_p) serves every window, batch and
 * head of this window size, so it can be computed once and cached [DE §2.A.4].
 *
 *   w          window side, 2..256
 *   mlp        host pointer; 1 <= n_freq <= 16, 1 <= hidden <= 128, 1 <= rank <= 32,
 *              and the weights, staged in LDS, must fit 64 KB (RIB_ERR_UNSUPPORTED)
 *   out_dtype  element type of q_p and k_p
 *   q_p, k_p   (device) outputs, [w*w, rank] each
 */
rib_status_t rib_posgen(int32_t w, const rib_mlp_t* mlp, rib_dtype_t out_dtype,
                        void* q_p, void* k_p, rib_stream_t stream);

/*
 * rib_window_partition / rib_window_unpartition - the window gather and its inverse.
 *
 * partition:   x [B, H, W, heads, d_c]  ->  x_win [B*(H/w)*(W/w), heads, w*w, d_c]
 * unpartition: x_win -> x (the exact inverse). A pure copy: bit-exact.
 * Only shape->B, H, W, heads, d_c and w are used (any d_c with d_c*esize a
 * multiple of 16 bytes).
 */
rib_status_t rib_window_partition(const rib_shape_t* shape, rib_dtype_t dtype,
                                  const void* x, void* x_win, rib_stream_t stream);
rib_status_t rib_window_unpartition(const rib_shape_t* shape, rib_dtype_t dtype,
                                    const void* x_win, void* x, rib_stream_t stream);

/* Bytes of device workspace rib_window_attn_fwd needs for this shape (0 when
 * the shape is invalid, at least 256 otherwise). Linear in the feature-map size:
 * no N x N buffer. bf16 windows whose side divides 64 (8, 16, 32, 64) with
 * r <= 16 read K_c and V in their maps and gather nothing. At w*w >= 2048 tokens
 * the bf16 path also reserves room for the partial results of its split tail:
 * at most 1024 pieces of 34 KiB (about 34 MiB), and 4 per eight work items of
 * 256 queries when there are fewer. */
size_t rib_fwd_workspace_size(const rib_shape_t* shape, rib_dtype_t dtype);

/*
 * rib_window_attn_fwd - RIB window attention, forward [EN §2.A.3-4], [ABS].
 *
 * For every unit (batch, window, head):
 *   O = softmax(scale * [Q_c | Q_p][K_c | K_p]^T) V
 * over the N = w*w tokens of the window, with the same (Q_p, K_p) for every
 * unit. The N x N score matrix is never written to memory.
 *
 *   scale          softmax scale; <= 0 selects 1/sqrt(d_c + r)
 *   q_c, k_c, v    (device) [B, H, W, heads, d_c], dtype
 *   q_p, k_p       (device) [w*w, r], dtype (as produced by rib_posgen)
 *   o              (device) output [B, H, W, heads, d_c], dtype
 *   lse            (device) output [B, H, W, heads] float32 natural-log
 *                  log-sum-exp of each score row, or NULL
 *   workspace      (device) at least rib_fwd_workspace_size() bytes, 256-byte aligned
 */
rib_status_t rib_window_attn_fwd(const rib_shape_t* shape, rib_dtype_t dtype, float scale,
                                 const void* q_c, const void* k_c, const void* v,
                                 const void* q_p, const void* k_p,
                                 void* o, float* lse,
                                 void* workspace, size_t workspace_bytes,
                                 rib_stream_t stream);

/*
 * rib_window_attn_fwd_noalloc - rib_window_attn_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument, and nothing is allocated.
 *
 * The workspace is an array of RIB_NOALLOC_WORKSPACE_BYTES in the library's own device
 * memory, one per GPU, held from the library's first use on that GPU until the process
 * ends; the first call on a GPU looks up its address there (a caller that captures graphs
 * makes one call before capturing). Shapes whose rib_fwd_workspace_size() exceeds it return
 * RIB_ERR_WORKSPACE: the 16x16, 32x32 and 64x64 window layers of a [2, 192, 192, 6, 32] map
 * fit (their K_c and V are read in place; at most the split tail's 35 MB), the 96x96 workload
 * of 16 windows x 6 heads (about 150 MB) does not. Every call
 * on one GPU uses that GPU's array and overwrites it, so calls that overlap on one GPU
 * (several streams, several host threads) race: the caller serialises them. No part of the
 * array needs clearing: each call writes everything it reads. `stream` must belong to the
 * current device (RIB_ERR_INVALID_ARG otherwise). Arguments, outputs and other errors as
 * for rib_window_attn_fwd.
 */
#define RIB_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
rib_status_t rib_window_attn_fwd_noalloc(const rib_shape_t* shape, rib_dtype_t dtype, float scale,
                                         const void* q_c, const void* k_c, const void* v,
                                         const void* q_p, const void* k_p,
                                         void* o, float* lse, rib_stream_t stream);

/*
 * rib_cla_gate - the gating map of convolutional local attention (CLA) [EN §2.B: a
 * depth-wise conv, a point-wise conv and a sigmoid produce a map that modulates the
 * attention output; DE §2.B: G, O' = O (.) G; ZH §2.B: 3x3 depth-wise, 1x1 point-wise].
 *
 * On the map X [B, H, W, C], C = heads * d_c:
 *   D[y, x, c] = b_dw[c] + sum_{ky, kx in 0..2} w_dw[c, ky, kx] X[y + ky - 1, x + kx - 1, c]
 *                (cross-correlation over the whole map, zero outside it),
 *   G[y, x, o] = sigmoid(b_pw[o] + sum_c w_pw[o, c] D[y, x, c]).
 * Channel c of G lines up with head c / d_c, channel c % d_c of an attention output in
 * [B, H, W, heads, d_c] (rib_window_attn_fwd_gated). The bf16 path rounds D and the
 * point-wise weights to bf16 for the matrix cores and accumulates in float32.
 *
 *   shape        B, H, W, heads, d_c are used (w and r are ignored); C must be a
 *                multiple of 32 in [32, 256] (RIB_ERR_UNSUPPORTED otherwise)
 *   x            (device) [B, H, W, C], dtype
 *   w_dw, b_dw   (device) float32 [C, 3, 3] and [C] (b_dw may be NULL for zeros)
 *   w_pw, b_pw   (device) float32 [C, C] (out, in) and [C] (b_pw may be NULL)
 *   g            (device) output [B, H, W, C], dtype
 * No workspace. Errors as for rib_window_attn_fwd.
 */
rib_status_t rib_cla_gate(const rib_shape_t* shape, rib_dtype_t dtype, const void* x,
                          const float* w_dw, const float* b_dw, const float* w_pw,
                          const float* b_pw, void* g, rib_stream_t stream);

/*
 * rib_window_attn_fwd_gated - rib_window_attn_fwd followed by the CLA modulation
 * O' = O (.) G [DE §2.B], fused into the attention kernel's output stage (no extra pass
 * over O). `gate` (device, required) is [B, H, W, heads, d_c] in dtype, e.g. the output of
 * rib_cla_gate; `o` receives O'; `lse` (optional) is that of the ungated attention.
 * Workspace: rib_fwd_workspace_size(). This is a forward (inference) entry: training
 * needs the ungated O for the backward, so it calls rib_window_attn_fwd and gates apart.
 */
rib_status_t rib_window_attn_fwd_gated(const rib_shape_t* shape, rib_dtype_t dtype, float scale,
                                       const void* q_c, const void* k_c, const void* v,
                                       const void* q_p, const void* k_p, const void* gate,
                                       void* o, float* lse,
                                       void* workspace, size_t workspace_bytes,
                                       rib_stream_t stream);

/* Bytes of device workspace rib_window_attn_bwd needs (0 when invalid). */
size_t rib_bwd_workspace_size(const rib_shape_t* shape, rib_dtype_t dtype);

/*
 * rib_window_attn_bwd - gradients of the forward above given dO, for training
 * [EN §4 "Efficiency": the RIB network trains 2.1x faster than the RPB one;
 * ABS: RIB cuts training and inference time; DE §2.A.2: the MLP that makes
 * Q_p, K_p is learned, so the positional tokens need gradients as well].
 *
 * Recomputes P from LSE (no N x N buffer) and returns the content-token
 * gradients dQ_c, dK_c, dV and the positional-token gradients dQ_p, dK_p,
 * which sum the contributions of every unit that shares them. Deterministic:
 * the same inputs give the same bits on every call.
 *
 *   o, lse         (device) the forward's output and log-sum-exp (required)
 *   d_o            (device) upstream gradient [B, H, W, heads, d_c], dtype
 *   dq_c, dk_c, dv (device) outputs [B, H, W, heads, d_c], dtype
 *   dq_p, dk_p     (device) outputs [w*w, r] float32
 *   workspace      (device) at least rib_bwd_workspace_size() bytes, 256-byte aligned
 */
rib_status_t rib_window_attn_bwd(const rib_shape_t* shape, rib_dtype_t dtype, float scale,
                                 const void* q_c, const void* k_c, const void* v,
                                 const void* q_p, const void* k_p,
                                 const void* o, const float* lse, const void* d_o,
                                 void* dq_c, void* dk_c, void* dv,
                                 float* dq_p, float* dk_p,
                                 void* workspace, size_t workspace_bytes,
                                 rib_stream_t stream);

/*
 * rib_posgen_bwd - weight gradients of the position MLP [DE §2.A.2: a
 * lightweight MLP maps the Fourier features to Q_p and K_p; it is trained with
 * the network, so the positional gradients continue into its weights].
 *
 * With phi the Fourier features of rib_posgen (no parameters), z = W1 phi + b1,
 * h = GELU(z) (erf form) and d_out = [dQ_p | dK_p] per token:
 *   dW2 = sum_t d_out h^T, db2 = sum_t d_out,
 *   dz = (W2^T d_out) * GELU'(z), GELU'(z) = Phi(z) + z phi(z) (normal CDF, density),
 *   dW1 = sum_t dz phi^T, db1 = sum_t dz.
 * Outputs are overwritten, not accumulated. Deterministic: up to 1024 blocks
 * each sum a fixed set of token tiles (up to 32 tokens) into their own slot of
 * the workspace, and a second kernel adds the slots in a fixed order (four
 * contiguous ranges of blocks, each in block order, then the four range sums
 * in order). Float32 throughout.
 *
 *   w, mlp      as for rib_posgen (same limits; b1 / b2 may be NULL for zeros);
 *               W1, b1, W2 and one token's tile, staged in LDS, must fit 64 KB
 *               (every MLP rib_posgen accepts does)
 *   dq_p, dk_p  (device) float32 [w*w, rank]: gradients w.r.t. Q_p and K_p, e.g.
 *               the dq_p / dk_p of rib_window_attn_bwd (summed over every unit)
 *   dw1         (device) output float32 [hidden, 4F]
 *   db1         (device) output float32 [hidden], or NULL to skip
 *   dw2         (device) output float32 [2r, hidden]
 *   db2         (device) output float32 [2r], or NULL to skip
 *   workspace   (device) at least rib_posgen_bwd_workspace_size() bytes, 4-byte
 *               aligned, caller-owned; its contents on return are unspecified
 * Errors: RIB_ERR_INVALID_ARG for bad sizes, NULL or misaligned pointers;
 * RIB_ERR_WORKSPACE for a missing or short workspace; RIB_ERR_UNSUPPORTED beyond
 * the limits above. Nothing is launched when an error is returned.
 */
size_t rib_posgen_bwd_workspace_size(int32_t w, const rib_mlp_t* mlp);
rib_status_t rib_posgen_bwd(int32_t w, const rib_mlp_t* mlp, const float* dq_p, const float* dk_p,
                            float* dw1, float* db1, float* dw2, float* db2,
                            void* workspace, size_t workspace_bytes, rib_stream_t stream);

/* Bytes of device workspace rib_rpb_window_attn_fwd needs (0 when invalid). */
size_t rib_rpb_fwd_workspace_size(const rib_shape_t* shape, rib_dtype_t dtype);

/*
 * rib_rpb_window_attn_fwd - the relative-position-bias (RPB) attention that
 * RIB replaces [EN "Problem Statement": an additive bias B indexed by relative
 * position breaks the fused kernel's plain QK^T structure and its table grows
 * with the window area; ES §1], as a comparison kernel on the same shapes.
 *
 * For every unit (batch, window, head h), over the N = w*w tokens of the window:
 *   O = softmax(scale * Q_c K_c^T + B_h) V,
 *   B_h[i, j] = table[h][(y_i - y_j + w - 1) * (2w - 1) + (x_i - x_j + w - 1)]
 * with token t = y*w + x. The bias is gathered per score from the table (no
 * N x N bias or score matrix in memory); the table is staged per workgroup in
 * LDS as fp16 after multiplication by log2(e), so entries must satisfy
 * |b| < 45000 and carry fp16 rounding (relative 2^-11).
 *
 *   shape          as for rib_window_attn_fwd; shape->r is ignored. d_c = 32;
 *                  w is limited by LDS: the (2w-1)^2 fp16 table plus the tile
 *                  ring must fit one CU's 160 KB (w <= 121), else
 *                  RIB_ERR_UNSUPPORTED
 *   dtype          RIB_BF16 only (RIB_ERR_UNSUPPORTED otherwise)
 *   scale          <= 0 selects 1/sqrt(d_c)
 *   q_c, k_c, v    (device) [B, H, W, heads, d_c] bfloat16
 *   table          (device) [heads, (2w-1)^2] float32
 *   o              (device) output [B, H, W, heads, d_c] bfloat16
 *   lse            (device) output [B, H, W, heads] float32 or NULL
 *   workspace      (device) at least rib_rpb_fwd_workspace_size() bytes,
 *                  256-byte aligned; contents on return unspecified
 * Errors as for rib_window_attn_fwd.
 */
rib_status_t rib_rpb_window_attn_fwd(const rib_shape_t* shape, rib_dtype_t dtype, float scale,
                                     const void* q_c, const void* k_c, const void* v,
                                     const float* table, void* o, float* lse,
                                     void* workspace, size_t workspace_bytes,
                                     rib_stream_t stream);

/*
 * Kernel timing, a measurement aid: while enabled, every posgen / forward /
 * backward call brackets each of its kernel groups with HIP events recorded
 * on the call's stream. rib_kernel_timing_read() waits for the recorded
 * events of one group, returns their summed duration in milliseconds and the
 * number of timed launches, and forgets them. Disabled by default; while
 * disabled no events are created. The recorded events are process-wide
 * host state guarded by a mutex.
 *
 * Each event pair sits between two launches on the stream and costs a few
 * microseconds of idle GPU there, so a caller that needs one group's launch
 * time while timing a whole step selects that group alone:
 * rib_kernel_timing_select(mask) times group k when bit k of mask is set
 * (0 turns timing off; bits past the last group are RIB_ERR_INVALID_ARG).
 * rib_kernel_timing_enable(e) selects every group (e != 0) or none.
 */
typedef enum {
  RIB_KERNEL_POSGEN = 0,       /* the posgen kernel */
  RIB_KERNEL_PARTITION = 1,    /* the gathers of one call (map -> window layouts, positional packing) */
  RIB_KERNEL_ATTN_FWD = 2,     /* the forward attention kernel alone */
  RIB_KERNEL_UNPARTITION = 3,  /* the scatters of one call (window layout -> map); for the
                                  bf16 forward, the combine of its split tail */
  RIB_KERNEL_BWD_PREP = 4,     /* D = rowsum(dO * O) and log2-domain LSE */
  RIB_KERNEL_ATTN_BWD_DKV = 5, /* the backward dK / dV kernel alone */
  RIB_KERNEL_ATTN_BWD_DQ = 6,  /* the backward dQ kernel alone */
  RIB_KERNEL_POS_REDUCE = 7,   /* the fixed-order sum of the dQ_p / dK_p partials */
  RIB_KERNEL_POSGEN_BWD = 8,   /* the position-MLP weight-gradient kernels (partials + sum) */
  RIB_KERNEL_RPB_ATTN_FWD = 9, /* the RPB comparison attention kernel alone */
  RIB_KERNEL_CLA_GATE = 10,    /* the CLA gate kernel */
  RIB_KERNEL_COUNT = 11
} rib_kernel_t;

rib_status_t rib_kernel_timing_enable(int32_t enable);
rib_status_t rib_kernel_timing_select(uint32_t mask);
rib_status_t rib_kernel_timing_read(rib_kernel_t kernel, double* total_ms, int64_t* launches);

/* Static text naming a status code. */
const char* rib_status_string(rib_status_t status);

/* Detail of the last failing call on this host thread ("" if none). */
const char* rib_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RIB_H */
