// Launchers shared between the kernel files and the C-ABI layer. Every
// launcher only enqueues work on `stream` and returns hipGetLastError().
#pragma once

#include "common.hpp"

namespace rib {

// Windowed layouts of the gathers:
//   rows   [units][n_rows][d]  token-major, rows >= N zero
//   kappa  [units][d][n_rows]  channel-major; inside every group of 16 tokens the
//                              positions are permuted by swapping bits 2 and 3 of
//                              the token index (bf16 MFMA operands)

hipError_t launch_posgen(int w, const rib_mlp_t& mlp, rib_dtype_t out_dtype, void* q_p, void* k_p,
                         hipStream_t stream);
// Dynamic LDS bytes the posgen kernel needs for this MLP.
size_t posgen_lds_bytes(const rib_mlp_t& mlp);
// Position-MLP weight gradients from dQ_p, dK_p (float32 [w*w, rank] each):
// per-block partial sums into `workspace`, then a fixed-order reduction.
hipError_t launch_posgen_bwd(int w, const rib_mlp_t& mlp, const float* dq_p, const float* dk_p, float* dw1,
                             float* db1, float* dw2, float* db2, void* workspace, hipStream_t stream);
// LDS bytes of the smallest (one-token) tile: the MLP is supported iff this fits 64 KB.
size_t posgen_bwd_lds_bytes(const rib_mlp_t& mlp);
size_t posgen_bwd_workspace_bytes(int w, const rib_mlp_t& mlp);

// x [B,H,W,heads,d] -> windowed rows (rows >= N zero-filled).
hipError_t launch_partition(const Geom& g, int esize, const void* x, void* xw, hipStream_t stream);
// bf16, d_c = 32: K_c -> rows, V -> kappa, and the per-64-key partial maxima of
// |[k_c | k_p]|^2 (kp: [N][rp] rows, rp = 0 for none) and of |v| in one pass; kmax2 holds
// 2 * units * key_bound_parts(N) floats (the |k_hat|^2 maxima, then the |v| maxima).
hipError_t launch_gather_kv_bound(const Geom& g, int rp, const void* k, const void* v, const void* kp, void* kw,
                                  void* vt, float* kmax2, hipStream_t stream);
// bf16, d_c = 32 backward preparation in one pass (gather_bwd_kernel): maps
// [B, H, W, heads, 32] -> rows [units][n_rows][32]; lse [B, H, W, heads] -> -LSE2, and
// -D from dO and O, per row [units][n_rows]; Q_p, K_p [N][r] -> rows [n_rows][rp].
struct BwdGather {
  PixelMap pm;
  int N, n_rows, r, rp;
  float c;   // scale * log2(e): the Q_c, Q_p rows are stored as bf16(c q)
  const bf16 *q, *k, *v, *d_o, *o;
  const float* lse;
  const bf16 *q_p, *k_p;
  bf16 *qw, *kw, *vw, *dow;   // kw, vw nullptr: not written (the kernels read the maps)
  float *dd, *lse2;
  bf16 *qp, *kp;
};
hipError_t launch_gather_bwd(const BwdGather& a, int units, hipStream_t stream);
// windowed rows -> x [B,H,W,heads,d].
hipError_t launch_unpartition(const Geom& g, int esize, const void* xw, void* x, hipStream_t stream);
// Public plain gather / scatter ([units][N][d], no padding).
hipError_t launch_partition_plain(const Geom& g, int esize, const void* x, void* xw, hipStream_t stream);
hipError_t launch_unpartition_plain(const Geom& g, int esize, const void* xw, void* x, hipStream_t stream);

// [N, r] positional tokens -> [n_rows, rp] zero-padded copy in `out_esize`
// precision (rows >= N and columns >= r zero). In and out may differ in type.
hipError_t launch_pack_pos(int N, int n_rows, int r, int rp, int in_esize, const void* in, int out_esize,
                           void* out, hipStream_t stream);

struct FwdArgs {
  Geom g;
  float c;              // scale * log2(e)
  const void* qw;       // [units][n_rows][d_c] (simple path)
  const void* q_map;    // bf16 path: Q_c in the [B, H, W, heads, 32] map
  // bf16, one positional K-step, w dividing 64: K_c and V read in their maps by the attention
  // kernel (kw, vw and kmax2 unused); nullptr otherwise
  const void* k_map = nullptr;
  const void* v_map = nullptr;
  const void* kw;       // [units][n_rows][d_c]
  const void* vw;       // MFMA path: [units][32][n_rows] kappa layout; simple path: [units][n_rows][d_c]
  const void* qp;       // [n_rows][rp]
  const void* kp;       // [n_rows][rp]
  void* ow;             // [units][n_rows][d_c] (simple path)
  void* o_map;          // bf16 path: O in the [B, H, W, heads, 32] map
  float* lse;           // [B,H,W,heads] or nullptr
  float* kmax2;         // [2][units][key_bound_parts(N)] partial maxima of |[k_c | k_p]|^2, then of |v| (bf16 path)
  int rp;               // padded rank, 16 or 32 (0: the RPB comparison kernel)
  // RPB comparison kernel only (from launch_rpb_prep)
  const _Float16* rpb_tab16 = nullptr;  // [heads][rpb_stride] table * log2(e), fp16, zero-padded
  const float* rpb_max = nullptr;       // [heads] maximum of each fp16 row
  const int* rpb_kidx = nullptr;        // [n_rows] per-key LDS byte offsets into the table
  int rpb_stride = 0;                   // rpb_table_stride(w)
  // optional CLA gate [B, H, W, heads, d_c] (same dtype as O): O' = O * G in the epilogue
  const void* gate = nullptr;
  // Split tail (bf16 kernel, not the RPB one): each XCD's items past its last whole round
  // of workgroup slots are cut into split_s key ranges whose unnormalized partials go to
  // `part` and are summed by the combine kernel. split_spx = 0: no split.
  int split_spx = 0;       // workgroup slots per XCD
  int split_s = 1;         // key ranges per split item (2 or 4)
  int split_tail_max = 0;  // largest number of split items of one XCD
  float* part = nullptr;   // [8][split_tail_max][split_s] pieces of kSplitPieceFloats
};
// One split piece: the unnormalized O of 256 queries x 32 channels (float32), then per query
// its row sum and the shift m it is taken against.
constexpr int kSplitPieceFloats = 256 * 32 + 256 * 2;
// Workspace reserved for split pieces (shape-only bound, planned within at launch) and the
// smallest key-tile count (64 keys each) worth splitting.
constexpr int kMaxSplitPieces = 1024;
constexpr int kSplitMinTiles = 32;
size_t split_region_pieces(int units, int N);
// Sets the split fields of `a` (a.part must name split_region_pieces() pieces, or be null
// for no split) from the device's workgroup slots; leaves them at "no split" when the
// launch has no partial last round or the windows are too small.
hipError_t plan_fwd_split(FwdArgs& a);
hipError_t launch_fwd_split_combine(const FwdArgs& a, hipStream_t stream);
// Partial key-norm maxima per unit of the bf16 forward: one per 64 keys.
int key_bound_parts(int N);
hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream);
// One thread per query on windowed rows (qw, kw, vw, ow) of esize-byte elements with
// g.d_c in {32, 64} channels: float32 runs, and bf16 runs with d_c = 64.
hipError_t launch_attn_fwd_simple(const FwdArgs& a, int esize, hipStream_t stream);
// RPB comparison kernel: table [heads][(2w-1)^2] float32 -> fp16 log2-unit rows,
// row maxima and per-key offsets; then the attention (K/V windowed as for bf16).
int rpb_table_stride(int w);
size_t rpb_fwd_lds_bytes(int w);
hipError_t launch_rpb_prep(const Geom& g, const float* table, _Float16* tab16, float* tmax, int* kidx,
                           hipStream_t stream);
hipError_t launch_attn_fwd_rpb(const FwdArgs& a, hipStream_t stream);

// CLA gate G = sigmoid(PW_1x1(DW_3x3(X))) on a [B, H, W, C] map.
struct GateArgs {
  const void* x;        // [B, H, W, C], bf16 or float32
  const float* w_dw;    // [C, 3, 3]
  const float* b_dw;    // [C] or nullptr
  const float* w_pw;    // [C, C] (out, in)
  const float* b_pw;    // [C] or nullptr
  void* g;              // [B, H, W, C], same dtype as x
  int B, H, W, C;
};
bool cla_channels_supported(int C);
hipError_t launch_cla_gate(const GateArgs& a, int esize, hipStream_t stream);

struct BwdArgs {
  Geom g;
  float c;              // scale * log2(e)
  float scale;
  int rp;
  // windowed inputs
  const void* qw;       // [units][n_rows][d_c] rows
  const void* kw;       // [units][n_rows][d_c] rows
  const void* vw;       // [units][n_rows][d_c] rows
  const void* dow;      // [units][n_rows][d_c] rows
  const void* qp;       // [n_rows][rp]
  const void* kp;       // [n_rows][rp]
  const float* lse2;    // [units][n_rows]  log2-domain LSE (negated on the bf16 path)
  const float* dd;      // [units][n_rows]  D_i = sum_c dO_ic O_ic (negated on the bf16 path)
  // outputs: windowed (simple path) or in the [B, H, W, heads, 32] map (bf16 MFMA path)
  void* dqw;            // [units][n_rows][d_c] (simple path)
  void* dkw;            // [units][n_rows][d_c] (simple path)
  void* dvw;            // [units][n_rows][d_c] (simple path)
  void* dq_map;
  void* dk_map;
  void* dv_map;
  // bf16, one positional K-step, w dividing 64: K_c and V read in their maps by the kernels
  // (kw, vw unused); nullptr otherwise
  const void* k_map = nullptr;
  const void* v_map = nullptr;
  float* dqp_part;      // [units][n_rows][rp]
  float* dkp_part;      // [units][n_rows][rp]
};
// D and log2-domain LSE in windowed order, from O, dO and LSE in map layout (the simple
// kernels; the bf16 path gets -D and -LSE2 from launch_gather_bwd).
hipError_t launch_bwd_prep(const Geom& g, int esize, const void* o, const void* d_o, const float* lse,
                           float* dd, float* lse2, hipStream_t stream);
hipError_t launch_attn_bwd_dkv_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_attn_bwd_dq_bf16(const BwdArgs& a, hipStream_t stream);
// One thread per key (dkv) / query (dq) on windowed rows of esize-byte elements, d_c in {32, 64}.
hipError_t launch_attn_bwd_dkv_simple(const BwdArgs& a, int esize, hipStream_t stream);
hipError_t launch_attn_bwd_dq_simple(const BwdArgs& a, int esize, hipStream_t stream);
// Fixed-order sums over units of the [units][n_rows][rp] dQ_p and dK_p partials -> [N][r]
// float32 each, in one launch (units = 0: zeros).
hipError_t launch_reduce_pos_grads(int units, int N, int n_rows, int r, int rp, const float* part_q, float* out_q,
                                   const float* part_k, float* out_k, hipStream_t stream);

}  // namespace rib
