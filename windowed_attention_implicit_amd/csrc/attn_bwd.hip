// RIB window attention, backward, for gfx950.
//
// Given dO, recomputes P = exp(scale S - LSE) per tile (no N x N buffer) and
// forms the textbook softmax gradients dV = P^T dO, dP = dO V^T,
// dS = P * (dP - D) with D_i = sum_c dO_ic O_ic, and
// d[Q_c|Q_p] = scale dS [K_c|K_p], d[K_c|K_p] = scale dS^T [Q_c|Q_p]. The
// positional parts are summed over every (batch, window, head) unit because
// one (Q_p, K_p) serves all of them (gist.science/de "Technische
// Zusammenfassung" §2.A.4: Q_p, K_p depend only on the window geometry).
//
// bf16 design: two MFMA kernels, deterministic (no atomics):
//  * dkv: a workgroup owns 256 keys (4 waves x 64); it streams 64-query tiles
//    of Q_hat and dO (token-major rows) and their -LSE2, -D through LDS.
//    S = Q_hat K_hat^T and dP = dO V^T come out with one key per lane, so P
//    and dS feed dV^T += dO^T P and dK_hat^T += Q_hat^T dS directly as MFMA B
//    operands; the channel-major A operands dO^T, Q_hat^T come from the same
//    rows by transposing LDS reads (tr_frag).
//  * dq: a workgroup owns 256 queries; it streams 64-key tiles of K_hat and V
//    rows and accumulates dQ_hat^T += K_hat^T dS^T with one query per lane,
//    like the forward (K_hat^T by transposing reads).
//  * The Q_c, Q_p rows arrive pre-scaled by c = scale * log2(e) and rounded to
//    bf16 exactly as the forward rounds them (the one-pass backward gather), so
//    both kernels form the forward's scores and the score MFMA yields log2-domain
//    logits directly. dK_hat = scale dS^T Q_hat is formed from the same pre-scaled
//    rows and multiplied by scale / c (one more bf16 rounding of Q_hat, not
//    visible in bf16 outputs; sum_j dK_hat[j] = 0 holds for any Q rows). In dkv (one key per lane, queries along the accumulator
//    rows) -LSE2 / -D enter as the accumulator inputs of the score / dP MFMAs,
//    so P = exp2(acc) and dS = P * acc: per score one exp2, one multiply and
//    the bf16 packs. In dq (one query per lane) -LSE2 is a lane constant held
//    as the score MFMA's accumulator input, and at r <= 16 -D enters through a
//    third dP K-step against a constant ones fragment; at r <= 32 there are no
//    registers for that and -D is added on the vector pipe.
//  * Both kernels are compiled with the VGPR form of the MFMAs (build flag):
//    their state exceeds 256 arch VGPRs, and the AGPR form the compiler would
//    otherwise pick costs a register copy per score.
//  * Positional-gradient partials are written per unit in float32 and summed
//    over units in a fixed order by a separate reduction.
//  * MAPKV (one positional K-step, windows whose side w divides 64): a 64-key
//    tile is 64 / w whole window rows, so K_c and V tiles (and the owned keys'
//    K_c, V) are read in their [B, H, W, heads, 32] maps, each token's 64 bytes
//    at its pixel; the gather then writes only the pre-scaled Q rows, the dO rows
//    and the row statistics. (dkv keeps reading dO tiles from windowed rows:
//    map-addressed offsets for them would cost it the last registers it has.)
#include "internal.hpp"
#include "tile_dma.hpp"

namespace rib {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4v;

constexpr int kTile = 64;          // streamed tile (queries in dkv, keys in dq)
constexpr int kPerBlock = 256;     // owned keys (dkv) / queries (dq) per workgroup

template <int KP>
struct BwdCfg {
  static constexpr int kSteps = 2 + KP;           // 16-channel steps of [content | pos]
  static constexpr int kCRow = 5;                 // chunks per content / dO / V row in LDS (4 + 1 pad)
  static constexpr int kPRow = 2 * KP + 1;        // chunks per positional row (2KP + 1 pad)
  static constexpr int kPosRows = 16 * KP;
};

// LDS tile layouts (parts in DMA order). dkv streams query tiles: Q_hat
// content and positional rows, dO rows, and the tile's -LSE2 and -D.
template <int KP>
struct DkvTile {
  static constexpr TileLayout<5> get() {
    return {{{kTile, 4, 5}, {kTile, 2 * KP, 2 * KP + 1}, {kTile, 4, 5}, {1, 16, 16}, {1, 16, 16}}};
  }
};
// dq streams key tiles: K_hat content and positional rows and V rows.
template <int KP>
struct DqTile {
  static constexpr TileLayout<3> get() { return {{{kTile, 4, 5}, {kTile, 2 * KP, 2 * KP + 1}, {kTile, 4, 5}}}; }
};
// LDS tile rings. dkv at r <= 16 runs two workgroups per CU with a 2-deep ring (tile t + 1 in
// flight while tile t is processed, 15 KB per tile): a deeper ring costs it the registers it
// has left (3 buffers spill 14 VGPRs to scratch). dkv at r <= 32 (one workgroup per CU) and dq
// (two) fetch tile t + 3 while processing tile t.
template <int KP>
constexpr int kBufsDkv = KP == 1 ? 2 : 4;
constexpr int kBufsDq = 4;

// Workgroup barrier without the release fence of __syncthreads, which would
// wait for every tile DMA in flight. Callers wait for the DMA they depend on
// first; the waves write no LDS in the main loops. The memory clobber keeps
// the compiler from moving LDS reads or DMA issue across it.
__device__ __forceinline__ void barrier_dma() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 lds_frag(const u32x4* p) { return __builtin_bit_cast(bf16x8, *p); }

__device__ __forceinline__ bf16x8 zero_frag() { return __builtin_bit_cast(bf16x8, u32x4(0u)); }

// Channel-major MFMA operand from token-major rows in LDS (part: the rows' first chunk,
// row_chunks: the row pitch in 16-byte chunks) by transposing reads (ds_read_b64_tr_b16): in
// each 16-lane group, lane i gets element i & 3 of the 8 bytes read by lanes (i >> 2) + 4j,
// j = 0..3. Lane si of the group reads rows row0 + (si >> 2) and row0 + 8 + (si >> 2) at
// channels ch0 + 4 (si & 3) .. + 3, so lane i gets channel ch0 + i of rows row0 + 0..3 and
// row0 + 8..11 (the order of the P / dS operands: bits 2 and 3 of the row swapped). row0 and
// ch0 must be uniform over each 16-lane group.
__device__ __forceinline__ bf16x8 tr_frag(const u32x4* part, int row_chunks, int row0, int ch0, int lane) {
  const int si = lane & 15;
  auto* b = (__attribute__((address_space(3))) char*)part + (ch0 + 4 * (si & 3)) * 2;
  const int r = row0 + (si >> 2);
  const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4v*)(b + r * row_chunks * 16));
  const bf16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4v*)(b + (r + 8) * row_chunks * 16));
  bf16x8 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[j] = lo[j];
    out[4 + j] = hi[j];
  }
  return out;
}


// Epilogue stores of a 32-channel bf16 result whose lane holds the channels 8 gq + 4 h + i
// (i < 4) of token (block nb, lane % 32): stored as they are, each store instruction would
// touch 32 map rows with 8 bytes each. The wave stages its 64 rows in its own LDS region
// ([64 rows][5 chunks]) and writes whole 64-byte rows back, 16 rows per store instruction.
// `row_of(t)` is the map element offset of token t, `val(nb, v)` the lane's value v of block nb.
constexpr int kStageRow = 5;
template <class RowOf, class Val>
__device__ __forceinline__ void stage_store_rows(bf16* stage, bf16* dst, int t0, int N, int lane, RowOf row_of, Val val) {
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      bf16 o4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = f32_to_bf16(val(nb, 4 * gq + i));
      *(uint2*)(stage + (nb * 32 + l32) * kStageRow * 8 + 8 * gq + 4 * half) = *(const uint2*)o4;
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rl = (lane >> 2) + 16 * j, ch = 8 * (lane & 3);
    const u32x4 v = *(const u32x4*)(stage + rl * kStageRow * 8 + ch);
    if (t0 + rl < N) *(u32x4*)(dst + row_of(t0 + rl) + ch) = v;
  }
}

// Loads the lane's 8 channels (16s + 8h ..) of a [content 32 | pos rp] token whose content and
// positional rows start at `content` and `pos`.
__device__ __forceinline__ bf16x8 token_frag(const bf16* content, const bf16* pos, int s, int half) {
  u32x4 v;
  if (s < 2) v = *(const u32x4*)(content + s * 16 + half * 8);
  else v = *(const u32x4*)(pos + (s - 2) * 16 + half * 8);
  return __builtin_bit_cast(bf16x8, v);
}

// Where the token rows of a unit live: its windowed rows (32 elements each) or, for MAPKV,
// its window in a [B, H, W, heads, 32] map: token t at base + (t / w) W heads 32 +
// (t % w) heads 32 elements (w a power of two, lw = log2 w). dma() describes 64-token tiles
// of such rows for tile_dma.
template <bool MAPKV>
struct TokenRows {
  const bf16* base;
  int lw, row_bytes, pix_bytes, span_bytes;
  __device__ TokenRows(const void* map, const void* rows, const Geom& g, int unit) {
    if constexpr (MAPKV) {
      base = (const bf16*)map + make_pixel_map(g).pixel_head(unit, 0) * 32;
      lw = __builtin_ctz(g.w);
      row_bytes = g.W * g.heads * 64;
      pix_bytes = g.heads * 64;
      span_bytes = (g.w - 1) * row_bytes + (g.w - 1) * pix_bytes + 64;
    } else {
      base = (const bf16*)rows + (int64_t)unit * g.n_rows * 32;
      lw = row_bytes = pix_bytes = 0;
      span_bytes = g.n_rows * 64;
    }
  }
  __device__ const bf16* row(int t) const {
    if constexpr (MAPKV) return base + (int64_t)(t >> lw) * (row_bytes / 2) + (int64_t)(t & ((1 << lw) - 1)) * (pix_bytes / 2);
    else return base + (int64_t)t * 32;
  }
  __device__ DmaSrc dma() const {
    if constexpr (MAPKV) return {base, span_bytes, row_bytes, (kTile >> lw) * row_bytes, lw, pix_bytes};
    else return {base, span_bytes, 64, kTile * 64};
  }
};

// Positional gradients at r = 16 on v_mfma_f32_16x16x32_bf16. A 32-key (dkv) or
// 32-query (dq) column block's dS leaves the score layout as sb[2]: lane l holds, for
// column l % 32, the 16 contraction indices 16 s + 8 (j / 4) + 4 h + j % 4 (h = l / 32,
// j < 8) of the sub-tile. Swapping the odd 16-lane rows of sb[1] with the even rows of
// sb[0] (v_permlane16_swap) leaves two B operands of 16 columns each: b[0] columns 0-15,
// b[1] columns 16-31, and in both, k-block l / 16 = 0, 1, 2, 3 holds (s, h) = (1, 0),
// (0, 0), (1, 1), (0, 1), i.e. (s, h) = (c / 2, c % 2) with c = pos16_chunk(l): the A
// fragment of lane l is channel l % 16 of the sub-tile's rows 16 s + 4 h + 0..3 and
// 16 s + 8 + 4 h + 0..3.
__device__ __forceinline__ int pos16_chunk(int lane) {
  const int kb = lane >> 4;
  return 2 * (1 - (kb & 1)) + (kb >> 1);
}

__device__ __forceinline__ void pos16_b(const bf16x8 (&sb)[2], bf16x8 (&b)[2]) {
  const u32x4 x = __builtin_bit_cast(u32x4, sb[1]), y = __builtin_bit_cast(u32x4, sb[0]);
  u32x4 bx, by;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const auto r = __builtin_amdgcn_permlane16_swap(x[d], y[d], false, false);
    bx[d] = r[0];
    by[d] = r[1];
  }
  b[0] = __builtin_bit_cast(bf16x8, bx);
  b[1] = __builtin_bit_cast(bf16x8, by);
}

// ------------------------------------------------------------------ dK, dV
template <int KP, bool MAPKV = false>
// Compiled with the register budget of one workgroup per CU: the schedule the compiler makes
// under it is 4-7 % faster at every window size measured (16 to 96) than under the budget of two,
// and the counters still show about two workgroups resident per CU. (Holding the dQ kernel to
// one resident workgroup per CU makes it 35 % slower.)
__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_kernel(BwdArgs a) {
  static_assert(!MAPKV || KP == 1, "map-addressed K / V: one positional K-step only");
  typedef BwdCfg<KP> C;
  typedef DkvTile<KP> LP;
  constexpr auto L = LP::get();
  constexpr int oQc = L.offset(0), oQp = L.offset(1), oDo = L.offset(2), oL = L.offset(3), oD = L.offset(4);
  constexpr int kBufs = kBufsDkv<KP>, kAhead = kBufs - 1;   // tiles in flight ahead of the current one
  __shared__ u32x4 sT[kBufs][L.chunks()];

  const Geom& g = a.g;
  const int N = g.N, n_rows = g.n_rows;
  const int nkb = (N + kPerBlock - 1) / kPerBlock;
  const int logical = xcd_remap(blockIdx.x, g.units * nkb);
  const int unit = logical / nkb;
  const int kb = logical - unit * nkb;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int rp = 16 * KP;

  const int64_t ub = (int64_t)unit * n_rows;
  const bf16* qw = (const bf16*)a.qw + ub * 32;
  const TokenRows<MAPKV> kr(a.k_map, a.kw, g, unit), vr(a.v_map, a.vw, g, unit);
  const TokenRows<false> dr(nullptr, a.dow, g, unit);
  const bf16* qp = (const bf16*)a.qp;
  const bf16* kp = (const bf16*)a.kp;
  const float* lse2 = a.lse2 + ub;
  const float* dd = a.dd + ub;

  // owned keys: B operands of S = Q_hat K_hat^T and dP = dO V^T
  const int k0 = kb * kPerBlock + wave * 64;
  bf16x8 kf[2][C::kSteps], vf[2][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int key = k0 + nb * 32 + l32;
    const bool ok = key < N;
    const bf16* krow = kr.row(ok ? key : 0);
    const bf16* vrow = vr.row(ok ? key : 0);
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s)
      kf[nb][s] = ok ? token_frag(krow, kp + (int64_t)key * rp, s, half) : zero_frag();
#pragma unroll
    for (int s = 0; s < 2; ++s)
      vf[nb][s] = ok ? __builtin_bit_cast(bf16x8, *(const u32x4*)(vrow + s * 16 + half * 8)) : zero_frag();
  }

  // acc_dkp: KP = 2, dK_p^T on 32x32 tiles; KP = 1, its 16 channels on two 16x16 tiles per
  // column block (keys 0-15 / 16-31 of the block), 8 registers instead of 16
  f32x16 acc_dv[2], acc_dk[2], acc_dkp[2];
  f32x4 acc_dkp16[2][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc_dv[nb][i] = 0.f; acc_dk[nb][i] = 0.f; acc_dkp[nb][i] = 0.f; }
    acc_dkp16[nb][0] = acc_dkp16[nb][1] = f32x4(0.f);
  }

  // query tiles reach LDS by DMA (buffer_load ... lds), three tiles ahead
  const int row64 = n_rows * 64, pos_bytes = n_rows * rp * 2;
  const DmaSrc src[5] = {
      {qw, row64, 64, kTile * 64},        {qp, pos_bytes, rp * 2, kTile * rp * 2}, dr.dma(),
      {lse2, n_rows * 4, 256, kTile * 4}, {dd, n_rows * 4, 256, kTile * 4},
  };
  TileDma<L.kParts, L.slots()> dma;
  tile_dma_init<LP>(dma, src, wave, lane);

  const int nqt = (N + kTile - 1) / kTile;
#pragma unroll
  for (int i = 0; i < kAhead; ++i) tile_dma_issue<LP>(dma, wave, min(i, nqt - 1), sT[i]);
  tile_dma_wait<LP, kAhead - 1>(wave);
  __syncthreads();
  for (int t = 0; t < nqt; ++t) {
    // tile t + kAhead (the last tile again past the end) into the buffer tile t - 1 used
    tile_dma_issue<LP>(dma, wave, min(t + kAhead, nqt - 1), sT[(t + kAhead) % kBufs]);
    const u32x4* T = sT[t % kBufs];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int row = sub * 32 + l32;
      bf16x8 qa[C::kSteps], da[2];
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s)
        qa[s] = s < 2 ? lds_frag(&T[oQc + row * C::kCRow + 2 * s + half])
                      : lds_frag(&T[oQp + row * C::kPRow + 2 * (s - 2) + half]);
#pragma unroll
      for (int s = 0; s < 2; ++s) da[s] = lds_frag(&T[oDo + row * C::kCRow + 2 * s + half]);
      // -LSE2 and -D of the lane's 16 accumulator rows (queries 8(v/4) + 4h + v%4)
      f32x16 nl, nd;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int qi = sub * 32 + 8 * gq + 4 * half;
        const f32x4 l4 = __builtin_bit_cast(f32x4, T[oL + qi / 4]);
        const f32x4 d4 = __builtin_bit_cast(f32x4, T[oD + qi / 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) { nl[4 * gq + i] = l4[i]; nd[4 * gq + i] = d4[i]; }
      }
      bf16x8 dta[2], qta[2], qpta[2];
      const int ch0 = 16 * ((lane >> 4) & 1);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int r0 = sub * 32 + s * 16 + 4 * half;
        dta[s] = tr_frag(&T[oDo], C::kCRow, r0, ch0, lane);
        qta[s] = tr_frag(&T[oQc], C::kCRow, r0, ch0, lane);
        if constexpr (KP == 2) qpta[s] = tr_frag(&T[oQp], C::kPRow, r0, ch0, lane);
      }
      // KP = 1: A of the 16x16x32 dK_p MFMA, channel lane % 16, the sub-tile's queries of
      // k-block lane / 16 in the order pos16_b() leaves dS in
      if constexpr (KP == 1) {
        const int c = pos16_chunk(lane);
        qpta[0] = tr_frag(&T[oQp], C::kPRow, sub * 32 + 16 * (c >> 1) + 4 * (c & 1), 0, lane);
      }
      // scores and dP of both key blocks first, so the vector work of block 0 runs while
      // block 1's MFMAs are in the matrix pipe
      f32x16 scs[2], dps[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        // sc = S' - LSE2 (log2 domain), dp = dP - D
        f32x16 sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0], kf[nb][0], nl, 0, 0, 0);
#pragma unroll
        for (int s = 1; s < C::kSteps; ++s) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kf[nb][s], sc, 0, 0, 0);
        f32x16 dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[0], vf[nb][0], nd, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[1], vf[nb][1], dp, 0, 0, 0);
        scs[nb] = sc;
        dps[nb] = dp;
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const f32x16 sc = scs[nb], dp = dps[nb];
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int v = 8 * s + j;
            const float p = __builtin_amdgcn_exp2f(sc[v]);
            pb[s][j] = f32_to_bf16(p);
            sb[s][j] = f32_to_bf16(p * dp[v]);
          }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          acc_dv[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dta[s], pb[s], acc_dv[nb], 0, 0, 0);
          acc_dk[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta[s], sb[s], acc_dk[nb], 0, 0, 0);
          if constexpr (KP == 2)
            acc_dkp[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qpta[s], sb[s], acc_dkp[nb], 0, 0, 0);
        }
        if constexpr (KP == 1) {
          bf16x8 b16[2];
          pos16_b(sb, b16);
#pragma unroll
          for (int m = 0; m < 2; ++m)
            acc_dkp16[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qpta[0], b16[m], acc_dkp16[nb][m], 0, 0, 0);
        }
      }
    }
    tile_dma_wait<LP, kAhead - 1>(wave);   // tile t + 1 landed (this wave's part); later ones may be in flight
    barrier_dma();
  }

  // epilogue: lane = key, accumulator rows = channels 8(v/4) + 4h + v%4; dK_c and dV rows go
  // straight to the [B, H, W, heads, 32] map (row of token t = window base + (t / w) W heads +
  // (t % w) heads)
  const int64_t map_base = make_pixel_map(g).pixel_head(unit, 0) * 32;
  const int64_t row_elems = (int64_t)g.W * g.heads * 32, pix_elems = (int64_t)g.heads * 32;
  bf16* dkm = (bf16*)a.dk_map;
  bf16* dvm = (bf16*)a.dv_map;
  float* dkp = a.dkp_part + ub * rp;
  const float scale = a.scale;
  const float kscale = a.scale / a.c;   // dK_hat from the pre-scaled Q_hat rows
  {
    // dV, then dK, staged through the wave's LDS region (the tile ring is free once the DMA of
    // tiles past the end has drained and every wave is past the loop)
    static_assert(4 * 64 * kStageRow <= kBufs * L.chunks(), "staging fits the tile ring");
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __syncthreads();
    bf16* stage = (bf16*)&sT[0][0] + wave * 64 * kStageRow * 8;
    auto row_of = [&](int t) { return map_base + (int64_t)(t / g.w) * row_elems + (int64_t)(t % g.w) * pix_elems; };
    stage_store_rows(stage, dvm, k0, N, lane, row_of, [&](int nb, int v) { return acc_dv[nb][v]; });
    stage_store_rows(stage, dkm, k0, N, lane, row_of, [&](int nb, int v) { return acc_dk[nb][v] * kscale; });
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int key = k0 + nb * 32 + l32;
    if (key >= N) continue;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int ch = 8 * gq + 4 * half;
      if (KP == 2) {
        f32x4 p4;
#pragma unroll
        for (int i = 0; i < 4; ++i) p4[i] = acc_dkp[nb][4 * gq + i] * kscale;
        *(f32x4*)(dkp + (int64_t)key * rp + ch) = p4;
      }
    }
  }
  if constexpr (KP == 1) {
    // 16x16 tiles: lane holds channels 4 (lane / 16) + i of key 16 m + lane % 16 of the block
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int key = k0 + nb * 32 + 16 * m + (lane & 15);
        if (key < N) *(f32x4*)(dkp + (int64_t)key * rp + 4 * (lane >> 4)) = acc_dkp16[nb][m] * kscale;
      }
  }
}

// ------------------------------------------------------------------ dQ
template <int KP, bool MAPKV = false>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(BwdArgs a) {
  static_assert(!MAPKV || KP == 1, "map-addressed K / V: one positional K-step only");
  typedef BwdCfg<KP> C;
  typedef DqTile<KP> LP;
  constexpr auto L = LP::get();
  constexpr int oKc = L.offset(0), oKp = L.offset(1), oV = L.offset(2);
  __shared__ u32x4 sT[kBufsDq][L.chunks()];

  const Geom& g = a.g;
  const int N = g.N, n_rows = g.n_rows;
  const int nqb = (N + kPerBlock - 1) / kPerBlock;
  const int logical = xcd_remap(blockIdx.x, g.units * nqb);
  const int unit = logical / nqb;
  const int qb = logical - unit * nqb;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int rp = 16 * KP;

  const int64_t ub = (int64_t)unit * n_rows;
  const bf16* qw = (const bf16*)a.qw + ub * 32;
  const TokenRows<MAPKV> kr(a.k_map, a.kw, g, unit), vr(a.v_map, a.vw, g, unit);
  const TokenRows<false> dr(nullptr, a.dow, g, unit);
  const bf16* qp = (const bf16*)a.qp;
  const bf16* kp = (const bf16*)a.kp;

  // owned queries: B operands of S^T = K_hat Q_hat^T and dP^T = V dO^T
  const int q0 = qb * kPerBlock + wave * 64;
  // KP = 1: dP - D comes out of the dP MFMAs: a third K-step pairs channels 0 and 1 of a
  // constant "ones" V fragment (vone) with -D split into two bf16 parts (dext, hi + lo,
  // about 16 significant bits) on the dO side, which takes the per-score subtraction off
  // the vector pipe for one MFMA of the matrix pipe's slack. Padded keys get dP - D = -D,
  // harmless: their K_hat rows are zero. (KP = 2 has no registers to spare for it and adds
  // -D on the vector pipe.)
  constexpr bool kDext = KP == 1;
  bf16x8 qf[2][C::kSteps], df[2][2], dext[2], vone, lext[2], kone;
  float nlq[2], ndq[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) vone[j] = (half == 0 && j < 2) ? (bf16)1.0f : (bf16)0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) kone[j] = (half == 0 && j < 3) ? (bf16)1.0f : (bf16)0.0f;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int q = q0 + nb * 32 + l32;
    const bool ok = q < N;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s)   // rows stored pre-scaled
      qf[nb][s] = ok ? token_frag(qw + (int64_t)q * 32, qp + (int64_t)q * rp, s, half) : zero_frag();
    const bf16* drow = dr.row(ok ? q : 0);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      df[nb][s] = ok ? __builtin_bit_cast(bf16x8, *(const u32x4*)(drow + s * 16 + half * 8)) : zero_frag();
    nlq[nb] = ok ? a.lse2[ub + q] : -INFINITY;   // stored negated: -LSE2, -D
    const float nd = ok ? a.dd[ub + q] : 0.f;
    ndq[nb] = nd;
    const bf16 hi = f32_to_bf16(nd);
    const bf16 lo = f32_to_bf16(nd - (float)hi);
#pragma unroll
    for (int j = 0; j < 8; ++j) dext[nb][j] = half == 0 && j == 0 ? hi : (half == 0 && j == 1 ? lo : (bf16)0.0f);
    // -LSE2 in three bf16 parts for the score MFMA's extra K-step: 3 x 8 significant bits hold
    // the float32 value, so the K-step yields it exactly and the scores equal those of the
    // accumulator-input form bit for bit, while the 32 registers of that input are free for the
    // second column block's scores. A non-finite value (padded queries: -inf) goes whole into
    // the first part.
    const float nl = nlq[nb];
    const bool fin = __builtin_isfinite(nl);
    const bf16 l0 = f32_to_bf16(nl);
    const float r1 = fin ? nl - (float)l0 : 0.f;
    const bf16 l1 = f32_to_bf16(r1);
    const bf16 l2 = f32_to_bf16(r1 - (float)l1);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      lext[nb][j] = half != 0 ? (bf16)0.0f : (j == 0 ? l0 : (j == 1 ? l1 : (j == 2 ? l2 : (bf16)0.0f)));
  }

  // acc_dqp: as acc_dkp in dkv (16x16 tiles at KP = 1)
  f32x16 acc_dq[2], acc_dqp[2], cl[2];
  f32x4 acc_dqp16[2][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc_dq[nb][i] = 0.f; acc_dqp[nb][i] = 0.f; if (!kDext) cl[nb][i] = nlq[nb]; }
    acc_dqp16[nb][0] = acc_dqp16[nb][1] = f32x4(0.f);
  }

  // key tiles reach LDS by DMA (buffer_load ... lds), three tiles ahead
  const int pos_bytes = n_rows * rp * 2;
  const DmaSrc src[3] = {kr.dma(), {kp, pos_bytes, rp * 2, kTile * rp * 2}, vr.dma()};
  TileDma<L.kParts, L.slots()> dma;
  tile_dma_init<LP>(dma, src, wave, lane);

  const int nkt = (N + kTile - 1) / kTile;
  constexpr int kAhead = kBufsDq - 1;
#pragma unroll
  for (int i = 0; i < kAhead; ++i) tile_dma_issue<LP>(dma, wave, min(i, nkt - 1), sT[i]);
  tile_dma_wait<LP, kAhead - 1>(wave);
  __syncthreads();
  for (int t = 0; t < nkt; ++t) {
    // tile t + kAhead (the last tile again past the end) into the buffer tile t - 1 used
    tile_dma_issue<LP>(dma, wave, min(t + kAhead, nkt - 1), sT[(t + kAhead) % kBufsDq]);
    const u32x4* T = sT[t % kBufsDq];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int row = sub * 32 + l32;
      bf16x8 ka[C::kSteps], va[2], kta[2], kpta[2];
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s)
        ka[s] = s < 2 ? lds_frag(&T[oKc + row * C::kCRow + 2 * s + half])
                      : lds_frag(&T[oKp + row * C::kPRow + 2 * (s - 2) + half]);
      const int ch0 = 16 * ((lane >> 4) & 1);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        va[s] = lds_frag(&T[oV + row * C::kCRow + 2 * s + half]);
        const int r0 = sub * 32 + s * 16 + 4 * half;
        kta[s] = tr_frag(&T[oKc], C::kCRow, r0, ch0, lane);
        if constexpr (KP == 2) kpta[s] = tr_frag(&T[oKp], C::kPRow, r0, ch0, lane);
      }
      if constexpr (KP == 1) {
        const int c = pos16_chunk(lane);
        kpta[0] = tr_frag(&T[oKp], C::kPRow, sub * 32 + 16 * (c >> 1) + 4 * (c & 1), 0, lane);
      }
      // scores and dP of both column blocks first, so the vector work of block 0 runs while
      // block 1's MFMAs are in the matrix pipe
      f32x16 scs[2], dps[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        // one query per lane: KP = 1, -LSE2 through an extra score K-step (ones x its three
        // bf16 parts) and -D through the third dP K-step; KP = 2, -LSE2 as the accumulator input
        f32x16 sc = kDext ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(kone, lext[nb], f32x16(0.f), 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[nb][0], cl[nb], 0, 0, 0);
#pragma unroll
        for (int s = kDext ? 0 : 1; s < C::kSteps; ++s)
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qf[nb][s], sc, 0, 0, 0);
        f32x16 dp = kDext ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(vone, dext[nb], f32x16(0.f), 0, 0, 0)
                          : f32x16(0.f);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[0], df[nb][0], dp, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[1], df[nb][1], dp, 0, 0, 0);
        scs[nb] = sc;
        dps[nb] = dp;
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const f32x16 sc = scs[nb], dp = dps[nb];
        bf16x8 sb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int v = 8 * s + j;
            sb[s][j] = f32_to_bf16(__builtin_amdgcn_exp2f(sc[v]) * (kDext ? dp[v] : dp[v] + ndq[nb]));
          }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          acc_dq[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kta[s], sb[s], acc_dq[nb], 0, 0, 0);
          if constexpr (KP == 2)
            acc_dqp[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kpta[s], sb[s], acc_dqp[nb], 0, 0, 0);
        }
        if constexpr (KP == 1) {
          bf16x8 b16[2];
          pos16_b(sb, b16);
#pragma unroll
          for (int m = 0; m < 2; ++m)
            acc_dqp16[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kpta[0], b16[m], acc_dqp16[nb][m], 0, 0, 0);
        }
      }
    }
    tile_dma_wait<LP, kAhead - 1>(wave);   // tile t + 1 landed (this wave's part); later ones may be in flight
    barrier_dma();
  }

  // dQ_c rows go straight to the [B, H, W, heads, 32] map
  const int64_t map_base = make_pixel_map(g).pixel_head(unit, 0) * 32;
  const int64_t row_elems = (int64_t)g.W * g.heads * 32, pix_elems = (int64_t)g.heads * 32;
  bf16* dqm = (bf16*)a.dq_map;
  float* dqp = a.dqp_part + ub * rp;
  const float scale = a.scale;
  {
    static_assert(4 * 64 * kStageRow <= kBufsDq * L.chunks(), "staging fits the tile ring");
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __syncthreads();
    bf16* stage = (bf16*)&sT[0][0] + wave * 64 * kStageRow * 8;
    auto row_of = [&](int t) { return map_base + (int64_t)(t / g.w) * row_elems + (int64_t)(t % g.w) * pix_elems; };
    stage_store_rows(stage, dqm, q0, N, lane, row_of, [&](int nb, int v) { return acc_dq[nb][v] * scale; });
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int q = q0 + nb * 32 + l32;
    if (q >= N) continue;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int ch = 8 * gq + 4 * half;
      if (KP == 2) {
        f32x4 p4;
#pragma unroll
        for (int i = 0; i < 4; ++i) p4[i] = acc_dqp[nb][4 * gq + i] * scale;
        *(f32x4*)(dqp + (int64_t)q * rp + ch) = p4;
      }
    }
  }
  if constexpr (KP == 1) {
    // 16x16 tiles: lane holds channels 4 (lane / 16) + i of query 16 m + lane % 16 of the block
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int q = q0 + nb * 32 + 16 * m + (lane & 15);
        if (q < N) *(f32x4*)(dqp + (int64_t)q * rp + 4 * (lane >> 4)) = acc_dqp16[nb][m] * scale;
      }
  }
}

// ------------------------------------------------------------------ prep
// D_i = sum_c dO_ic O_ic and LSE2_i = LSE_i * log2(e) per window row, for the simple
// kernels (the bf16 MFMA path takes them negated from its one-pass gather).
// Up to four lanes share a row, each reading 16-byte chunks (a group of lanes covers
// 64 contiguous bytes per load), and the partial dot products meet by lane shuffles.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(Geom g, PixelMap pm, const T* __restrict__ o,
                                                       const T* __restrict__ d_o, const float* __restrict__ lse,
                                                       float* __restrict__ dd, float* __restrict__ lse2) {
  constexpr int kEl = 16 / (int)sizeof(T);     // elements per 16-byte chunk
  constexpr int kCpr = D / kEl;                // chunks per row
  constexpr int kL = kCpr < 4 ? kCpr : 4;      // lanes per row
  constexpr int kCpl = kCpr / kL;              // chunks per lane
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kL;
  const int sub = threadIdx.x % kL;
  const int64_t total = (int64_t)g.units * g.n_rows;
  if (i >= total) return;   // the kL lanes of a row leave together
  const int unit = (int)(i / g.n_rows);
  const int t = (int)(i - (int64_t)unit * g.n_rows);
  if (t >= g.N) {
    if (sub == 0) {
      dd[i] = 0.f;
      lse2[i] = INFINITY;   // P = 0 for padded rows
    }
    return;
  }
  const int64_t ph = pm.pixel_head(unit, t);
  const u32x4* orow = (const u32x4*)(o + ph * D);
  const u32x4* grow = (const u32x4*)(d_o + ph * D);
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kCpl; ++j) {
    const u32x4 ov = orow[sub + kL * j], gv = grow[sub + kL * j];
    if constexpr (sizeof(T) == 2) {
      const bf16x8 oe = __builtin_bit_cast(bf16x8, ov), ge = __builtin_bit_cast(bf16x8, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)oe[e], (float)ge[e], acc);
    } else {
      const f32x4 oe = __builtin_bit_cast(f32x4, ov), ge = __builtin_bit_cast(f32x4, gv);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(oe[e], ge[e], acc);
    }
  }
#pragma unroll
  for (int m = 1; m < kL; m <<= 1) acc += __shfl_xor(acc, m);
  if (sub == 0) {
    dd[i] = acc;
    lse2[i] = lse[ph] * 1.44269504088896340736f;
  }
}

// ------------------------------------------------------------------ simple kernels
// float32 arithmetic on T (float or bf16) rows with D content channels: float32
// runs and content widths the MFMA kernels do not cover (d_c = 64).
// dK, dV: SPLIT threads per key (1 at d_c = 32; 2 at d_c = 64, each owning half of the
// channels, so the key's registers fit without spilling), query tiles of 64 in LDS.
template <typename T, int D, int RP>
__global__ __launch_bounds__(256) void attn_bwd_dkv_simple_kernel(BwdArgs a) {
  constexpr int DH = D + RP;
  constexpr int SPLIT = D > 32 ? 2 : 1;
  constexpr int DS = D / SPLIT, RS = RP / SPLIT;   // this thread's content / positional channels
  constexpr int KPB = 256 / SPLIT;                  // keys per block
  __shared__ float sQ[kTile][DH + 1];
  __shared__ float sDo[kTile][D + 1];
  __shared__ float sL[kTile], sD[kTile];
  const Geom& g = a.g;
  const int N = g.N, n_rows = g.n_rows;
  const int nkb = (N + KPB - 1) / KPB;
  const int unit = blockIdx.x / nkb;
  const int key = (blockIdx.x - unit * nkb) * KPB + threadIdx.x / SPLIT;
  const int part = threadIdx.x % SPLIT;
  const int c0 = part * DS, p0 = part * RS;         // first content / positional channel of this thread
  const int64_t ub = (int64_t)unit * n_rows;
  const T* qw = (const T*)a.qw + ub * D;
  const T* dow = (const T*)a.dow + ub * D;
  const T* qp = (const T*)a.qp;
  const int kk = key < N ? key : 0;
  float kc[DS], kpv[RS], vv[DS], gk[DS], gkp[RS], gv[DS];
#pragma unroll
  for (int i = 0; i < DS; ++i) {
    kc[i] = (float)((const T*)a.kw)[(ub + kk) * D + c0 + i];
    vv[i] = (float)((const T*)a.vw)[(ub + kk) * D + c0 + i];
    gk[i] = 0.f;
    gv[i] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < RS; ++i) {
    kpv[i] = (float)((const T*)a.kp)[(int64_t)kk * RP + p0 + i];
    gkp[i] = 0.f;
  }
  const float c = a.c;
  const int nqt = (N + kTile - 1) / kTile;
  for (int t = 0; t < nqt; ++t) {
    const int q0 = t * kTile;
    for (int i = threadIdx.x; i < kTile * DH; i += 256) {
      int r = i / DH, ch = i - r * DH;
      sQ[r][ch] = (float)(ch < D ? qw[(int64_t)(q0 + r) * D + ch] : qp[(int64_t)(q0 + r) * RP + ch - D]);
    }
    for (int i = threadIdx.x; i < kTile * D; i += 256) {
      int r = i / D, ch = i - r * D;
      sDo[r][ch] = (float)dow[(int64_t)(q0 + r) * D + ch];
    }
    if (threadIdx.x < kTile) {
      sL[threadIdx.x] = a.lse2[ub + q0 + threadIdx.x];
      sD[threadIdx.x] = a.dd[ub + q0 + threadIdx.x];
    }
    __syncthreads();
    for (int r = 0; r < kTile; ++r) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < DS; ++i) {
        s = fmaf(sQ[r][c0 + i], kc[i], s);
        dp = fmaf(sDo[r][c0 + i], vv[i], dp);
      }
#pragma unroll
      for (int i = 0; i < RS; ++i) s = fmaf(sQ[r][D + p0 + i], kpv[i], s);
      if constexpr (SPLIT == 2) {   // the key's two threads are adjacent lanes
        s += __shfl_xor(s, 1);
        dp += __shfl_xor(dp, 1);
      }
      const float p = exp2f(fmaf(s, c, -sL[r]));
      const float ds = p * (dp - sD[r]);
#pragma unroll
      for (int i = 0; i < DS; ++i) {
        gv[i] = fmaf(p, sDo[r][c0 + i], gv[i]);
        gk[i] = fmaf(ds, sQ[r][c0 + i], gk[i]);
      }
#pragma unroll
      for (int i = 0; i < RS; ++i) gkp[i] = fmaf(ds, sQ[r][D + p0 + i], gkp[i]);
    }
    __syncthreads();
  }
  if (key < N) {
    T* dkw = (T*)a.dkw + (ub + key) * D + c0;
    T* dvw = (T*)a.dvw + (ub + key) * D + c0;
#pragma unroll
    for (int i = 0; i < DS; ++i) {
      dkw[i] = (T)(gk[i] * a.scale);
      dvw[i] = (T)gv[i];
    }
#pragma unroll
    for (int i = 0; i < RS; ++i) a.dkp_part[(ub + key) * RP + p0 + i] = gkp[i] * a.scale;
  }
}

// dQ: one thread per query, key tiles of 64 in LDS.
template <typename T, int D, int RP>
__global__ __launch_bounds__(256) void attn_bwd_dq_simple_kernel(BwdArgs a) {
  constexpr int DH = D + RP;
  __shared__ float sK[kTile][DH + 1];
  __shared__ float sV[kTile][D + 1];
  const Geom& g = a.g;
  const int N = g.N, n_rows = g.n_rows;
  const int nqb = (N + 255) / 256;
  const int unit = blockIdx.x / nqb;
  const int q = (blockIdx.x - unit * nqb) * 256 + threadIdx.x;
  const int64_t ub = (int64_t)unit * n_rows;
  const T* kw = (const T*)a.kw + ub * D;
  const T* vw = (const T*)a.vw + ub * D;
  const T* kp = (const T*)a.kp;
  const int qq = q < N ? q : 0;
  float qh[DH], gd[D], gq[DH];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qh[i] = (float)((const T*)a.qw)[(ub + qq) * D + i];
    gd[i] = (float)((const T*)a.dow)[(ub + qq) * D + i];
  }
#pragma unroll
  for (int i = 0; i < RP; ++i) qh[D + i] = (float)((const T*)a.qp)[(int64_t)qq * RP + i];
#pragma unroll
  for (int i = 0; i < DH; ++i) gq[i] = 0.f;
  const float l2 = a.lse2[ub + qq], dq_d = a.dd[ub + qq];
  const float c = a.c;
  const int nkt = (N + kTile - 1) / kTile;
  for (int t = 0; t < nkt; ++t) {
    const int k0 = t * kTile;
    for (int i = threadIdx.x; i < kTile * DH; i += 256) {
      int r = i / DH, ch = i - r * DH;
      sK[r][ch] = (float)(ch < D ? kw[(int64_t)(k0 + r) * D + ch] : kp[(int64_t)(k0 + r) * RP + ch - D]);
    }
    for (int i = threadIdx.x; i < kTile * D; i += 256) {
      int r = i / D, ch = i - r * D;
      sV[r][ch] = (float)vw[(int64_t)(k0 + r) * D + ch];
    }
    __syncthreads();
    const int nk = min(kTile, N - k0);
    for (int r = 0; r < nk; ++r) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < DH; ++i) s = fmaf(qh[i], sK[r][i], s);
#pragma unroll
      for (int i = 0; i < D; ++i) dp = fmaf(gd[i], sV[r][i], dp);
      const float p = exp2f(fmaf(s, c, -l2));
      const float ds = p * (dp - dq_d);
#pragma unroll
      for (int i = 0; i < DH; ++i) gq[i] = fmaf(ds, sK[r][i], gq[i]);
    }
    __syncthreads();
  }
  if (q < N) {
    T* dqw = (T*)a.dqw + (ub + q) * D;
#pragma unroll
    for (int i = 0; i < D; ++i) dqw[i] = (T)(gq[i] * a.scale);
#pragma unroll
    for (int i = 0; i < RP; ++i) a.dqp_part[(ub + q) * RP + i] = gq[D + i] * a.scale;
  }
}

// ------------------------------------------------------------------ reduction
// out[t][j] = sum over units (in unit order, per slice) of part[u][t][j]; 8 unit
// slices per column are combined in slice order: a fixed summation order.
__global__ __launch_bounds__(256) void reduce_pos_grads_kernel(int units, int N, int n_rows, int r, int rp,
                                                               const float* __restrict__ part_q,
                                                               float* __restrict__ out_q,
                                                               const float* __restrict__ part_k,
                                                               float* __restrict__ out_k) {
  __shared__ float red[8][32];
  // blockIdx.y: 0 reduces the dQ_p partials, 1 the dK_p partials
  const float* part = blockIdx.y ? part_k : part_q;
  float* out = blockIdx.y ? out_k : out_q;
  const int col = blockIdx.x * 32 + (threadIdx.x & 31);
  const int slice = threadIdx.x >> 5;
  const int ncols = N * rp;
  // slice k adds units k, k + 8, k + 16, ... in that order; the loads are fetched eight at a time
  // so that they overlap (thousands of units at small windows)
  float acc = 0.f;
  if (col < ncols) {
    const int64_t stride = (int64_t)n_rows * rp;
    int u = slice;
    for (; u + 56 < units; u += 64) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = part[(int64_t)(u + 8 * i) * stride + col];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += v[i];
    }
    for (; u < units; u += 8) acc += part[(int64_t)u * stride + col];
  }
  red[slice][threadIdx.x & 31] = acc;
  __syncthreads();
  if (slice == 0 && col < ncols) {
    float s = red[0][threadIdx.x];
#pragma unroll
    for (int k = 1; k < 8; ++k) s += red[k][threadIdx.x];
    const int t = col / rp, j = col - t * rp;
    if (j < r) out[(int64_t)t * r + j] = s;
  }
}

}  // namespace

hipError_t launch_bwd_prep(const Geom& g, int esize, const void* o, const void* d_o, const float* lse, float* dd,
                           float* lse2, hipStream_t stream) {
  const int64_t total = (int64_t)g.units * g.n_rows;
  if (total == 0) return hipSuccess;
  const PixelMap pm = make_pixel_map(g);
  // lanes per row: min(4, 16-byte chunks per row), as in the kernel
  const int lanes = std::min(4, g.d_c * esize / 16);
  const dim3 grid((unsigned)((total * lanes + 255) / 256)), block(256);
#define RIB_PREP(T, D) \
  hipLaunchKernelGGL((bwd_prep_kernel<T, D>), grid, block, 0, stream, g, pm, (const T*)o, (const T*)d_o, lse, dd, lse2)
  if (esize == 2) {
    if (g.d_c == 32) RIB_PREP(bf16, 32); else RIB_PREP(bf16, 64);
  } else {
    if (g.d_c == 32) RIB_PREP(float, 32); else RIB_PREP(float, 64);
  }
#undef RIB_PREP
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkv_bf16(const BwdArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.g.units * ((a.g.N + kPerBlock - 1) / kPerBlock);
  if (blocks == 0) return hipSuccess;
  if (a.rp == 16 && a.k_map) hipLaunchKernelGGL((attn_bwd_dkv_kernel<1, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else if (a.rp == 16) hipLaunchKernelGGL(attn_bwd_dkv_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(attn_bwd_dkv_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dq_bf16(const BwdArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.g.units * ((a.g.N + kPerBlock - 1) / kPerBlock);
  if (blocks == 0) return hipSuccess;
  if (a.rp == 16 && a.k_map) hipLaunchKernelGGL((attn_bwd_dq_kernel<1, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else if (a.rp == 16) hipLaunchKernelGGL(attn_bwd_dq_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(attn_bwd_dq_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

#define RIB_BWD_SIMPLE(K, T, D, RP) \
  hipLaunchKernelGGL((K<T, D, RP>), dim3((unsigned)blocks), dim3(256), 0, stream, a)
#define RIB_BWD_SIMPLE_ALL(K)                                                                              \
  do {                                                                                                     \
    if (esize == 4) {                                                                                      \
      if (a.g.d_c == 32) { if (a.rp == 16) RIB_BWD_SIMPLE(K, float, 32, 16); else RIB_BWD_SIMPLE(K, float, 32, 32); } \
      else { if (a.rp == 16) RIB_BWD_SIMPLE(K, float, 64, 16); else RIB_BWD_SIMPLE(K, float, 64, 32); }                \
    } else {                                                                                               \
      if (a.g.d_c == 32) { if (a.rp == 16) RIB_BWD_SIMPLE(K, bf16, 32, 16); else RIB_BWD_SIMPLE(K, bf16, 32, 32); }    \
      else { if (a.rp == 16) RIB_BWD_SIMPLE(K, bf16, 64, 16); else RIB_BWD_SIMPLE(K, bf16, 64, 32); }                  \
    }                                                                                                      \
  } while (0)

hipError_t launch_attn_bwd_dkv_simple(const BwdArgs& a, int esize, hipStream_t stream) {
  const int kpb = a.g.d_c > 32 ? 128 : 256;   // keys per block (two threads per key at d_c = 64)
  const int64_t blocks = (int64_t)a.g.units * ((a.g.N + kpb - 1) / kpb);
  if (blocks == 0) return hipSuccess;
  RIB_BWD_SIMPLE_ALL(attn_bwd_dkv_simple_kernel);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dq_simple(const BwdArgs& a, int esize, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.g.units * ((a.g.N + 255) / 256);
  if (blocks == 0) return hipSuccess;
  RIB_BWD_SIMPLE_ALL(attn_bwd_dq_simple_kernel);
  return hipGetLastError();
}
#undef RIB_BWD_SIMPLE_ALL
#undef RIB_BWD_SIMPLE

hipError_t launch_reduce_pos_grads(int units, int N, int n_rows, int r, int rp, const float* part_q, float* out_q,
                                   const float* part_k, float* out_k, hipStream_t stream) {
  const int ncols = N * rp;
  hipLaunchKernelGGL(reduce_pos_grads_kernel, dim3((ncols + 31) / 32, 2), dim3(256), 0, stream, units, N, n_rows, r,
                     rp, part_q, out_q, part_k, out_k);
  return hipGetLastError();
}

}  // namespace rib
