// RIB window attention, forward, for gfx950.
//
// O = softmax(scale * [Q_c | Q_p][K_c | K_p]^T) V per (batch, window, head)
// unit: the positional tokens are appended channel-wise to the content tokens
// so the positional bias is part of one dot product and no N x N bias (or
// score) matrix is ever stored (gist.science/paper/2603.06738, "Technical
// Summary" §2.A.3-4, "Content + Bias" equation; khansong-paper-with-me.hf.space
// abstract).
//
// bf16 kernel design (CDNA4, wave64, v_mfma_f32_32x32x16_bf16):
//  * The score tile is computed transposed, S^T = K_hat Q'^T: keys are the
//    MFMA rows, queries the columns, so every lane owns one query and holds 16
//    of its scores.
//  * The concatenation is virtual: the contraction runs over two 16-channel
//    content steps (d_c = 32) and one or two 16-channel positional steps
//    (r padded to 16 / 32 with zeros), K_c and K_p staged side by side in LDS.
//  * Q' = bf16(scale * log2(e) * [Q_c | Q_p]) so scores come out in the log2
//    domain and P = exp2(S' - m) needs no multiply.
//  * O^T = V^T P^T: P leaves the score accumulator directly as the B operand.
//    The accumulator holds, for half h of the wave, keys 8(v/4) + 4h + v%4;
//    V^T is stored with tokens permuted inside every 16-token group (bits 2
//    and 3 of the token index swapped) so each lane's eight keys are one
//    contiguous 16-byte LDS read.
//  * Fast pass (no running max): by Cauchy-Schwarz every score of query i is
//    at most m_i = |q'_i| * max_j |k_hat_j|, so P = exp2(S' - m_i) <= 1 never
//    overflows and needs no rescaling. The subtraction is free: the score
//    MFMA accumulates onto a constant -m_i. The row sums go to the matrix
//    pipe too: a v_mfma_f32_16x16x32_bf16 of each P block against a 0/1
//    selector sums the exact bf16 P values the PV MFMA consumes (dot2 would
//    occupy the matrix pipe anyway and fp32 adds cost more vector issue).
//    Per score the vector work is one exp2 and half a pack.
//  * Exact pass (fallback): if some row sum of a workgroup came out below
//    2^-60 (the bound overshot so far that small terms could underflow) or is
//    not finite, the workgroup recomputes its rows with the classic online
//    softmax (running max, rescaling when the max grows by more than 2^8).
//  * A workgroup is 4 waves x 64 queries; K and V^T tiles of 64 keys are
//    shared by the 4 waves through a ring of four LDS buffers filled by
//    global-to-LDS DMA (buffer_load ... lds), issued three tiles ahead with
//    fixed per-lane source offsets, so tile staging costs neither VGPRs nor
//    vector instructions. Workgroups of one unit are kept on one XCD (its L2
//    holds the unit's K and V).
//  * Split tail: the items of an XCD past its last whole round of workgroup
//    slots may be cut into 2 or 4 key ranges (chosen by a slot model of the
//    XCD); each piece writes its unnormalized O, row sums and shifts, and
//    fwd_split_combine_kernel adds them in a fixed order into O and LSE.
#include <algorithm>
#include <mutex>

#include "internal.hpp"

namespace rib {
namespace {

constexpr int kWaves = 4;
constexpr int kQPerWave = 64;             // two 32-query MFMA column blocks
constexpr int kKeyTile = 64;
constexpr float kLazyTau = 8.0f;          // log2 units
constexpr float kUnderflowGuard = 8.673617379884035e-19f;  // 2^-60
constexpr int kKeyBoundTile = 64;         // keys per partial key-norm maximum (one per gather block)
// Tiers of the bounded softmax with one positional K-step. P = exp2(S' - s) may reach 2^64
// when every |v| of the unit is at most kNoShiftVMax: the row sums and O accumulators then
// stay below 2^14 * 2^64 * 2^40 < 2^128. So the shift of row i is s_i = max(0, m_i - 64)
// with m_i its score bound; when every s_i of a workgroup is 0, P = exp2(S') needs no shift
// at all and P lies in [2^-64, 2^64] (no underflow either). A row sum can fall below the
// underflow guard only when the bound overshoots the row's largest score by more than
// 124 log2 units. With a larger |v| the shift is the bound itself (P <= 1).
constexpr float kNoShiftMax = 64.0f;
constexpr float kNoShiftVMax = 1099511627776.0f;   // 2^40

// s_waitcnt immediates (gfx9 encoding) waiting on the vector-memory counter
// only: vmcnt in bits 3:0, expcnt (7) and lgkmcnt (15) left at their maxima.
constexpr int kVmcntOnly = 0x0F70;
constexpr int kVmcnt0 = kVmcntOnly | 0;
constexpr int kVmcnt1 = kVmcntOnly | 1;
constexpr int kVmcnt2 = kVmcntOnly | 2;
constexpr int kVmcnt3 = kVmcntOnly | 3;
constexpr int kVmcnt4 = kVmcntOnly | 4;

__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// Workgroup barrier without the release fence of __syncthreads: with tile DMA
// in flight that fence waits for every outstanding vector-memory load, which
// would cap the DMA lead at one tile. Callers wait explicitly for the DMA they
// depend on; the waves write no LDS themselves. The memory clobber keeps the
// compiler from moving LDS reads or DMA issue across it.
__device__ __forceinline__ void barrier_dma() { asm volatile("s_barrier" ::: "memory"); }

// Keeps x in VGPRs at this point of the instruction stream. Between two pins the compiler
// cannot move the instruction that consumes or produces x: the fast pass uses pairs of pins
// to fix the issue order of every MFMA, exp and pack (a wave issues in order, so the
// order decides how well its matrix and vector work overlap). Emits no instruction.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// KP: positional 16-channel steps, 1 (r <= 16) or 2 (r <= 32); 0 with RPB:
// the relative-position-bias comparison variant (content-only scores plus a
// bias gathered from a per-head table).
template <int KP, bool RPB = false>
struct FwdCfg {
  static_assert(!RPB || KP == 0, "the RPB variant has no positional channels");
  static constexpr int kSteps = 2 + KP;             // MFMA K-steps of the score
  // One LDS tile buffer, in 16-byte chunks: K_c [64 keys][4 + 1 pad], then
  // K_p [64 keys][2KP + 1 pad], then V^T [32 channels][8 + 1 pad] (padded to
  // whole DMA instructions), then (RPB) the 64 keys' table byte offsets. The
  // odd row strides keep the fragment reads free of bank conflicts.
  static constexpr int kKcRow = 5;
  static constexpr int kKpRow = KP ? 2 * KP + 1 : 0;
  static constexpr int kVRow = kKeyTile / 8 + 1;
  static constexpr int kKcOff = 0;
  static constexpr int kKpOff = kKcOff + kKeyTile * kKcRow;
  static constexpr int kVOff = kKpOff + kKeyTile * kKpRow;
  static constexpr int kKcDma = kKeyTile * kKcRow / 64;          // DMA instructions per tile part
  static constexpr int kKpDma = kKeyTile * kKpRow / 64;
  static constexpr int kVDma = (32 * kVRow + 63) / 64;
  static constexpr int kIdxOff = kVOff + 64 * kVDma;
  static constexpr int kIdxDma = RPB ? 1 : 0;                   // 64 int32 = 16 chunks (+48 zeroed)
  static constexpr int kDma = kKcDma + kKpDma + kVDma + kIdxDma;
  static constexpr int kChunks = kIdxOff + 64 * kIdxDma;
  // waves per workgroup: the RPB table fills most of a CU's LDS, so its
  // workgroups are twice as wide to keep two waves per SIMD
  static constexpr int kWv = RPB ? 2 * kWaves : kWaves;
  static constexpr int kQPerBlock = kWv * kQPerWave;
  static_assert(kKeyTile * kKcRow % 64 == 0 && kKeyTile * kKpRow % 64 == 0, "whole DMA instructions");
  static_assert(kDma <= 4 * kWv && kDma >= kWv, "one to four DMA instructions per wave and tile");
};
constexpr int kBufs = 4;                  // LDS tile ring depth
// word 3 of a raw buffer resource on gfx9-class parts (32-bit data format)
constexpr int kRsrcWord3 = 0x00020000;

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4v;

template <bool V>
struct BoolTag {
  static constexpr bool value = V;
};

// GATE: O' = O * G with G read in the map layout by the output stage.
// MAPKV (one positional K-step, windows whose side divides 64: a 64-key tile is 64 / w whole
// window rows): K_c and V tiles reach LDS by DMA straight from the [B, H, W, heads, 32] maps,
// both token-major; the PV MFMA's channel-major V^T fragments come from transposing LDS reads
// (ds_read_b64_tr_b16). No gather runs and no key-norm bound exists: the fast pass takes
// P = exp2(S') unshifted and the exact pass reruns a workgroup whose row sums or accumulators
// came out non-finite or below the underflow guard.
template <int KP, bool RPB = false, bool GATE = false, bool MAPKV = false>
__global__ __launch_bounds__(RPB ? 512 : 256, RPB ? 1 : 2) void attn_fwd_bf16_kernel(FwdArgs a) {
  typedef FwdCfg<KP, RPB> C;
  // Ring of kBufs tile buffers. While tile t is processed, tiles t and t + 1
  // are read (V^T of t, K of t and, prefetched, of t + 1) and the DMA for
  // tile t + 3 fills the buffer tile t - 1 used; tile t + 2 must have landed
  // by the end of tile t. Each DMA thus has two tiles of compute to arrive.
  __shared__ u32x4 sT[kBufs][C::kChunks];

  const Geom& g = a.g;
  const int N = g.N, n_rows = g.n_rows;
  const int nqb = (N + C::kQPerBlock - 1) / C::kQPerBlock;
  const int total = g.units * nqb;
  const int nkt = (N + kKeyTile - 1) / kKeyTile;
  // Work item and key-tile range. Items are numbered so that consecutive ones share an
  // XCD (the hardware deals workgroups to the 8 XCDs in turn). With a split tail, the
  // items of an XCD past its last whole round of slots are cut into split_s key ranges
  // (pieces), dealt to that XCD after its whole items; trailing padding blocks exit.
  int logical, t0 = 0, t1 = nkt, piece = -1;
  if (RPB || a.split_spx == 0) {
    logical = xcd_remap(blockIdx.x, total);
  } else {
    const int xcd = blockIdx.x % 8, i = blockIdx.x / 8;
    const int q8 = total / 8, rem = total % 8;
    const int n_x = q8 + (xcd < rem ? 1 : 0);
    const int base = xcd < rem ? xcd * (q8 + 1) : rem * (q8 + 1) + (xcd - rem) * q8;
    const int full = n_x / a.split_spx * a.split_spx;
    if (i < full) {
      logical = base + i;
    } else {
      const int j = i - full, k = j / a.split_s, r = j - k * a.split_s;
      if (k >= n_x - full) return;   // padding block
      logical = base + full + k;
      t0 = r * nkt / a.split_s;
      t1 = (r + 1) * nkt / a.split_s;
      piece = (xcd * a.split_tail_max + k) * a.split_s + r;
    }
  }
  const int unit = logical / nqb;
  const int qb = logical - unit * nqb;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int rp = 16 * KP;

  // Q_c rows are read and O rows written straight in the [B, H, W, heads, d_c]
  // map: the window addressing is folded into these once-per-wave accesses
  // (row of token t = window base + (t / w) * W * heads + (t % w) * heads).
  const PixelMap pm = make_pixel_map(g);
  const int64_t map_base = pm.pixel_head(unit, 0) * 32;
  const int64_t row_elems = (int64_t)g.W * g.heads * 32, pix_elems = (int64_t)g.heads * 32;
  auto map_row = [&](int t) { return map_base + (int64_t)(t / g.w) * row_elems + (int64_t)(t % g.w) * pix_elems; };
  const bf16* qmap = (const bf16*)a.q_map;
  static_assert(!MAPKV || (KP == 1 && !RPB), "map-addressed K / V: one positional K-step only");
  // map-addressed tiles: key k of a tile sits at (k / w) window rows and (k % w) pixels from the
  // tile's first key, and tile t starts t * (64 / w) window rows below the window's first row
  const int row_bytes = g.W * g.heads * 64, pix_bytes = g.heads * 64;
  const int tile_step = MAPKV ? (kKeyTile / g.w) * row_bytes : 0;
  const bf16* kw = MAPKV ? (const bf16*)a.k_map + map_base : (const bf16*)a.kw + (int64_t)unit * n_rows * 32;
  const bf16* vt = MAPKV ? (const bf16*)a.v_map + map_base : (const bf16*)a.vw + (int64_t)unit * 32 * n_rows;
  // bytes from the window's first pixel-head row to the end of its last one
  const int span_bytes = MAPKV ? (g.w - 1) * row_bytes + (g.w - 1) * pix_bytes + 64 : n_rows * 64;
  const bf16* qp = (const bf16*)a.qp;
  const bf16* kp = (const bf16*)a.kp;
  const float c = a.c;

  // ---- per-unit key-norm bound: max over the partial maxima of the unit
  const int nkparts = (N + kKeyBoundTile - 1) / kKeyBoundTile;
  float km = 0.f, vm = 0.f;
  for (int i = lane; !MAPKV && i < nkparts; i += 64) {
    km = fmaxf(km, a.kmax2[(int64_t)unit * nkparts + i]);
    vm = fmaxf(vm, a.kmax2[((int64_t)g.units + unit) * nkparts + i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    km = fmaxf(km, __shfl_xor(km, o));
    vm = fmaxf(vm, __shfl_xor(vm, o));
  }
  const float kmax = sqrtf(km);

  // ---- RPB: the head's table, prepared in fp16 log2 units (entries padded to
  // whole 1 KiB DMA blocks), is copied into LDS by DMA before the first tile;
  // its maximum joins the softmax bound.
  extern __shared__ _Float16 sTab[];
  float bmax = 0.f;
  if constexpr (RPB) {
    const int head = unit % g.heads;
    const int tblocks = a.rpb_stride / 512;
    const _Float16* tab = a.rpb_tab16 + (int64_t)head * a.rpb_stride;
    const __amdgpu_buffer_rsrc_t rs_t = __builtin_amdgcn_make_buffer_rsrc((void*)tab, 0, a.rpb_stride * 2, kRsrcWord3);
    for (int i = wave; i < tblocks; i += C::kWv)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_t, (__attribute__((address_space(3))) void*)&sTab[512 * i], 16,
                                               lane * 16 + i * 1024, 0, 0, 0);
    bmax = a.rpb_max[head];
  }

  // ---- query fragments (B operand), pre-scaled into the log2 domain
  const int q0 = qb * C::kQPerBlock + wave * kQPerWave;
  bf16x8 qf[2][C::kSteps];
  float mref[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int q = q0 + nb * 32 + l32;
    const bool ok = q < N;
    float sq = 0.f;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      u32x4 v = u32x4(0u);
      if (ok) {
        if (s < 2) v = *(const u32x4*)(qmap + map_row(q) + s * 16 + half * 8);
        else v = *(const u32x4*)(qp + (int64_t)q * rp + (s - 2) * 16 + half * 8);
      }
      const bf16x8 raw = __builtin_bit_cast(bf16x8, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16 e = f32_to_bf16((float)raw[j] * c);
        qf[nb][s][j] = e;
        sq = fmaf((float)e, (float)e, sq);
      }
    }
    sq += swap_halves(sq);
    mref[nb] = sqrtf(sq) * kmax + bmax;
  }
  // RPB: the bias of query q and key k is table[(w-1)(2w-1) + (w-1) + QI(q) - QI(k)] with
  // QI(t) = (t / w)(2w-1) + t % w. Per column block the lane keeps the LDS byte address of
  // its query's part; the key part arrives with every tile as the byte offset -2 QI(k)
  // (0 for padded keys, which are masked).
  unsigned tab_base[2] = {0u, 0u};
  if constexpr (RPB) {
    const int w2 = 2 * g.w - 1;
    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)sTab;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int q = min(q0 + nb * 32 + l32, N - 1);
      const int qi = (q / g.w) * w2 + q % g.w;
      tab_base[nb] = lds0 + 2u * (unsigned)((g.w - 1) * w2 + (g.w - 1) + qi);
    }
  }

  // ---- tile DMA: buffer_load ... lds writes lane l's 16 bytes to chunk l of
  // the 64-chunk block its LDS base names. Instruction i of a tile fills
  // chunks [64 i, 64 i + 64) of the buffer and is issued by wave i % 4; the
  // per-lane source offsets are fixed, only the key offset moves per tile.
  // Pad chunks fetch a duplicate of their row's first chunk.
  const __amdgpu_buffer_rsrc_t rs_kc = __builtin_amdgcn_make_buffer_rsrc((void*)kw, 0, span_bytes, kRsrcWord3);
  // K_p has N rows (rows past N read zero): either the packed copy or the caller's buffer
  const __amdgpu_buffer_rsrc_t rs_kp = __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, N * rp * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc((void*)vt, 0, span_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_i = __builtin_amdgcn_make_buffer_rsrc((void*)a.rpb_kidx, 0, n_rows * 4, kRsrcWord3);
  int dma_off[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int i = C::kWv * jj + wave;
    const int c = 64 * i + lane;
    int off = 0;
    if (i < C::kKcDma) {
      const int r = c / C::kKcRow, k = c % C::kKcRow;
      off = (MAPKV ? (r / g.w) * row_bytes + (r % g.w) * pix_bytes : r * 64) + (k < 4 ? k : 0) * 16;
    } else if (i < C::kKcDma + C::kKpDma) {
      const int c2 = c - C::kKpOff;
      constexpr int kKpRowNz = C::kKpRow ? C::kKpRow : 1;   // no positional part: branch never taken
      const int r = c2 / kKpRowNz, k = c2 % kKpRowNz;
      off = r * rp * 2 + (k < 2 * KP ? k : 0) * 16;
    } else if (i < C::kKcDma + C::kKpDma + C::kVDma) {
      const int c3 = c - C::kVOff;
      if constexpr (MAPKV) {   // token-major V rows laid out as the K_c rows: [64 keys][5 chunks]
        const int r = c3 / C::kKcRow, k = c3 % C::kKcRow;
        off = (r / g.w) * row_bytes + (r % g.w) * pix_bytes + (k < 4 ? k : 0) * 16;
      } else {
        int r = c3 / C::kVRow, k = c3 % C::kVRow;
        if (r >= 32) r = 0, k = 0;
        off = r * n_rows * 2 + (k < 8 ? k : 0) * 16;
      }
    } else {
      off = lane < 16 ? lane * 16 : (int)0x80000000;   // 64 key offsets; the rest of the block reads zeros
    }
    dma_off[jj] = off;
  }
  const int dma_count = (C::kDma - wave + C::kWv - 1) / C::kWv;   // DMA instructions of this wave per tile
  auto dma_tile = [&](int t, int buf) {
    const int k0 = t * kKeyTile;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int i = C::kWv * jj + wave;
      if (i < C::kDma) {
        auto* dst = (__attribute__((address_space(3))) void*)&sT[buf][64 * i];
        if (i < C::kKcDma)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_kc, dst, 16, dma_off[jj] + (MAPKV ? t * tile_step : k0 * 64), 0,
                                                   0, 0);
        else if (i < C::kKcDma + C::kKpDma)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_kp, dst, 16, dma_off[jj] + k0 * rp * 2, 0, 0, 0);
        else if (i < C::kKcDma + C::kKpDma + C::kVDma)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_v, dst, 16, dma_off[jj] + (MAPKV ? t * tile_step : k0 * 2), 0, 0,
                                                   0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_i, dst, 16, dma_off[jj] + k0 * 4, 0, 0, 0);
      }
    }
  };
  // wait until only the newest tile's DMA (of this wave) may be in flight
  auto dma_wait_older = [&]() {
    if (dma_count == 4) __builtin_amdgcn_s_waitcnt(kVmcnt4);
    else if (dma_count == 3) __builtin_amdgcn_s_waitcnt(kVmcnt3);
    else if (dma_count == 2) __builtin_amdgcn_s_waitcnt(kVmcnt2);
    else __builtin_amdgcn_s_waitcnt(kVmcnt1);
  };
  // score fragments of one 32-key subtile
  auto load_kf = [&](int buf, int sub, bf16x8* kf) {
    const int row = sub * 32 + l32;
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      const int ch = s < 2 ? C::kKcOff + row * C::kKcRow + 2 * s + half
                           : C::kKpOff + row * C::kKpRow + 2 * (s - 2) + half;
      kf[s] = __builtin_bit_cast(bf16x8, sT[buf][ch]);
    }
  };
  auto vfrag = [&](int buf, int sub, int s) -> bf16x8 {
    if constexpr (MAPKV) {
      // Transposing LDS read: in each 16-lane group, lane i gets element i & 3 of the 8 bytes
      // read by lanes (i >> 2) + 4j, j = 0..3. Lane si of group G reads key 4 half + (si >> 2)
      // (+ 8 for the second read) at channels 16 (G & 1) + 4 (si & 3) .. + 3, so lane l gets
      // channel l % 32 of keys 4 half + 0..3 and 8 + 4 half + 0..3: the A operand in the key
      // order of the P words (bits 2 and 3 of the key swapped).
      const int si = lane & 15;
      const int key = sub * 32 + s * 16 + 4 * half + (si >> 2);
      const int ch = 16 * ((lane >> 4) & 1) + 4 * (si & 3);
      auto* vb = (__attribute__((address_space(3))) char*)&sT[buf][C::kVOff];
      const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4v*)(vb + key * (16 * C::kKcRow) + ch * 2));
      const bf16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4v*)(vb + (key + 8) * (16 * C::kKcRow) + ch * 2));
      bf16x8 out;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        out[j] = lo[j];
        out[4 + j] = hi[j];
      }
      return out;
    } else {
      return __builtin_bit_cast(bf16x8, sT[buf][C::kVOff + l32 * C::kVRow + 4 * sub + 2 * s + half]);
    }
  };
  // RPB: the log2-domain bias of the lane's 16 accumulator rows (keys 8(v/4) + 4h + v%4 of
  // subtile sub) for both column blocks, gathered from the LDS table ...
  auto gather_bias = [&](int buf, int sub, _Float16 (*bh)[16]) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const u32x4 k4 = sT[buf][C::kIdxOff + (sub * 32 + 8 * g4 + 4 * half) / 4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          bh[nb][4 * g4 + i] = *(const __attribute__((address_space(3))) _Float16*)(size_t)(tab_base[nb] + k4[i]);
    }
  };
  // ... and the score MFMA's accumulator init from it: bias + mneg, -inf for keys >= N
  auto bias_cinit = [&](const _Float16 (*bh)[16], const float* mneg, int key0, f32x16* ci) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) ci[nb][v] = (float)bh[nb][v] + mneg[nb];
    if (key0 + 32 > N) {
      const int kbase = key0 + 4 * half;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (kbase + 8 * (v >> 2) + (v & 3) >= N) ci[0][v] = ci[1][v] = -INFINITY;
    }
  };
  auto mask_tail = [&](f32x16* sc, int key0) {
    const int kbase = key0 + 4 * half;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kbase + 8 * (v >> 2) + (v & 3);
      if (key >= N) { sc[0][v] = -INFINITY; sc[1][v] = -INFINITY; }
    }
  };
  auto pv = [&](int buf, int sub, const bf16x8 (*pf)[2], f32x16* acc) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 vf = vfrag(buf, sub, s);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nb][s], acc[nb], 0, 0, 0);
    }
  };

  f32x16 acc[2];
  float m_run[2], l_run[2];

  // ===== fast pass: fixed per-query bound, software-pipelined over subtiles.
  // Each half step takes the softmax of one 32-key subtile while the score
  // MFMAs of the next subtile and the PV MFMAs of this one run; the source
  // order below (pinned by scheduling fences) alternates one MFMA with a
  // slice of the exp / pack / row-sum work so both pipes stay busy within a
  // wave. Keys past N (last tile only) have zero K rows and zero V^T columns:
  // their P = exp2(-m) adds nothing to O and is subtracted from the row sum.
  // With RPB the accumulator init carries each score's bias too (rebuilt per
  // subtile) and padded keys start at -inf, so their P is zero.
  float pad_sub[2] = {0.f, 0.f};
  // Early exit (one positional K-step): after the range's first two tiles every row's partial
  // sum must already reach the underflow guard; rows whose bound overshoots their scores by
  // more than the guard allows (the case the exact pass exists for) show it there, and the
  // workgroup goes to the exact pass without finishing the fast one. The partial sum is a sum
  // over fewer keys than the final one, so it exits only where the final check could fail too
  // or, for rows whose large scores all lie past the first 128 keys, a little more often.
  bool fast_exit = false;
  if constexpr (KP == 1 && !RPB) {
    // ===== fast pass, one positional K-step. Per 32-key subtile h (a half step) a wave
    // forms 16 P words (2 exp2 + 1 pack each, 32 scores) and issues 14 MFMAs: the six score
    // MFMAs (three K-steps x two 32-query column blocks), four PV MFMAs and four row-sum
    // MFMAs. They are issued in a fixed order of 16 slots, one word and at most one MFMA per
    // slot, so that the wave's in-order issue alternates matrix and vector work:
    //   slot  1- 3: S(s, nb 1) of subtile h        words (0,0,*)   [block (nb, s)]
    //   slot  4: R(1,1) of h-1    5: R(0,0)    6: P(0,0)    7: P(1,1) of h-1   words (0,1,*)
    //   slot  9, 11, 13: S(s, nb 0) of subtile h+1   10: R(1,0)   12: P(1,0)   words (1,0,*)
    //   slot 14: R(0,1)   15: P(0,1)                                           words (1,1,*)
    // The score registers roll: nb 0 scores of h+1 overwrite those of h once their 8 words
    // are formed (slot 9), nb 1 scores are formed at the start of their own half step. The
    // last block's R and P wait for the next half step. K fragments of h+1 are read after
    // slot 3, V^T fragment 1 of h after slot 7 and fragment 0 of h+1 after slot 15.
    const bool small_v = vm <= kNoShiftVMax;
    const bool shift = __syncthreads_or(!(fmaxf(mref[0], mref[1]) <= kNoShiftMax) || !small_v);
    auto fast_pass = [&](auto tier) {
      constexpr bool SH = decltype(tier)::value;
      float msub[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) msub[nb] = !SH ? 0.f : (small_v ? fmaxf(mref[nb] - kNoShiftMax, 0.f) : mref[nb]);
      f32x16 sc[2];
      bf16x8 kf[C::kSteps], vf[2];
      u32x4 wd[2][2];
      f32x4 lsum[2];
      bf16x8 rsel;   // row-sum selector (see below)
      {
        const bf16 one = (lane & 15) == ((lane >> 4) & 1) ? (bf16)1.0f : (bf16)0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) rsel[j] = one;
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        acc[nb] = f32x16(0.f);
        lsum[nb] = f32x4(0.f);
        wd[1][nb] = u32x4(0u);
        m_run[nb] = msub[nb];
      }
      vf[1] = __builtin_bit_cast(bf16x8, u32x4(0u));
      // Row sums on the matrix pipe: v_mfma_f32_16x16x32_bf16 with a 0/1 selector as A. Read
      // as that MFMA's B operand, lane l of a P block holds query l % 16 + 16 * ((l / 16) % 2);
      // the selector puts lane groups 0 and 2 into row 0 and groups 1 and 3 into row 1, so rows
      // 0 and 1 of the 16x16 accumulator (lanes 0-15, elements 0 and 1) collect the sums of the
      // block's queries 0-15 and 16-31 over the exact bf16 P values the PV MFMA consumes.
      auto word_exp = [&](int nb, int s, int w, float& p0, float& p1) {
        float x0 = sc[nb][8 * s + 2 * w], x1 = sc[nb][8 * s + 2 * w + 1];
        if constexpr (SH) {
          x0 -= msub[nb];
          x1 -= msub[nb];
        }
        pin(x0);
        pin(x1);
        p0 = __builtin_amdgcn_exp2f(x0);
        p1 = __builtin_amdgcn_exp2f(x1);
        pin(p0);
        pin(p1);
      };
      auto word_pack = [&](int nb, int s, int w, float p0, float p1) {
        bf16x2 pr;
        pr[0] = f32_to_bf16(p0);
        pr[1] = f32_to_bf16(p1);
        unsigned u = __builtin_bit_cast(unsigned, pr);
        pin(u);
        wd[nb][s][w] = u;
      };
      auto S = [&](int s, int nb) {
        pin(kf[s]);
        sc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[nb][s], s == 0 ? f32x16(0.f) : sc[nb], 0, 0, 0);
        pin(sc[nb]);
      };
      auto R = [&](int s, int nb) {
        pin(lsum[nb]);
        lsum[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rsel, __builtin_bit_cast(bf16x8, wd[nb][s]), lsum[nb],
                                                           0, 0, 0);
        pin(lsum[nb]);
      };
      auto P = [&](int s, int nb) {
        pin(acc[nb]);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s], __builtin_bit_cast(bf16x8, wd[nb][s]), acc[nb], 0,
                                                          0, 0);
        pin(acc[nb]);
      };
      // one slot: the word's two exp2, then the MFMA (if any), then the pack (the MFMA also
      // separates the second exp2 from the pack that reads it)
      auto slot = [&](int nb, int s, int w, auto mfma) {
        float p0, p1;
        word_exp(nb, s, w, p0, p1);
        mfma();
        word_pack(nb, s, w, p0, p1);
      };
      auto none = [] {};
      // half step h: (cbuf, csub) holds subtile h, (nbuf, nsub) subtile h + 1
      auto hstep = [&](int cbuf, int csub, int nbuf, int nsub) {
        slot(0, 0, 0, [&] { S(0, 1); });
        slot(0, 0, 1, [&] { S(1, 1); });
        slot(0, 0, 2, [&] { S(2, 1); });
        load_kf(nbuf, nsub, kf);
        slot(0, 0, 3, [&] { R(1, 1); });
        slot(0, 1, 0, [&] { R(0, 0); });
        slot(0, 1, 1, [&] { P(0, 0); });
        slot(0, 1, 2, [&] { P(1, 1); });
        vf[1] = vfrag(cbuf, csub, 1);
        slot(0, 1, 3, none);
        slot(1, 0, 0, [&] { S(0, 0); });
        slot(1, 0, 1, [&] { R(1, 0); });
        slot(1, 0, 2, [&] { S(1, 0); });
        slot(1, 0, 3, [&] { P(1, 0); });
        slot(1, 1, 0, [&] { S(2, 0); });
        slot(1, 1, 1, [&] { R(0, 1); });
        slot(1, 1, 2, [&] { P(0, 1); });
        vf[0] = vfrag(nbuf, nsub, 0);
        slot(1, 1, 3, none);
      };

      // prologue: tiles t0 and t0 + 1 in LDS, t0 + 2 on its way; nb 0 scores of the first
      // subtile. Tiles past the range repeat its last tile (read only by the unused scores
      // of the subtile after the last). Buffers are numbered from t0. The deferred block of
      // the (nonexistent) previous subtile is zero.
      dma_tile(t0, 0);
      dma_tile(min(t0 + 1, t1 - 1), 1);
      dma_tile(min(t0 + 2, t1 - 1), 2);
      dma_wait_older();
      __syncthreads();
      load_kf(0, 0, kf);
#pragma unroll
      for (int s2 = 0; s2 < C::kSteps; ++s2) S(s2, 0);
      vf[0] = vfrag(0, 0, 0);
      for (int t = t0; t < t1; ++t) {
        const int b0 = (t - t0) % kBufs, b1 = (t - t0 + 1) % kBufs;
        dma_tile(min(t + 3, t1 - 1), (t - t0 + 3) % kBufs);
        hstep(b0, 0, b0, 1);
        hstep(b0, 1, b1, 0);
        dma_wait_older();   // tile t + 2 landed (this wave's part)
        if (t == t0 + 1 && t + 1 < t1) {
          // the partial row sums (the block deferred to the next half step not yet added)
          bool low = false;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const float r0 = __shfl(lsum[nb][0], l32 & 15), r1 = __shfl(lsum[nb][1], l32 & 15);
            low |= !((l32 < 16 ? r0 : r1) >= kUnderflowGuard);
          }
          if (__syncthreads_or(low)) {
            fast_exit = true;
            break;
          }
        } else {
          barrier_dma();
        }
      }
      if (fast_exit) {
        l_run[0] = l_run[1] = 0.f;
        return;
      }
      R(1, 1);
      P(1, 1);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        // query l32 of block nb: row l32 / 16 of lane l32 % 16; kept on half 0
        const float r0 = __shfl(lsum[nb][0], l32 & 15), r1 = __shfl(lsum[nb][1], l32 & 15);
        l_run[nb] = half == 0 ? (l32 < 16 ? r0 : r1) : 0.f;
        // keys past N have zero K rows: their P is exp2(0 - shift), rounded as the MFMA saw it
        if (t1 == nkt)
          pad_sub[nb] = (float)(nkt * kKeyTile - N) * (SH ? (float)f32_to_bf16(__builtin_amdgcn_exp2f(-msub[nb])) : 1.f);
      }
    };
    if (!MAPKV && shift) fast_pass(BoolTag<true>());
    else fast_pass(BoolTag<false>());
  } else {
    f32x16 cinit[2];
    const float mneg[2] = {-mref[0], -mref[1]};
    _Float16 bh[2][16];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[nb][i] = 0.f;
        cinit[nb][i] = mneg[nb];
      }
      m_run[nb] = mref[nb];
    }
    // Row sums on the matrix pipe: v_mfma_f32_16x16x32_bf16 with a 0/1 selector
    // as A. Read as that MFMA's B operand, lane l of a P block holds query
    // l % 16 + 16 * ((l / 16) % 2); the selector puts lane groups 0 and 2
    // into row 0 and groups 1 and 3 into row 1, so rows 0 and 1 of the 16x16
    // accumulator (lanes 0-15, elements 0 and 1) collect the sums of the
    // block's queries 0-15 and 16-31 over the exact bf16 P values the PV MFMA
    // consumes. (A dot2 on the vector pipe would wait for the matrix pipe.)
    f32x4 lsum[2];
    bf16x8 rsel;
    {
      const bf16 one = (lane & 15) == ((lane >> 4) & 1) ? (bf16)1.0f : (bf16)0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) rsel[j] = one;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) lsum[nb] = f32x4(0.f);
    }

    // half step: softmax of sc_in, scores of the subtile whose K fragments are in
    // kf into sc_out, O += V^T(vbuf, vsub) P^T. Once the last score MFMA has
    // read kf, the fragments of the next half step's subtile (nkbuf, nksub),
    // already in LDS, are fetched into kf so their latency hides behind the
    // rest of this half step.
    auto half_step = [&](const f32x16* sc_in, bf16x8* kf, int nkbuf, int nksub, int nkey0, int vbuf, int vsub,
                         f32x16* sc_out) {
      bf16x8 vf[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) vf[s] = vfrag(vbuf, vsub, s);
      u32x4 words[2][2];
      // P words w0, w0+1 of block (nb, s): 4 exp2, 2 packs
      auto pslice = [&](int nb, int s, int w0) {
#pragma unroll
        for (int w = w0; w < w0 + 2; ++w) {
          bf16x2 pr;
          pr[0] = f32_to_bf16(__builtin_amdgcn_exp2f(sc_in[nb][8 * s + 2 * w]));
          pr[1] = f32_to_bf16(__builtin_amdgcn_exp2f(sc_in[nb][8 * s + 2 * w + 1]));
          words[nb][s][w] = __builtin_bit_cast(unsigned, pr);
        }
      };
      auto rsmfma = [&](int s, int nb) {
        lsum[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rsel, __builtin_bit_cast(bf16x8, words[nb][s]), lsum[nb],
                                                           0, 0, 0);
      };
      auto smfma = [&](int s, int nb) {
        sc_out[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[nb][s], s == 0 ? cinit[nb] : sc_out[nb], 0,
                                                             0, 0);
      };
      auto pvmfma = [&](int s, int nb) {
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s], __builtin_bit_cast(bf16x8, words[nb][s]), acc[nb],
                                                          0, 0, 0);
      };
      pslice(0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      smfma(0, 0);
      pslice(0, 0, 2);
      __builtin_amdgcn_sched_barrier(0);
      smfma(0, 1);
      pslice(1, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      smfma(1, 0);
      rsmfma(0, 0);
      pslice(1, 0, 2);
      __builtin_amdgcn_sched_barrier(0);
      smfma(1, 1);
      pslice(0, 1, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (C::kSteps > 2) smfma(2, 0);
      rsmfma(0, 1);
      pslice(0, 1, 2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 2; s < C::kSteps; ++s) {
        if (s > 2) smfma(s, 0);
        smfma(s, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      load_kf(nkbuf, nksub, kf);
      if constexpr (RPB) gather_bias(nkbuf, nksub, bh);
      pslice(1, 1, 0);
      __builtin_amdgcn_sched_barrier(0);
      pvmfma(0, 0);
      rsmfma(1, 0);
      pslice(1, 1, 2);
      __builtin_amdgcn_sched_barrier(0);
      pvmfma(0, 1);
      pvmfma(1, 0);
      pvmfma(1, 1);
      rsmfma(1, 1);
      if constexpr (RPB) bias_cinit(bh, mneg, nkey0, cinit);
      __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: tiles t0 and t0 + 1 in LDS, t0 + 2 on its way, scores of the
    // first subtile, K fragments of the second. Tiles past the range repeat its
    // last tile (read only by the unused scores of the subtile after the last).
    // Buffers are numbered from t0.
    dma_tile(t0, 0);
    dma_tile(min(t0 + 1, t1 - 1), 1);
    dma_tile(min(t0 + 2, t1 - 1), 2);
    dma_wait_older();
    __syncthreads();
    f32x16 sc_a[2], sc_b[2];
    bf16x8 kf[C::kSteps];
    load_kf(0, 0, kf);
    if constexpr (RPB) {
      gather_bias(0, 0, bh);
      bias_cinit(bh, mneg, 0, cinit);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      sc_a[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[nb][0], cinit[nb], 0, 0, 0);
#pragma unroll
      for (int s = 1; s < C::kSteps; ++s)
        sc_a[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[nb][s], sc_a[nb], 0, 0, 0);
    }
    load_kf(0, 1, kf);
    if constexpr (RPB) {
      gather_bias(0, 1, bh);
      bias_cinit(bh, mneg, 32, cinit);
    }
    for (int t = t0; t < t1; ++t) {
      const int b0 = (t - t0) % kBufs, b1 = (t - t0 + 1) % kBufs;
      const int k1 = (t + 1) * kKeyTile;
      dma_tile(min(t + 3, t1 - 1), (t - t0 + 3) % kBufs);
      half_step(sc_a, kf, b1, 0, k1, b0, 0, sc_b);        // softmax (t, 0); scores (t, 1); prefetch (t + 1, 0)
      half_step(sc_b, kf, b1, 1, k1 + 32, b0, 1, sc_a);   // softmax (t, 1); scores (t + 1, 0); prefetch (t + 1, 1)
      dma_wait_older();                          // tile t + 2 landed (this wave's part)
      barrier_dma();
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      // query l32 of block nb: row l32 / 16 of lane l32 % 16; kept on half 0
      const float r0 = __shfl(lsum[nb][0], l32 & 15), r1 = __shfl(lsum[nb][1], l32 & 15);
      l_run[nb] = half == 0 ? (l32 < 16 ? r0 : r1) : 0.f;
      if (!RPB && t1 == nkt)
        pad_sub[nb] = (float)(nkt * kKeyTile - N) * (float)f32_to_bf16(__builtin_amdgcn_exp2f(-mref[nb]));
    }
  }

  bool bad = fast_exit;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    // both halves of the wave hold part of each row sum; the padded keys are
    // removed once from the half-0 share
    l_run[nb] -= half == 0 ? pad_sub[nb] : 0.f;
    const float l_tot = l_run[nb] + swap_halves(l_run[nb]);
    bad |= !(l_tot >= kUnderflowGuard) || !(l_tot < INFINITY);
    if constexpr (MAPKV) {   // no bound: an overflow may have reached the accumulators
      float asum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) asum += fabsf(acc[nb][i]);
      bad |= !(asum < INFINITY);
    }
  }

  // ===== exact pass (rare fallback): classic online softmax, double-buffered
  if (__syncthreads_or(bad)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nb][i] = 0.f;
      m_run[nb] = -INFINITY;
      l_run[nb] = 0.f;
    }
    // drain the fast pass's DMA (tiles past the end) before reusing buffers
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    dma_tile(t0, 0);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
      const int buf = (t - t0) & 1;
      if (t + 1 < t1) dma_tile(t + 1, buf ^ 1);
      const bool tail = (t + 1) * kKeyTile > N;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        bf16x8 kf[C::kSteps];
        load_kf(buf, sub, kf);
        f32x16 sc[2];
        if constexpr (RPB) {
          _Float16 bh[2][16];
          const float zero[2] = {0.f, 0.f};
          gather_bias(buf, sub, bh);
          bias_cinit(bh, zero, t * kKeyTile + sub * 32, sc);
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if constexpr (!RPB)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[nb][i] = 0.f;
#pragma unroll
          for (int s = 0; s < C::kSteps; ++s)
            sc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[nb][s], sc[nb], 0, 0, 0);
        }
        if (tail) mask_tail(sc, t * kKeyTile + sub * 32);
        bf16x8 pf[2][2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          float mx = sc[nb][0];
#pragma unroll
          for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[nb][v]);
          mx = fmaxf(mx, swap_halves(mx));
          const float m_new = fmaxf(m_run[nb], mx);
          if (__any(m_new > m_run[nb] + kLazyTau)) {
            const float alpha = (m_new == m_run[nb]) ? 1.f : exp2f(m_run[nb] - m_new);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nb][i] *= alpha;
            l_run[nb] *= alpha;
            m_run[nb] = m_new;
          }
          const float mneg = -m_run[nb];
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float p = exp2f(sc[nb][8 * s + j] + mneg);
              l_run[nb] += p;
              pf[nb][s][j] = f32_to_bf16(p);
            }
        }
        pv(buf, sub, pf, acc);
      }
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();
    }
  }

  // ---- split piece: the unnormalized O, the row sums and the shifts go to the piece's slot
  // (all 256 queries of the item, padded ones included); the combine kernel adds the pieces
  if (!RPB && piece >= 0) {
    float* po = a.part + (int64_t)piece * kSplitPieceFloats;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int ql = wave * kQPerWave + nb * 32 + l32;
      const float l_tot = l_run[nb] + swap_halves(l_run[nb]);
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = acc[nb][4 * gq + i];
        *(f32x4*)(po + ql * 32 + 8 * gq + 4 * half) = o4;
      }
      if (half == 0) *(float2*)(po + 256 * 32 + 2 * ql) = make_float2(l_tot, m_run[nb]);
    }
    return;
  }

  // ---- epilogue: normalize, optionally gate (O' = O * G, G in the same map layout), write O
  // rows (map layout) and the LSE of the ungated attention
  bf16* omap = (bf16*)a.o_map;
  const float kLn2 = 0.69314718055994530942f;
  if constexpr (!RPB) {
    // A lane holds 16 of its query's 32 channels in 4-channel pieces; stored as they are, every
    // store instruction would touch 32 rows with 8 bytes each. Instead each wave stages its 64
    // normalized rows in its own LDS region ([64 rows][5 chunks], the tile ring is free: every
    // wave is past the loops and the DMA of tiles past the range has drained) and writes them
    // back as whole 64-byte rows, 16 rows per store instruction.
    constexpr int kORow = 5;
    static_assert(C::kWv * kQPerWave * kORow <= kBufs * C::kChunks, "O staging fits the tile ring");
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    bf16* stage = (bf16*)&sT[0][0] + wave * kQPerWave * kORow * 8;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int q = q0 + nb * 32 + l32;
      const float l_tot = l_run[nb] + swap_halves(l_run[nb]);
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float gv[4] = {inv, inv, inv, inv};
        if constexpr (GATE) {
          if (q < N) {
            bf16 g4[4];
            *(uint2*)g4 = *(const uint2*)((const bf16*)a.gate + map_row(q) + 8 * gq + 4 * half);
#pragma unroll
            for (int i = 0; i < 4; ++i) gv[i] = inv * (float)g4[i];
          }
        }
        bf16 o4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = f32_to_bf16(acc[nb][4 * gq + i] * gv[i]);
        *(uint2*)(stage + (nb * 32 + l32) * kORow * 8 + 8 * gq + 4 * half) = *(const uint2*)o4;
      }
      if (q < N && a.lse && half == 0) a.lse[pm.pixel_head(unit, q)] = (m_run[nb] + log2f(l_tot)) * kLn2;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rl = (lane >> 2) + 16 * j, ch = 8 * (lane & 3);
      const int q = q0 + rl;
      const u32x4 v = *(const u32x4*)(stage + rl * kORow * 8 + ch);
      if (q < N) *(u32x4*)(omap + map_row(q) + ch) = v;
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int q = q0 + nb * 32 + l32;
      const float l_tot = l_run[nb] + swap_halves(l_run[nb]);
      const float inv = 1.f / l_tot;
      if (q < N) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          bf16 o4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = f32_to_bf16(acc[nb][4 * gq + i] * inv);
          *(uint2*)(omap + map_row(q) + 8 * gq + 4 * half) = *(const uint2*)o4;
        }
        if (a.lse && half == 0) a.lse[pm.pixel_head(unit, q)] = (m_run[nb] + log2f(l_tot)) * kLn2;
      }
    }
  }
}

// RPB preparation. Block h < heads converts table row h to fp16 in log2 units
// (zero-padded to `stride` entries) and writes its maximum; block `heads`
// writes the per-key byte offsets -2 ((k / w)(2w - 1) + k % w) for k < N and
// 0 for the padded rows.
__global__ __launch_bounds__(256) void rpb_prep_kernel(const float* __restrict__ table, int heads, int entries,
                                                       int stride, int w, int N, int n_rows,
                                                       _Float16* __restrict__ tab16, float* __restrict__ tmax,
                                                       int* __restrict__ kidx) {
  __shared__ float red[4];
  if ((int)blockIdx.x < heads) {
    const float* src = table + (int64_t)blockIdx.x * entries;
    _Float16* dst = tab16 + (int64_t)blockIdx.x * stride;
    constexpr float kLog2e = 1.44269504088896340736f;
    float mx = -INFINITY;
    for (int i = threadIdx.x; i < stride; i += 256) {
      _Float16 h = (_Float16)0.f;
      if (i < entries) {
        h = (_Float16)(src[i] * kLog2e);
        mx = fmaxf(mx, (float)h);
      }
      dst[i] = h;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) tmax[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  } else {
    const int w2 = 2 * w - 1;
    for (int t = threadIdx.x; t < n_rows; t += 256) kidx[t] = t < N ? -2 * ((t / w) * w2 + t % w) : 0;
  }
}

// ---------------------------------------------------------------------------
// Simple kernel: one thread per query, K/V tiles of 64 keys in LDS, exact online
// softmax per tile, float32 arithmetic on T (float or bf16) rows with D content
// channels. It serves float32 runs and content widths the MFMA kernel does not
// cover (d_c = 64): correctness-sized work.
template <typename T, int D, int RP>
__global__ __launch_bounds__(256) void attn_fwd_simple_kernel(FwdArgs a) {
  constexpr int DH = D + RP;
  __shared__ float sK[kKeyTile][DH + 1];
  __shared__ float sV[kKeyTile][D + 1];
  const Geom& g = a.g;
  const int N = g.N, n_rows = g.n_rows;
  const int nqb = (N + 255) / 256;
  const int unit = blockIdx.x / nqb;
  const int q = (blockIdx.x - unit * nqb) * 256 + threadIdx.x;
  const T* qw = (const T*)a.qw + (int64_t)unit * n_rows * D;
  const T* kw = (const T*)a.kw + (int64_t)unit * n_rows * D;
  const T* vw = (const T*)a.vw + (int64_t)unit * n_rows * D;
  const T* qp = (const T*)a.qp;
  const T* kp = (const T*)a.kp;
  float qh[DH];
  const int qq = q < N ? q : 0;
#pragma unroll
  for (int i = 0; i < D; ++i) qh[i] = (float)qw[(int64_t)qq * D + i];
#pragma unroll
  for (int i = 0; i < RP; ++i) qh[D + i] = (float)qp[(int64_t)qq * RP + i];
  float o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float c = a.c;
  const int nkt = (N + kKeyTile - 1) / kKeyTile;
  for (int t = 0; t < nkt; ++t) {
    const int k0 = t * kKeyTile;
    for (int i = threadIdx.x; i < kKeyTile * DH; i += 256) {
      int kk = i / DH, ch = i - kk * DH;
      sK[kk][ch] = ch < D ? (float)kw[(int64_t)(k0 + kk) * D + ch] : (float)kp[(int64_t)(k0 + kk) * RP + ch - D];
    }
    for (int i = threadIdx.x; i < kKeyTile * D; i += 256) {
      int kk = i / D, ch = i - kk * D;
      sV[kk][ch] = (float)vw[(int64_t)(k0 + kk) * D + ch];
    }
    __syncthreads();
    const int nk = min(kKeyTile, N - k0);
    float s[kKeyTile];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeyTile; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DH; ++i) acc = fmaf(qh[i], sK[j][i], acc);
      s[j] = j < nk ? acc * c : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2f(m - m_new);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] *= alpha;
    m = m_new;
#pragma unroll
    for (int j = 0; j < kKeyTile; ++j) {
      const float p = exp2f(s[j] - m);
      l += p;
#pragma unroll
      for (int i = 0; i < D; ++i) o[i] = fmaf(p, sV[j][i], o[i]);
    }
    __syncthreads();
  }
  if (q < N) {
    T* ow = (T*)a.ow + (int64_t)unit * n_rows * D + (int64_t)q * D;
    const float inv = 1.f / l;
    const PixelMap pm = make_pixel_map(g);
    const T* gt = a.gate ? (const T*)a.gate + pm.pixel_head(unit, q) * D : nullptr;
#pragma unroll
    for (int i = 0; i < D; ++i) ow[i] = (T)(gt ? o[i] * inv * (float)gt[i] : o[i] * inv);
    if (a.lse) a.lse[pm.pixel_head(unit, q)] = (m + log2f(l)) * 0.69314718055994530942f;
  }
}

}  // namespace

int key_bound_parts(int N) { return (N + kKeyBoundTile - 1) / kKeyBoundTile; }

int rpb_table_stride(int w) {
  const int entries = (2 * w - 1) * (2 * w - 1);
  return (entries + 511) / 512 * 512;
}

size_t rpb_fwd_lds_bytes(int w) {
  // tile ring + table + a margin for the compiler's own static LDS (256 bytes today)
  return sizeof(u32x4) * kBufs * FwdCfg<0, true>::kChunks + 2 * (size_t)rpb_table_stride(w) + 512;
}

hipError_t launch_rpb_prep(const Geom& g, const float* table, _Float16* tab16, float* tmax, int* kidx,
                           hipStream_t stream) {
  const int entries = (2 * g.w - 1) * (2 * g.w - 1);
  hipLaunchKernelGGL(rpb_prep_kernel, dim3(g.heads + 1), dim3(256), 0, stream, table, g.heads, entries,
                     rpb_table_stride(g.w), g.w, g.N, g.n_rows, tab16, tmax, kidx);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_rpb(const FwdArgs& a, hipStream_t stream) {
  typedef FwdCfg<0, true> C;
  const int nqb = (a.g.N + C::kQPerBlock - 1) / C::kQPerBlock;
  const int64_t blocks = (int64_t)a.g.units * nqb;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<0, true>), dim3((unsigned)blocks), dim3(64 * C::kWv),
                     2 * (size_t)a.rpb_stride, stream, a);
  return hipGetLastError();
}

namespace {

// Split-tail combine. Block (split item, 64 queries), thread (query, 8 channels): sums the
// item's pieces in a fixed order, O = sum_r 2^(m_r - M) O_r / sum_r 2^(m_r - M) l_r with
// M = max_r m_r (every piece of a fast pass has the same m, the query's bound), and writes
// O (times the gate, when there is one) to the map and LSE = (M + log2 L) ln 2.
__global__ __launch_bounds__(256) void fwd_split_combine_kernel(FwdArgs a) {
  const Geom& g = a.g;
  const int N = g.N;
  const int nqb = (N + FwdCfg<1>::kQPerBlock - 1) / FwdCfg<1>::kQPerBlock;
  const int total = g.units * nqb;
  const int slot = blockIdx.x / 4, qpart = blockIdx.x % 4;
  const int xcd = slot / a.split_tail_max, k = slot - xcd * a.split_tail_max;
  const int q8 = total / 8, rem = total % 8;
  const int n_x = q8 + (xcd < rem ? 1 : 0);
  const int base = xcd < rem ? xcd * (q8 + 1) : rem * (q8 + 1) + (xcd - rem) * q8;
  const int full = n_x / a.split_spx * a.split_spx;
  if (k >= n_x - full) return;
  const int item = base + full + k, unit = item / nqb, qb = item - unit * nqb;
  const int ql = qpart * 64 + (int)threadIdx.x / 4, ch = 8 * ((int)threadIdx.x % 4);
  const int q = qb * FwdCfg<1>::kQPerBlock + ql;
  if (q >= N) return;
  const float* p0 = a.part + (int64_t)slot * a.split_s * kSplitPieceFloats;
  float M = -INFINITY;
  for (int r = 0; r < a.split_s; ++r) M = fmaxf(M, p0[r * kSplitPieceFloats + 256 * 32 + 2 * ql + 1]);
  float L = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  for (int r = 0; r < a.split_s; ++r) {
    const float* pr = p0 + r * kSplitPieceFloats;
    const float2 lm = *(const float2*)(pr + 256 * 32 + 2 * ql);
    const float wgt = exp2f(lm.y - M);
    L = fmaf(wgt, lm.x, L);
    const f32x4 a0 = *(const f32x4*)(pr + ql * 32 + ch), a1 = *(const f32x4*)(pr + ql * 32 + ch + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = fmaf(wgt, a0[i], o[i]);
      o[4 + i] = fmaf(wgt, a1[i], o[4 + i]);
    }
  }
  const float inv = 1.f / L;
  const PixelMap pm = make_pixel_map(g);
  const int64_t ph = pm.pixel_head(unit, q);
  float gv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) gv[i] = inv;
  if (a.gate) {
    const bf16x8 g8 = *(const bf16x8*)((const bf16*)a.gate + ph * 32 + ch);
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = inv * (float)g8[i];
  }
  bf16x8 ob;
#pragma unroll
  for (int i = 0; i < 8; ++i) ob[i] = f32_to_bf16(o[i] * gv[i]);
  *(bf16x8*)((bf16*)a.o_map + ph * 32 + ch) = ob;
  if (a.lse && ch == 0) a.lse[ph] = (M + log2f(L)) * 0.69314718055994530942f;
}

// Compute units per XCD and workgroups per CU of the plain bf16 kernel (KP = 1, 2) on the
// current device; cus = 0 when the compute units do not divide into 8 XCDs.
struct XcdSlots {
  int cus = 0, occ = 0;
};
XcdSlots split_slots(int kp, hipError_t* err) {
  static XcdSlots cache[2][64];
  static bool have[2][64];
  static std::mutex mu;   // calls from several host threads fill the cache once
  int dev = 0;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return {};
  if (dev < 0 || dev >= 64) return {};
  std::lock_guard<std::mutex> lk(mu);
  if (!have[kp - 1][dev]) {
    int cus = 0, occ = 0;
    if ((*err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return {};
    *err = kp == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, attn_fwd_bf16_kernel<1>, 256, 0)
                   : hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, attn_fwd_bf16_kernel<2>, 256, 0);
    if (*err != hipSuccess) return {};
    cache[kp - 1][dev] = XcdSlots{cus % 8 == 0 ? cus / 8 : 0, occ};
    have[kp - 1][dev] = true;
  }
  return cache[kp - 1][dev];
}

// Slot model of one XCD's tail, measured on MI355X with this kernel: n pieces of `len` (in
// units of one whole item's time when `occ` workgroups share a CU) are dealt to the free
// slots of `cus` CUs, always to the least busy CU first; a workgroup on a CU that runs k
// workgroups runs at slot_rate(occ, k) times the speed of one of a full CU. Returns the
// time until the last piece finishes.
double slot_rate(int occ, int k) {
  // measured: one positional K-step, 3 workgroups per CU (w = 64 items alone on their
  // CUs, two per CU and four full rounds: 0.065, 0.103 and 0.127 ms per item round);
  // two workgroups per CU (the r = 32 instance): alone 1.82x
  if (occ == 3) return k == 1 ? 1.94 : (k == 2 ? 1.23 : 1.0);
  if (occ == 2) return k == 1 ? 1.82 : 1.0;
  return 1.0;
}
double tail_time(int n, double len, int cus, int occ) {
  constexpr int kMaxSlots = 64 * 4;
  if (n <= 0) return 0.0;
  if (cus * occ > kMaxSlots || cus <= 0 || occ <= 0) return 1e30;
  double rem[kMaxSlots];
  for (int s = 0; s < cus * occ; ++s) rem[s] = -1.0;
  auto busy = [&](int c) {
    int k = 0;
    for (int j = 0; j < occ; ++j) k += rem[c * occ + j] >= 0.0;
    return k;
  };
  int next = 0;
  auto deal = [&]() {
    for (int k = 0; k < occ; ++k)
      for (int c = 0; c < cus && next < n; ++c) {
        if (busy(c) != k) continue;
        for (int j = 0; j < occ; ++j)
          if (rem[c * occ + j] < 0.0) {
            rem[c * occ + j] = len;
            ++next;
            break;
          }
      }
  };
  deal();
  double t = 0.0;
  for (;;) {
    double dt = 1e30;
    for (int c = 0; c < cus; ++c) {
      const double rate = slot_rate(occ, busy(c));
      for (int j = 0; j < occ; ++j)
        if (rem[c * occ + j] >= 0.0) dt = std::min(dt, rem[c * occ + j] / rate);
    }
    if (dt >= 1e30) return t;
    t += dt;
    for (int c = 0; c < cus; ++c) {
      const double rate = slot_rate(occ, busy(c));
      for (int j = 0; j < occ; ++j) {
        double& r = rem[c * occ + j];
        if (r < 0.0) continue;
        r -= rate * dt;
        if (r <= 1e-9) r = -1.0;
      }
    }
    deal();
  }
}

// Blocks of the split launch: per XCD its whole items plus split_s pieces per tail item,
// every XCD padded to the largest count (the hardware deals blocks to XCDs in turn).
int64_t split_blocks(const FwdArgs& a) {
  const int nqb = (a.g.N + FwdCfg<1>::kQPerBlock - 1) / FwdCfg<1>::kQPerBlock;
  const int total = a.g.units * nqb, q8 = total / 8, rem = total % 8;
  int64_t most = 0;
  for (int x = 0; x < 8; ++x) {
    const int n_x = q8 + (x < rem ? 1 : 0), full = n_x / a.split_spx * a.split_spx;
    most = std::max<int64_t>(most, full + (int64_t)(n_x - full) * a.split_s);
  }
  return 8 * most;
}

}  // namespace

size_t split_region_pieces(int units, int N) {
  const int nkt = (N + kKeyTile - 1) / kKeyTile;
  if (nkt < kSplitMinTiles) return 0;
  const int64_t total = (int64_t)units * ((N + FwdCfg<1>::kQPerBlock - 1) / FwdCfg<1>::kQPerBlock);
  return (size_t)std::min<int64_t>(kMaxSplitPieces, 8 * ((total + 7) / 8) * 4);
}

hipError_t plan_fwd_split(FwdArgs& a) {
  a.split_spx = 0;
  a.split_s = 1;
  a.split_tail_max = 0;
  if (!a.part || (a.rp != 16 && a.rp != 32)) return hipSuccess;
  const size_t region = split_region_pieces(a.g.units, a.g.N);
  if (region == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  const XcdSlots xs = split_slots(a.rp / 16, &e);
  if (e != hipSuccess) return e;
  const int spx = xs.cus * xs.occ;
  if (spx <= 0) return hipSuccess;
  const int nqb = (a.g.N + FwdCfg<1>::kQPerBlock - 1) / FwdCfg<1>::kQPerBlock;
  const int total = a.g.units * nqb, q8 = total / 8, rem = total % 8;
  int tail_max = 0;
  for (int x = 0; x < 8; ++x) tail_max = std::max(tail_max, (q8 + (x < rem ? 1 : 0)) % spx);
  if (tail_max == 0) return hipSuccess;
  // Whole items, halves or quarters, whichever the slot model finishes first: a piece costs
  // its share of the keys plus 3 % of an item (pipeline fill and drain, prologue), and the
  // combine 4 % of an item; the split has to win by 1 % of an item.
  constexpr double kPieceCost = 0.03, kCombineCost = 0.04, kMinGain = 0.01;
  int S = 1;
  double best = tail_time(tail_max, 1.0, xs.cus, xs.occ) - kMinGain;
  for (int s2 : {2, 4}) {
    if ((size_t)8 * tail_max * s2 > region) continue;
    const double t = tail_time(tail_max * s2, 1.0 / s2 + kPieceCost, xs.cus, xs.occ) + kCombineCost;
    if (t < best) best = t, S = s2;
  }
  if (S < 2) return hipSuccess;
  a.split_spx = spx;
  a.split_s = S;
  a.split_tail_max = tail_max;
  return hipSuccess;
}

hipError_t launch_fwd_split_combine(const FwdArgs& a, hipStream_t stream) {
  if (a.split_spx == 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_split_combine_kernel, dim3((unsigned)(8 * a.split_tail_max * 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.g.N + FwdCfg<1>::kQPerBlock - 1) / FwdCfg<1>::kQPerBlock;
  int64_t blocks = (int64_t)a.g.units * nqb;
  if (blocks == 0) return hipSuccess;
  if (a.split_spx) blocks = split_blocks(a);
  if (a.k_map) {
    if (a.gate)
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<1, false, true, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<1, false, false, true>), dim3((unsigned)blocks), dim3(256), 0, stream,
                         a);
  } else if (a.gate) {
    if (a.rp == 16)
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<1, false, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<2, false, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  } else if (a.rp == 16) {
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_simple(const FwdArgs& a, int esize, hipStream_t stream) {
  const int nqb = (a.g.N + 255) / 256;
  const int64_t blocks = (int64_t)a.g.units * nqb;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(256);
#define RIB_FWD_SIMPLE(T, D, RP) hipLaunchKernelGGL((attn_fwd_simple_kernel<T, D, RP>), grid, block, 0, stream, a)
  const int d = a.g.d_c;
  if (esize == 4) {
    if (d == 32) { if (a.rp == 16) RIB_FWD_SIMPLE(float, 32, 16); else RIB_FWD_SIMPLE(float, 32, 32); }
    else { if (a.rp == 16) RIB_FWD_SIMPLE(float, 64, 16); else RIB_FWD_SIMPLE(float, 64, 32); }
  } else {
    if (d == 32) { if (a.rp == 16) RIB_FWD_SIMPLE(bf16, 32, 16); else RIB_FWD_SIMPLE(bf16, 32, 32); }
    else { if (a.rp == 16) RIB_FWD_SIMPLE(bf16, 64, 16); else RIB_FWD_SIMPLE(bf16, 64, 32); }
  }
#undef RIB_FWD_SIMPLE
  return hipGetLastError();
}

}  // namespace rib
