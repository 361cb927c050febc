// Global-to-LDS tile copies by DMA (buffer_load_dwordx4 ... lds) for gfx950.
//
// One DMA instruction moves 64 lanes x 16 bytes; lane l's bytes land in the
// l-th 16-byte slot of the 1 KB LDS block the instruction names (wave-uniform
// base in M0). A tile is a list of parts, each copying `rows` rows of `chunks`
// 16-byte chunks from a row-major global array into LDS rows padded to
// `lds_row` chunks (an odd stride keeps 16-byte reads across rows free of bank
// conflicts). Parts sit back to back in the tile buffer, each rounded up to
// whole instructions; instruction i is issued by wave i % 4. The layout is a
// compile-time constant and the issuing code is instantiated per wave, so a
// wave's instructions, their parts and its vmcnt budget are all constants;
// per lane only the source offset of each of its instructions is kept, and a
// tile moves it by the part's byte step. Pad slots fetch their row's first
// chunk again; slots past a part get an out-of-range offset, which the buffer
// range check turns into zeros.
#pragma once

#include "common.hpp"

namespace rib {

constexpr int kDmaWaves = 4;

// s_waitcnt immediate (gfx9 encoding) waiting only on the vector-memory
// counter: vmcnt bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) at max.
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

struct TilePart {
  int rows, chunks, lds_row;
};

template <int N>
struct TileLayout {
  TilePart p[N];
  static constexpr int kParts = N;
  constexpr int insts(int k) const { return (p[k].rows * p[k].lds_row + 63) / 64; }
  constexpr int first(int k) const {
    int f = 0;
    for (int i = 0; i < k; ++i) f += insts(i);
    return f;
  }
  constexpr int total() const { return first(N); }
  constexpr int part_of(int i) const {
    for (int k = 0; k < N; ++k)
      if (i < first(k + 1)) return k;
    return N;
  }
  constexpr int offset(int k) const { return 64 * first(k); }   // chunk offset of part k in a buffer
  constexpr int chunks() const { return 64 * total(); }
  constexpr int slots() const { return (total() + kDmaWaves - 1) / kDmaWaves; }
  constexpr int count(int w) const { return (total() - w + kDmaWaves - 1) / kDmaWaves; }
};

// Runtime side of the parts: buffer resources and per-tile byte steps, plus
// this lane's offsets (slot j = instruction kDmaWaves * j + wave).
template <int N, int SLOTS>
struct TileDma {
  __amdgpu_buffer_rsrc_t rsrc[N];
  unsigned step[N];
  unsigned off[SLOTS];
};

// base, addressable bytes, row stride and per-tile step in bytes of one part. With map_w > 0
// the rows are the tokens of a w x w window in a [B, H, W, heads, d] map, w = 2^map_w: row r
// sits r / w map rows (row_bytes each) and r % w pixels (pix_bytes each) below the base, which
// holds per tile when w divides the tile's 64 rows.
struct DmaSrc {
  const void* base;
  int num_bytes, row_bytes, tile_step;
  int map_w = 0, pix_bytes = 0;
};

template <class LP, int W>
__device__ __forceinline__ void tile_dma_init_w(TileDma<LP::get().kParts, LP::get().slots()>& d,
                                                const DmaSrc (&src)[LP::get().kParts], int lane) {
  constexpr auto L = LP::get();
#pragma unroll
  for (int j = 0; j < L.slots(); ++j) {
    const int i = kDmaWaves * j + W;   // constant once the loop is unrolled
    unsigned o = 0;
    if (i < L.total()) {
      const int k = L.part_of(i);
      const int c = (i - L.first(k)) * 64 + lane;
      const int r = c / L.p[k].lds_row, ch = c - r * L.p[k].lds_row;
      const int ro = src[k].map_w > 0 ? (r >> src[k].map_w) * src[k].row_bytes +
                                            (r & ((1 << src[k].map_w) - 1)) * src[k].pix_bytes
                                      : r * src[k].row_bytes;
      o = r < L.p[k].rows ? (unsigned)(ro + (ch < L.p[k].chunks ? ch : 0) * 16) : 0x80000000u;
    }
    d.off[j] = o;
  }
}

template <class LP>
__device__ __forceinline__ void tile_dma_init(TileDma<LP::get().kParts, LP::get().slots()>& d,
                                              const DmaSrc (&src)[LP::get().kParts], int wave, int lane) {
  constexpr auto L = LP::get();
#pragma unroll
  for (int k = 0; k < L.kParts; ++k) {
    d.rsrc[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src[k].base), 0, src[k].num_bytes, 0x00020000);
    d.step[k] = (unsigned)src[k].tile_step;
  }
  switch (wave) {
    case 0: tile_dma_init_w<LP, 0>(d, src, lane); break;
    case 1: tile_dma_init_w<LP, 1>(d, src, lane); break;
    case 2: tile_dma_init_w<LP, 2>(d, src, lane); break;
    default: tile_dma_init_w<LP, 3>(d, src, lane); break;
  }
}

template <class LP, int W>
__device__ __forceinline__ void tile_dma_issue_w(const TileDma<LP::get().kParts, LP::get().slots()>& d, int t,
                                                 void* buf) {
  constexpr auto L = LP::get();
#pragma unroll
  for (int j = 0; j < L.slots(); ++j) {
    const int i = kDmaWaves * j + W;
    if (i < L.total()) {
      const int k = L.part_of(i);
      auto* dst = (__attribute__((address_space(3))) void*)((char*)buf + 1024 * i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsrc[k], dst, 16, (int)(d.off[j] + (unsigned)t * d.step[k]), 0, 0,
                                               0);
    }
  }
}

// Issue this wave's instructions for tile t into the tile buffer `buf`.
template <class LP>
__device__ __forceinline__ void tile_dma_issue(const TileDma<LP::get().kParts, LP::get().slots()>& d, int wave, int t,
                                               void* buf) {
  switch (wave) {
    case 0: tile_dma_issue_w<LP, 0>(d, t, buf); break;
    case 1: tile_dma_issue_w<LP, 1>(d, t, buf); break;
    case 2: tile_dma_issue_w<LP, 2>(d, t, buf); break;
    default: tile_dma_issue_w<LP, 3>(d, t, buf); break;
  }
}

// Wait until at most `newer` tiles' worth of this wave's DMA is still in flight.
template <class LP, int NEWER>
__device__ __forceinline__ void tile_dma_wait(int wave) {
  constexpr auto L = LP::get();
  static_assert(NEWER * L.slots() < 64, "vmcnt is a 6-bit count");
  switch (wave) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_only(NEWER * L.count(0))); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_only(NEWER * L.count(1))); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_only(NEWER * L.count(2))); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_only(NEWER * L.count(3))); break;
  }
}

}  // namespace rib
