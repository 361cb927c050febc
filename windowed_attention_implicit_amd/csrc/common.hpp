// Shared device/host helpers of the RIB window-attention library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rib.h"

namespace rib {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Rows of every windowed work buffer are padded to a multiple of this many
// tokens; padded rows are zero so tiles can be loaded without bounds checks.
constexpr int kRowPad = 64;

__host__ __device__ inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Geometry of one call, derived once on the host.
struct Geom {
  int B, H, W, heads, d_c, w, r;
  int N;        // tokens per window, w*w
  int n_rows;   // N rounded up to kRowPad
  int nwy, nwx; // windows per column / row of the map
  int units;    // B * nwy * nwx * heads  (one per (batch, window, head))
};

inline Geom make_geom(const rib_shape_t& s) {
  Geom g;
  g.B = s.B; g.H = s.H; g.W = s.W; g.heads = s.heads; g.d_c = s.d_c; g.w = s.w; g.r = s.r;
  g.N = s.w * s.w;
  g.n_rows = (int)round_up(g.N, kRowPad);
  g.nwy = s.H / s.w;
  g.nwx = s.W / s.w;
  g.units = s.B * g.nwy * g.nwx * s.heads;
  return g;
}

// Offset (in elements of a [B, H, W, heads, d] tensor, excluding d) of token t
// of unit u, where u enumerates (batch, window row, window col, head) with
// heads innermost.
struct PixelMap {
  int H, W, heads, w, nwy, nwx;
  __device__ __forceinline__ int64_t pixel_head(int u, int t) const {
    int head = u % heads;
    int win = u / heads;
    int wx = win % nwx;
    int rest = win / nwx;
    int wy = rest % nwy;
    int b = rest / nwy;
    int iy = t / w, ix = t - (t / w) * w;
    int64_t y = (int64_t)wy * w + iy, x = (int64_t)wx * w + ix;
    return (((int64_t)b * H + y) * W + x) * heads + head;
  }
};

__host__ __device__ inline PixelMap make_pixel_map(const Geom& g) {
  PixelMap m;
  m.H = g.H; m.W = g.W; m.heads = g.heads; m.w = g.w; m.nwy = g.nwy; m.nwx = g.nwx;
  return m;
}

// Remaps a linear block id so that consecutive logical blocks land on the same
// XCD: the hardware hands out workgroups round-robin over the 8 XCDs, each of
// which has its own L2. Bijective for any total.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcd = 8;
  int q = total / kXcd, rem = total % kXcd;
  int xcd = bid % kXcd, i = bid / kXcd;
  int base = xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
  return base + i;
}

__device__ __forceinline__ float bf16_to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f32_to_bf16(float x) { return (bf16)x; }  // round to nearest even

}  // namespace rib
