// Window partition / unpartition gathers for gfx950.
//
// The pages use non-overlapping square windows (gist.science/paper/2603.06738,
// "Technical Summary" §3.2: windows up to 96 x 96) but never describe the
// split; this library takes windows row-major per image, token t = iy*w + ix
// inside a window, heads innermost.
//
// A [B, H, W, heads, d] map stores, for every pixel, heads*d contiguous
// channels; one window row of one head is w runs of d channels. The plain
// gather / scatter kernels walk the map in its own memory order (16-byte
// chunks, fully coalesced on the map side) and move whole d-channel runs
// (64 bytes for bf16, d = 32) on the windowed side; padded rows (t >= N) of
// the internal buffers are written as zeros by extra threads of the same
// launch. The bf16 attention path instead prepares each direction in one pass
// per (unit, 64-token group) block: gather_kv_bound_kernel (forward: K_c rows,
// V kappa, key-norm maxima) and gather_bwd_kernel (backward: Q_c, K_c, dO rows
// and kappa, V rows, -D and -LSE2, the positional packing).
#include "internal.hpp"

namespace rib {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

struct ChunkGeom {
  int H, W, heads, w, nwy, nwx;
  int cpr;          // 16-byte chunks per d-channel row
  int n_rows;       // rows per unit on the windowed side
  int N;
};

__device__ __forceinline__ void decode_pixel_chunk(const ChunkGeom& g, int64_t i, int64_t& u, int& t, int& c) {
  c = (int)(i % g.cpr);
  int64_t ph = i / g.cpr;
  int head = (int)(ph % g.heads);
  int64_t pix = ph / g.heads;
  int x = (int)(pix % g.W);
  int64_t rest = pix / g.W;
  int y = (int)(rest % g.H);
  int64_t b = rest / g.H;
  int wx = x / g.w, ix = x - wx * g.w;
  int wy = y / g.w, iy = y - wy * g.w;
  u = ((b * g.nwy + wy) * g.nwx + wx) * g.heads + head;
  t = iy * g.w + ix;
}

// map -> rows layout; threads past the map's chunks zero the padded rows.
__global__ __launch_bounds__(256) void gather_rows_kernel(ChunkGeom g, int64_t map_chunks, int64_t pad_chunks,
                                                          const u32x4* __restrict__ x, u32x4* __restrict__ xw) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < map_chunks) {
    int64_t u; int t, c;
    decode_pixel_chunk(g, i, u, t, c);
    xw[(u * g.n_rows + t) * g.cpr + c] = __builtin_nontemporal_load(x + i);
  } else if (i < map_chunks + pad_chunks) {
    int64_t j = i - map_chunks;
    int pad = g.n_rows - g.N;
    int c = (int)(j % g.cpr);
    int64_t r = j / g.cpr;
    int64_t u = r / pad;
    int t = g.N + (int)(r % pad);
    xw[(u * g.n_rows + t) * g.cpr + c] = u32x4(0u);
  }
}

// rows layout -> map.
__global__ __launch_bounds__(256) void scatter_rows_kernel(ChunkGeom g, int64_t map_chunks,
                                                           const u32x4* __restrict__ xw, u32x4* __restrict__ x) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= map_chunks) return;
  int64_t u; int t, c;
  decode_pixel_chunk(g, i, u, t, c);
  __builtin_nontemporal_store(xw[(u * g.n_rows + t) * g.cpr + c], x + i);
}

// Position inside a 16-token group after swapping bits 2 and 3 (an involution).
__device__ __forceinline__ int kappa16(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// Block -> (unit, 64-token group) of the one-pass gathers. One head's 32 bf16 channels are
// half of a 128-byte line of the map, shared with the next head (the next unit). Workgroups
// are dealt to the 8 XCDs round-robin, so in the unit-major order those two heads' blocks,
// `groups` ids apart, share an XCD (and its L2) only when groups is a multiple of 8; for the
// other window sizes (w = 16: 4 groups) the blocks run group-major, with consecutive logical
// ids kept on one XCD, so the heads of one token group run side by side on one XCD.
__device__ __forceinline__ void block_unit_group(int groups, int& u, int& gi) {
  if (groups % 8 == 0) {
    u = blockIdx.x / groups;
    gi = blockIdx.x - u * groups;
  } else {
    const int units = gridDim.x / groups;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    gi = logical / units;
    u = logical - gi * units;
  }
}

// The bf16 forward's whole preparation in one pass. Block (unit, 64-token group):
// K_c rows -> the token-major rows layout [units][n_rows][32] (rows >= N zero), V ->
// the channel-major kappa layout [units][32][n_rows] (64 tokens x 64 bytes staged in LDS,
// then every thread writes 8 consecutive kappa positions of one channel), and the group's
// largest |[k_c | k_p]|^2 -> kmax2[unit * groups + group] and the group's largest |v| ->
// kmax2[units * groups + unit * groups + group]: the per-key-tile partial maxima from which
// the attention kernel forms its softmax bound and picks its exponent tier (K_p rows have
// rp channels, rp = 0 for no positional part). The norms come from the registers that
// carry the rows, so K_c and V are read once.
__global__ __launch_bounds__(256) void gather_kv_bound_kernel(PixelMap pm, int N, int n_rows, int rp,
                                                              const bf16* __restrict__ k, const bf16* __restrict__ v,
                                                              const bf16* __restrict__ kp, bf16* __restrict__ kw,
                                                              bf16* __restrict__ vt, float* __restrict__ kmax2) {
  __shared__ bf16 tile[64][32 + 2];
  __shared__ float red[4], vred[4];
  const int groups = n_rows / 64;
  int u, gi;
  block_unit_group(groups, u, gi);
  const int g0 = gi * 64;
  const int tid = threadIdx.x;
  {
    const int tok = tid >> 2, c = tid & 3;
    const int t = g0 + tok;
    const int64_t ph = t < N ? pm.pixel_head(u, t) : 0;
    u32x4 kv = u32x4(0u), vv = u32x4(0u);
    if (t < N) {
      kv = *(const u32x4*)(k + ph * 32 + c * 8);
      vv = *(const u32x4*)(v + ph * 32 + c * 8);
    }
    *(u32x4*)(kw + ((int64_t)u * n_rows + t) * 32 + c * 8) = kv;
    float ss = 0.f;
    const bf16x8 ke = __builtin_bit_cast(bf16x8, kv);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf((float)ke[j], (float)ke[j], ss);
    if (t < N && c * 8 < rp) {   // rp <= 32: at most one positional chunk per lane
      const bf16x8 pe = __builtin_bit_cast(bf16x8, *(const u32x4*)(kp + (int64_t)t * rp + c * 8));
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf((float)pe[j], (float)pe[j], ss);
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);   // the token's |k_hat|^2 in its 4 lanes
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) ss = fmaxf(ss, __shfl_xor(ss, o));
    const bf16* pv = (const bf16*)&vv;
    float va = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) va = fmaxf(va, fabsf((float)pv[j]));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) va = fmaxf(va, __shfl_xor(va, o));
    if ((tid & 63) == 0) {
      red[tid >> 6] = ss;
      vred[tid >> 6] = va;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[tok][c * 8 + j] = pv[j];
  }
  __syncthreads();
  if (tid == 0) {
    kmax2[u * groups + gi] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    kmax2[(int64_t)gridDim.x + u * groups + gi] = fmaxf(fmaxf(vred[0], vred[1]), fmaxf(vred[2], vred[3]));
  }
  const int d = tid >> 3, pc = tid & 7;
  bf16 vals[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = pc * 8 + j;
    const int tok = (p & ~15) | kappa16(p & 15);
    vals[j] = tile[tok][d];
  }
  *(u32x4*)(vt + ((int64_t)u * 32 + d) * n_rows + g0 + pc * 8) = *(const u32x4*)vals;
}

// The bf16 backward's whole preparation in one pass. Block (unit, 64-token group):
// Q_c, K_c, dO and V -> the token-major rows layout (the Q_c and Q_p rows pre-scaled to
// bf16(c q) with c = scale log2(e) exactly as the forward rounds them, so both backward
// kernels form the forward's scores), and per row the negated softmax statistics the MFMA
// kernels add: -D with D = sum_c dO O, and -LSE2 = -LSE log2(e) (rows >= N: 0 and -inf,
// so P = 0). D comes from the dO registers the gather already holds. Blocks of unit 0 also
// pack Q_p and K_p for their 64 tokens (rows zero-padded to rp channels). The kernels take
// their channel-major operands from these rows by transposing LDS reads.
__global__ __launch_bounds__(256) void gather_bwd_kernel(BwdGather a) {
  const int groups = a.n_rows / 64;
  int u, gi;
  block_unit_group(groups, u, gi);
  const int g0 = gi * 64;
  const int tid = threadIdx.x;
  const int N = a.N, n_rows = a.n_rows;
  {
    const int tok = tid >> 2, c = tid & 3;
    const int t = g0 + tok;
    const int64_t ph = t < N ? a.pm.pixel_head(u, t) : 0;
    u32x4 x[4] = {u32x4(0u), u32x4(0u), u32x4(0u), u32x4(0u)}, ov = u32x4(0u);   // q, k, do, v; o
    if (t < N) {
      const int64_t off = ph * 32 + c * 8;
      x[0] = *(const u32x4*)(a.q + off);
      x[2] = *(const u32x4*)(a.d_o + off);
      ov = *(const u32x4*)(a.o + off);
      if (a.kw) {
        x[1] = *(const u32x4*)(a.k + off);
        x[3] = *(const u32x4*)(a.v + off);
      }
    }
    const int64_t row = ((int64_t)u * n_rows + t) * 32 + c * 8;
    {
      // Q_c rows pre-scaled into the log2 domain, rounded as the forward rounds them
      const bf16x8 qe = __builtin_bit_cast(bf16x8, x[0]);
      bf16x8 qs;
#pragma unroll
      for (int j = 0; j < 8; ++j) qs[j] = f32_to_bf16((float)qe[j] * a.c);
      *(bf16x8*)(a.qw + row) = qs;
    }
    *(u32x4*)(a.dow + row) = x[2];
    if (a.kw) {   // windows the kernels cannot read in the maps
      *(u32x4*)(a.kw + row) = x[1];
      *(u32x4*)(a.vw + row) = x[3];
    }
    const bf16x8 de = __builtin_bit_cast(bf16x8, x[2]), oe = __builtin_bit_cast(bf16x8, ov);
    float dsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) dsum = fmaf((float)de[j], (float)oe[j], dsum);
    dsum += __shfl_xor(dsum, 1);
    dsum += __shfl_xor(dsum, 2);
    if (c == 0) {
      const int64_t i = (int64_t)u * n_rows + t;
      a.dd[i] = t < N ? -dsum : 0.f;
      a.lse2[i] = t < N ? -(a.lse[ph] * 1.44269504088896340736f) : -INFINITY;
    }
  }
  if (u == 0) {   // positional tokens of this group: rows
    for (int i = tid; i < 64 * a.rp; i += 256) {
      const int tl = i / a.rp, j = i - tl * a.rp, t = g0 + tl;
      const bool ok = t < N && j < a.r;
      const bf16 qv = ok ? a.q_p[(int64_t)t * a.r + j] : (bf16)0.f;
      const bf16 kv = ok ? a.k_p[(int64_t)t * a.r + j] : (bf16)0.f;
      a.qp[(int64_t)t * a.rp + j] = f32_to_bf16((float)qv * a.c);   // pre-scaled, as Q_c
      a.kp[(int64_t)t * a.rp + j] = kv;
    }
  }
}

template <typename InT, typename OutT>
__global__ void pack_pos_kernel(int N, int n_rows, int r, int rp, const InT* __restrict__ in, OutT* __restrict__ out) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_rows * rp) return;
  int t = i / rp, j = i - t * rp;
  float v = (t < N && j < r) ? (float)in[(int64_t)t * r + j] : 0.f;
  out[i] = (OutT)v;
}

ChunkGeom chunk_geom(const Geom& g, int esize, int n_rows) {
  ChunkGeom c;
  c.H = g.H; c.W = g.W; c.heads = g.heads; c.w = g.w; c.nwy = g.nwy; c.nwx = g.nwx;
  c.cpr = g.d_c * esize / 16;
  c.n_rows = n_rows;
  c.N = g.N;
  return c;
}

int64_t blocks_for(int64_t n, int threads) { return (n + threads - 1) / threads; }

}  // namespace

hipError_t launch_partition(const Geom& g, int esize, const void* x, void* xw, hipStream_t stream) {
  ChunkGeom c = chunk_geom(g, esize, g.n_rows);
  int64_t map_chunks = (int64_t)g.B * g.H * g.W * g.heads * c.cpr;
  int64_t pad_chunks = (int64_t)g.units * (g.n_rows - g.N) * c.cpr;
  int64_t n = map_chunks + pad_chunks;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks_for(n, 256)), dim3(256), 0, stream, c, map_chunks,
                     pad_chunks, (const u32x4*)x, (u32x4*)xw);
  return hipGetLastError();
}

hipError_t launch_gather_kv_bound(const Geom& g, int rp, const void* k, const void* v, const void* kp, void* kw,
                                  void* vt, float* kmax2, hipStream_t stream) {
  if (g.units == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kv_bound_kernel, dim3((unsigned)((int64_t)g.units * (g.n_rows / 64))), dim3(256), 0,
                     stream, make_pixel_map(g), g.N, g.n_rows, rp, (const bf16*)k, (const bf16*)v, (const bf16*)kp,
                     (bf16*)kw, (bf16*)vt, kmax2);
  return hipGetLastError();
}

hipError_t launch_gather_bwd(const BwdGather& a, int units, hipStream_t stream) {
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_bwd_kernel, dim3((unsigned)((int64_t)units * (a.n_rows / 64))), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_unpartition(const Geom& g, int esize, const void* xw, void* x, hipStream_t stream) {
  ChunkGeom c = chunk_geom(g, esize, g.n_rows);
  int64_t map_chunks = (int64_t)g.B * g.H * g.W * g.heads * c.cpr;
  if (map_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)blocks_for(map_chunks, 256)), dim3(256), 0, stream, c,
                     map_chunks, (const u32x4*)xw, (u32x4*)x);
  return hipGetLastError();
}

hipError_t launch_partition_plain(const Geom& g, int esize, const void* x, void* xw, hipStream_t stream) {
  ChunkGeom c = chunk_geom(g, esize, g.N);
  int64_t map_chunks = (int64_t)g.B * g.H * g.W * g.heads * c.cpr;
  if (map_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks_for(map_chunks, 256)), dim3(256), 0, stream, c,
                     map_chunks, (int64_t)0, (const u32x4*)x, (u32x4*)xw);
  return hipGetLastError();
}

hipError_t launch_unpartition_plain(const Geom& g, int esize, const void* xw, void* x, hipStream_t stream) {
  ChunkGeom c = chunk_geom(g, esize, g.N);
  int64_t map_chunks = (int64_t)g.B * g.H * g.W * g.heads * c.cpr;
  if (map_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)blocks_for(map_chunks, 256)), dim3(256), 0, stream, c,
                     map_chunks, (const u32x4*)xw, (u32x4*)x);
  return hipGetLastError();
}

hipError_t launch_pack_pos(int N, int n_rows, int r, int rp, int in_esize, const void* in, int out_esize, void* out,
                           hipStream_t stream) {
  const int n = n_rows * rp;
  dim3 grid((n + 255) / 256), block(256);
  if (in_esize == 4 && out_esize == 4)
    hipLaunchKernelGGL((pack_pos_kernel<float, float>), grid, block, 0, stream, N, n_rows, r, rp, (const float*)in, (float*)out);
  else if (in_esize == 2 && out_esize == 2)
    hipLaunchKernelGGL((pack_pos_kernel<bf16, bf16>), grid, block, 0, stream, N, n_rows, r, rp, (const bf16*)in, (bf16*)out);
  else if (in_esize == 4 && out_esize == 2)
    hipLaunchKernelGGL((pack_pos_kernel<float, bf16>), grid, block, 0, stream, N, n_rows, r, rp, (const float*)in, (bf16*)out);
  else
    hipLaunchKernelGGL((pack_pos_kernel<bf16, float>), grid, block, 0, stream, N, n_rows, r, rp, (const bf16*)in, (float*)out);
  return hipGetLastError();
}

}  // namespace rib
