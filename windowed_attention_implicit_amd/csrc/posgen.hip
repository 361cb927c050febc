// Positional-token generation (RIB posgen) for gfx950.
//
// Each token of a w x w window gets the normalized coordinate
// c_i = (2i - (w-1)) / (w-1) per axis, is lifted by sin / cos at the
// frequencies 2^k pi, and passes through Linear -> GELU(erf) -> Linear to give
// its positional query and key tokens (Q_p, K_p). Sources: gist.science/de
// "Technische Zusammenfassung" §2.A.1-2 (normalized 2D coordinate in [-1, 1],
// Fourier features, lightweight MLP), gist.science/paper/2603.06738
// "Technical Summary" §2.A.1-2.
//
// Design: a 256-thread block handles 16 tokens. Phase 1 computes their
// Fourier features (one (token, frequency) pair per thread), phase 2 the
// hidden layer (one (token, hidden unit) pair per thread and step) and phase 3
// the outputs. The weights are staged once per block in LDS transposed
// (input-major), so the lanes of a wave, which differ in the output unit, read
// consecutive LDS words, while the token's features / hidden values are an LDS
// broadcast. The phase 2^k * n / (w-1) is reduced exactly in integer
// arithmetic (mod 2(w-1)) before sinpi/cospi, so the highest frequencies keep
// full float32 accuracy. The output is tiny and computed once per window size.
//
// Backward (weight gradients): the MLP is trained with the network, so the
// positional gradients dQ_p, dK_p continue by the chain rule through
// Linear -> GELU -> Linear: with z = W1 phi + b1, h = GELU(z) and
// d_out = [dQ_p | dK_p], dW2 = sum_t d_out h^T, db2 = sum_t d_out,
// dz = (W2^T d_out) * GELU'(z) with GELU'(z) = Phi(z) + z phi(z), dW1 =
// sum_t dz phi^T, db1 = sum_t dz. A block recomputes phi, z and h for tiles
// of up to 32 tokens and adds each tile's contributions into its own slot of
// partial sums (one thread per entry); a second kernel adds the partials of
// all blocks in a fixed order (deterministic, no atomics).
#include <algorithm>
#include <type_traits>

#include "internal.hpp"

namespace rib {
namespace {

constexpr int kTokPerBlock = 16;
constexpr int kThreads = 256;

// Features k, F + k, 2F + k, 3F + k of token t (sin / cos of 2^k pi x, then of
// 2^k pi y) into f[]. The phase (2^k n) mod 2(w-1) is reduced exactly in
// integers (|2^k n| < 2^23 for w <= 256), so sinpi / cospi see an angle / pi
// in [0, 2) with no rounding of large arguments.
__device__ __forceinline__ void fourier_pair(int w, int n_freq, int t, int k, float* f) {
  const int den = w - 1, mod = 2 * den;
  const int iy = t / w, ix = t - iy * w;
  const int nx = 2 * ix - den, ny = 2 * iy - den;
  const int px = ((nx * (1 << k)) % mod + mod) % mod;
  const int py = ((ny * (1 << k)) % mod + mod) % mod;
  const float ax = (float)px / (float)den;
  const float ay = (float)py / (float)den;
  f[k] = sinpif(ax);
  f[n_freq + k] = cospif(ax);
  f[2 * n_freq + k] = sinpif(ay);
  f[3 * n_freq + k] = cospif(ay);
}

template <typename OutT>
__device__ __forceinline__ void store_out(OutT* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<bf16>(bf16* p, float v) { *p = f32_to_bf16(v); }

// NF, HID, NOUT: the feature count 4F, hidden width and output width 2r when
// known at compile time (the configurations in use), 0 for the runtime values;
// fixed sizes let the loops unroll with immediate LDS offsets.
template <typename OutT, int NF, int HID, int NOUT>
__global__ __launch_bounds__(kThreads) void posgen_kernel(int w, int n_freq_arg, int hidden_arg, int rank_arg,
                                                          const float* __restrict__ w1, const float* __restrict__ b1,
                                                          const float* __restrict__ w2, const float* __restrict__ b2,
                                                          OutT* __restrict__ qp, OutT* __restrict__ kp) {
  extern __shared__ float smem[];
  const int n_freq = NF ? NF / 4 : n_freq_arg;
  const int nf = NF ? NF : 4 * n_freq_arg;
  const int hidden = HID ? HID : hidden_arg;
  const int nout = NOUT ? NOUT : 2 * rank_arg;
  const int rank = nout / 2;
  // transposed weights, rows padded by one word so that the staging stores of
  // consecutive threads (consecutive input index) fall in distinct banks
  const int ld1 = hidden + 1, ld2 = nout + 1;
  float* sW1t = smem;                       // [nf][hidden + 1]   (transposed W1)
  float* sB1 = sW1t + nf * ld1;             // [hidden]
  float* sW2t = sB1 + hidden;               // [hidden][nout + 1] (transposed W2)
  float* sB2 = sW2t + hidden * ld2;         // [nout]
  float* sF = sB2 + nout;                   // [kTokPerBlock][nf]
  float* sH = sF + kTokPerBlock * nf;       // [kTokPerBlock][hidden]
  const int tid = threadIdx.x;
  for (int i = tid; i < hidden * nf; i += kThreads) {
    const int j = i / nf, f = i - j * nf;
    sW1t[f * ld1 + j] = w1[i];
  }
  for (int i = tid; i < hidden; i += kThreads) sB1[i] = b1 ? b1[i] : 0.f;
  for (int i = tid; i < nout * hidden; i += kThreads) {
    const int o = i / hidden, j = i - o * hidden;
    sW2t[j * ld2 + o] = w2[i];
  }
  for (int i = tid; i < nout; i += kThreads) sB2[i] = b2 ? b2[i] : 0.f;

  const int N = w * w;
  const int t0 = blockIdx.x * kTokPerBlock;
  // phase 1: features of (token, frequency) pairs
  for (int i = tid; i < kTokPerBlock * n_freq; i += kThreads) {
    const int tl = i / n_freq, k = i - tl * n_freq;
    fourier_pair(w, n_freq, min(t0 + tl, N - 1), k, sF + tl * nf);
  }
  __syncthreads();
  // phase 2: hidden layer, GELU with the exact erf form
  const float kInvSqrt2 = 0.70710678118654752440f;
  auto hidden_unit = [&](int i) {
    const int tl = i / hidden, j = i - tl * hidden;
    const float* f = sF + tl * nf;
    float acc = sB1[j];
#pragma unroll
    for (int q = 0; q < nf; ++q) acc = fmaf(sW1t[q * ld1 + j], f[q], acc);
    sH[tl * hidden + j] = 0.5f * acc * (1.f + erff(acc * kInvSqrt2));
  };
  constexpr int kP2 = kTokPerBlock * HID;
  if constexpr (NF && HID && kP2 % kThreads == 0) {
#pragma unroll
    for (int m = 0; m < kP2 / kThreads; ++m) hidden_unit(tid + m * kThreads);
  } else {
    for (int i = tid; i < kTokPerBlock * hidden; i += kThreads) hidden_unit(i);
  }
  __syncthreads();
  // phase 3: outputs; the first rank go to Q_p, the next rank to K_p
  auto output_unit = [&](int i) {
    const int tl = i / nout, o = i - tl * nout;
    const int t = t0 + tl;
    const float* h = sH + tl * hidden;
    float acc = sB2[o];
#pragma unroll
    for (int j = 0; j < hidden; ++j) acc = fmaf(sW2t[j * ld2 + o], h[j], acc);
    if (t >= N) return;
    if (o < rank) store_out<OutT>(qp + (int64_t)t * rank + o, acc);
    else store_out<OutT>(kp + (int64_t)t * rank + (o - rank), acc);
  };
  constexpr int kP3 = kTokPerBlock * NOUT;
  if constexpr (HID && NOUT && kP3 % kThreads == 0) {
#pragma unroll
    for (int m = 0; m < kP3 / kThreads; ++m) output_unit(tid + m * kThreads);
  } else {
    for (int i = tid; i < kTokPerBlock * nout; i += kThreads) output_unit(i);
  }
}

// ------------------------------------------------------------ backward
constexpr int kBwdMaxTok = 32;    // tokens per tile, at most (fewer when the MLP is large)
constexpr int kBwdMaxBlocks = 1024;
constexpr int kBwdThreads = 1024;   // 4 waves per SIMD to hide LDS latency

__host__ __device__ inline int posgen_bwd_entries(int n_freq, int hidden, int rank) {
  return hidden * 4 * n_freq + hidden + 2 * rank * hidden + 2 * rank;
}

// One block: stage W1^T, b1, W2; for every tile of `tok` tokens it owns
// (tiles blockIdx.x, blockIdx.x + gridDim.x, ...) recompute phi, z, h and dz
// in LDS and add the tile's contributions to the block's own partial slot,
// laid out [dW1 hidden x 4F][db1 hidden][dW2 2r x hidden][db2 2r]. Every
// entry of the slot belongs to one thread, so the read-modify-writes need no
// synchronisation and their order is fixed.
// NF, HID, NOUT as for posgen_kernel (0: runtime sizes).
template <int TOK, int NF, int HID, int NOUT>
__global__ __launch_bounds__(kBwdThreads) void posgen_bwd_partial_kernel(int w, int n_freq_arg, int hidden_arg,
                                                                      int rank_arg, const float* __restrict__ w1,
                                                                      const float* __restrict__ b1,
                                                                      const float* __restrict__ w2,
                                                                      const float* __restrict__ dqp,
                                                                      const float* __restrict__ dkp,
                                                                      float* __restrict__ part) {
  extern __shared__ float smem[];
  constexpr int tok = TOK;
  const int n_freq = NF ? NF / 4 : n_freq_arg;
  const int nf = NF ? NF : 4 * n_freq_arg;
  const int hidden = HID ? HID : hidden_arg;
  const int nout = NOUT ? NOUT : 2 * rank_arg;
  const int rank = nout / 2;
  const int ld1 = hidden + 1;                // padded rows: conflict-free transposed staging
  float* sW1t = smem;                        // [nf][hidden + 1] (transposed W1)
  float* sB1 = sW1t + nf * ld1;              // [hidden]
  float* sW2 = sB1 + hidden;                 // [nout][hidden]
  float* sF = sW2 + nout * hidden;           // [tok][nf]      features
  float* sH = sF + tok * nf;                 // [tok][hidden]  GELU(z)
  float* sZ = sH + tok * hidden;             // [tok][hidden]  dz
  float* sD = sZ + tok * hidden;             // [tok][nout]    d_out
  const int tid = threadIdx.x;
  for (int i = tid; i < hidden * nf; i += kBwdThreads) {
    const int j = i / nf, f = i - j * nf;
    sW1t[f * ld1 + j] = w1[i];
  }
  for (int i = tid; i < hidden; i += kBwdThreads) sB1[i] = b1 ? b1[i] : 0.f;
  for (int i = tid; i < nout * hidden; i += kBwdThreads) sW2[i] = w2[i];

  const int N = w * w;
  const int ntiles = (N + tok - 1) / tok;
  const int n_w1 = hidden * nf, n_b1 = n_w1 + hidden, n_w2 = n_b1 + nout * hidden;
  float* out = part + (int64_t)blockIdx.x * posgen_bwd_entries(n_freq, hidden, rank);
  const float kInvSqrt2 = 0.70710678118654752440f;
  const float kInvSqrt2Pi = 0.39894228040143267794f;
  constexpr bool kFixed = NF && HID && NOUT;
  // Runs body(i) for i = tid, tid + kBwdThreads, ... < n: a fixed trip count (unrolled)
  // when n is a compile-time multiple of the block, a runtime loop otherwise.
  auto each = [&](auto cn, int n, auto&& body) {
    constexpr int kN = decltype(cn)::value;
    if constexpr (kN > 0 && kN % kBwdThreads == 0) {
#pragma unroll
      for (int m = 0; m < kN / kBwdThreads; ++m) body(tid + m * kBwdThreads);
    } else {
      for (int i = tid; i < n; i += kBwdThreads) body(i);
    }
  };
  using NZ = std::integral_constant<int, kFixed ? tok * HID : 0>;
  using NW1 = std::integral_constant<int, kFixed ? HID * NF : 0>;
  using NW2 = std::integral_constant<int, kFixed ? NOUT * HID : 0>;
  using NRT = std::integral_constant<int, 0>;

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int t0 = tile * tok;
    __syncthreads();   // the previous tile's LDS values are consumed (and the weights staged)
    for (int i = tid; i < tok * n_freq; i += kBwdThreads) {
      const int tl = i / n_freq, k = i - tl * n_freq;
      fourier_pair(w, n_freq, min(t0 + tl, N - 1), k, sF + tl * nf);
    }
    // d_out = [dQ_p | dK_p]; tokens past N contribute zero
    for (int i = tid; i < tok * nout; i += kBwdThreads) {
      const int tl = i / nout, o = i - tl * nout;
      const int t = t0 + tl;
      float v = 0.f;
      if (t < N) v = o < rank ? dqp[(int64_t)t * rank + o] : dkp[(int64_t)t * rank + (o - rank)];
      sD[i] = v;
    }
    __syncthreads();
    // z, h = GELU(z) = z Phi(z), dz = (W2^T d_out) * (Phi(z) + z phi(z))
    each(NZ{}, tok * hidden, [&](int i) {
      const int tl = i / hidden, j = i - tl * hidden;
      const float* f = sF + tl * nf;
      float z = sB1[j];
#pragma unroll 16
      for (int q = 0; q < nf; ++q) z = fmaf(sW1t[q * ld1 + j], f[q], z);
      const float cdf = 0.5f * (1.f + erff(z * kInvSqrt2));
      const float pdf = kInvSqrt2Pi * expf(-0.5f * z * z);
      const float* d = sD + tl * nout;
      float dh = 0.f;
#pragma unroll 16
      for (int o = 0; o < nout; ++o) dh = fmaf(d[o], sW2[o * hidden + j], dh);
      sH[i] = z * cdf;
      sZ[i] = dh * fmaf(z, pdf, cdf);
    });
    __syncthreads();
    // the tile's contributions, one region of the slot at a time (dW1, db1, dW2, db2), so
    // each loop has fixed strides; lanes differ in the inner index (consecutive LDS words)
    const bool first = tile == (int)blockIdx.x;
    auto put = [&](int e, float a) { out[e] = first ? a : out[e] + a; };
    each(NW1{}, hidden * nf, [&](int e) {   // dW1[j][f] += sum_t dz[t][j] phi[t][f]
      const int j = e / nf, f = e - j * nf;
      float a = 0.f;
#pragma unroll
      for (int tl = 0; tl < tok; ++tl) a = fmaf(sZ[tl * hidden + j], sF[tl * nf + f], a);
      put(e, a);
    });
    each(NRT{}, hidden, [&](int j) {        // db1[j] += sum_t dz[t][j]
      float a = 0.f;
#pragma unroll
      for (int tl = 0; tl < tok; ++tl) a += sZ[tl * hidden + j];
      put(n_w1 + j, a);
    });
    each(NW2{}, nout * hidden, [&](int e) {  // dW2[o][j] += sum_t d_out[t][o] h[t][j]
      const int o = e / hidden, j = e - o * hidden;
      float a = 0.f;
#pragma unroll
      for (int tl = 0; tl < tok; ++tl) a = fmaf(sD[tl * nout + o], sH[tl * hidden + j], a);
      put(n_b1 + e, a);
    });
    each(NRT{}, nout, [&](int o) {          // db2[o] += sum_t d_out[t][o]
      float a = 0.f;
#pragma unroll
      for (int tl = 0; tl < tok; ++tl) a += sD[tl * nout + o];
      put(n_w2 + o, a);
    });
  }
}

// Sums the per-block partials of every entry in a fixed order and scatters them
// to dW1, db1, dW2, db2 (db1 / db2 may be null). A block covers 64 entries; wave
// s adds the partials of blocks [s nb / 4, (s + 1) nb / 4) in block order (lanes
// read consecutive entries), and the four range sums are added in wave order.
__global__ __launch_bounds__(kThreads) void posgen_bwd_reduce_kernel(int nblk, int hidden, int nf, int nout,
                                                                     const float* __restrict__ part,
                                                                     float* __restrict__ dw1, float* __restrict__ db1,
                                                                     float* __restrict__ dw2, float* __restrict__ db2) {
  __shared__ float red[kThreads / 64][64];
  const int per = hidden * nf + hidden + nout * hidden + nout;
  const int lane = threadIdx.x & 63, s = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int b0 = (int)((int64_t)nblk * s / (kThreads / 64)), b1 = (int)((int64_t)nblk * (s + 1) / (kThreads / 64));
  float acc = 0.f;
  if (e < per) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {   // loads fetched 8 at a time so they overlap
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = part[(int64_t)(b + i) * per + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += v[i];
    }
    for (; b < b1; ++b) acc += part[(int64_t)b * per + e];
  }
  red[s][lane] = acc;
  __syncthreads();
  if (s != 0 || e >= per) return;
  acc = red[0][lane];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) acc += red[i][lane];
  int k = e;
  if (k < hidden * nf) { dw1[k] = acc; return; }
  k -= hidden * nf;
  if (k < hidden) { if (db1) db1[k] = acc; return; }
  k -= hidden;
  if (k < nout * hidden) { dw2[k] = acc; return; }
  k -= nout * hidden;
  if (db2) db2[k] = acc;
}

size_t bwd_lds_for(const rib_mlp_t& mlp, int tok) {
  const size_t nf = 4 * (size_t)mlp.n_freq, nout = 2 * (size_t)mlp.rank, hd = mlp.hidden;
  return sizeof(float) * (nf * (hd + 1) + hd + nout * hd + (size_t)tok * (nf + 2 * hd + nout));
}

// Tokens per tile: the largest power of two <= 32 whose tile fits 64 KB with
// the weights, halved further (down to 1) while that leaves fewer than 128
// tiles, so small windows still spread over many CUs (0: nothing fits).
int bwd_tile_tokens(const rib_mlp_t& mlp, int w) {
  int tok = kBwdMaxTok;
  while (tok >= 1 && bwd_lds_for(mlp, tok) > 65536) tok /= 2;
  while (tok > 1 && (w * w + tok - 1) / tok < 128) tok /= 2;
  return tok;
}

int bwd_blocks(int w, int tok) { return std::min((w * w + tok - 1) / tok, kBwdMaxBlocks); }

}  // namespace

size_t posgen_bwd_lds_bytes(const rib_mlp_t& mlp) { return bwd_lds_for(mlp, 1); }

size_t posgen_bwd_workspace_bytes(int w, const rib_mlp_t& mlp) {
  const int tok = std::max(bwd_tile_tokens(mlp, w), 1);
  return sizeof(float) * (size_t)bwd_blocks(w, tok) * posgen_bwd_entries(mlp.n_freq, mlp.hidden, mlp.rank);
}

hipError_t launch_posgen_bwd(int w, const rib_mlp_t& mlp, const float* dq_p, const float* dk_p, float* dw1,
                             float* db1, float* dw2, float* db2, void* workspace, hipStream_t stream) {
  const int tok = bwd_tile_tokens(mlp, w);
  if (tok == 0) return hipErrorInvalidValue;
  const int nblk = bwd_blocks(w, tok);
  const int nf = 4 * mlp.n_freq, nout = 2 * mlp.rank;
  float* part = (float*)workspace;
  const size_t lds = bwd_lds_for(mlp, tok);
#define RIB_PGB_LAUNCH(T, NF, HID, NOUT)                                                                   \
  hipLaunchKernelGGL((posgen_bwd_partial_kernel<T, NF, HID, NOUT>), dim3(nblk), dim3(kBwdThreads), lds, stream, \
                     w, mlp.n_freq, mlp.hidden, mlp.rank, mlp.w1, mlp.b1, mlp.w2, dq_p, dk_p, part)
#define RIB_PGB_TOK(NF, HID, NOUT)                \
  switch (tok) {                                  \
    case 32: RIB_PGB_LAUNCH(32, NF, HID, NOUT); break; \
    case 16: RIB_PGB_LAUNCH(16, NF, HID, NOUT); break; \
    case 8: RIB_PGB_LAUNCH(8, NF, HID, NOUT); break;   \
    case 4: RIB_PGB_LAUNCH(4, NF, HID, NOUT); break;   \
    case 2: RIB_PGB_LAUNCH(2, NF, HID, NOUT); break;   \
    default: RIB_PGB_LAUNCH(1, NF, HID, NOUT); break;  \
  }
  // the 16-frequency, 64-wide MLP with r = 8 or 16 has fixed-size instances
  const bool fixed = mlp.n_freq == 16 && mlp.hidden == 64 && (mlp.rank == 8 || mlp.rank == 16);
  if (fixed && mlp.rank == 8) RIB_PGB_TOK(64, 64, 16)
  else if (fixed) RIB_PGB_TOK(64, 64, 32)
  else RIB_PGB_TOK(0, 0, 0)
#undef RIB_PGB_TOK
#undef RIB_PGB_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per = posgen_bwd_entries(mlp.n_freq, mlp.hidden, mlp.rank);
  hipLaunchKernelGGL(posgen_bwd_reduce_kernel, dim3((per + 63) / 64), dim3(kThreads), 0, stream,
                     nblk, mlp.hidden, nf, nout, part, dw1, db1, dw2, db2);
  return hipGetLastError();
}

size_t posgen_lds_bytes(const rib_mlp_t& mlp) {
  const size_t nf = 4 * (size_t)mlp.n_freq, nout = 2 * (size_t)mlp.rank, hd = mlp.hidden;
  return sizeof(float) * (nf * (hd + 1) + hd + hd * (nout + 1) + nout + kTokPerBlock * nf + kTokPerBlock * hd);
}

hipError_t launch_posgen(int w, const rib_mlp_t& mlp, rib_dtype_t out_dtype, void* q_p, void* k_p,
                         hipStream_t stream) {
  const int N = w * w;
  const int blocks = (N + kTokPerBlock - 1) / kTokPerBlock;
  const size_t lds = posgen_lds_bytes(mlp);
#define RIB_POSGEN(T, NF, HID, NOUT)                                                                            \
  hipLaunchKernelGGL((posgen_kernel<T, NF, HID, NOUT>), dim3(blocks), dim3(kThreads), lds, stream, w, mlp.n_freq, \
                     mlp.hidden, mlp.rank, mlp.w1, mlp.b1, mlp.w2, mlp.b2, (T*)q_p, (T*)k_p)
  // the 16-frequency, 64-wide MLP with r = 8 or 16 has fixed-size instances
  const bool fixed = mlp.n_freq == 16 && mlp.hidden == 64 && (mlp.rank == 8 || mlp.rank == 16);
  if (out_dtype == RIB_F32) {
    if (fixed && mlp.rank == 8) RIB_POSGEN(float, 64, 64, 16);
    else if (fixed) RIB_POSGEN(float, 64, 64, 32);
    else RIB_POSGEN(float, 0, 0, 0);
  } else {
    if (fixed && mlp.rank == 8) RIB_POSGEN(bf16, 64, 64, 16);
    else if (fixed) RIB_POSGEN(bf16, 64, 64, 32);
    else RIB_POSGEN(bf16, 0, 0, 0);
  }
#undef RIB_POSGEN
  return hipGetLastError();
}

}  // namespace rib
