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
#include "internal.hpp"

namespace rib {
namespace {

constexpr int kTokPerBlock = 16;
constexpr int kThreads = 256;

template <typename OutT>
__device__ __forceinline__ void store_out(OutT* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<bf16>(bf16* p, float v) { *p = f32_to_bf16(v); }

template <typename OutT>
__global__ __launch_bounds__(kThreads) void posgen_kernel(int w, int n_freq, int hidden, int rank,
                                                          const float* __restrict__ w1, const float* __restrict__ b1,
                                                          const float* __restrict__ w2, const float* __restrict__ b2,
                                                          OutT* __restrict__ qp, OutT* __restrict__ kp) {
  extern __shared__ float smem[];
  const int nf = 4 * n_freq;
  const int nout = 2 * rank;
  float* sW1t = smem;                       // [nf][hidden]   (transposed W1)
  float* sB1 = sW1t + nf * hidden;          // [hidden]
  float* sW2t = sB1 + hidden;               // [hidden][nout] (transposed W2)
  float* sB2 = sW2t + hidden * nout;        // [nout]
  float* sF = sB2 + nout;                   // [kTokPerBlock][nf]
  float* sH = sF + kTokPerBlock * nf;       // [kTokPerBlock][hidden]
  const int tid = threadIdx.x;
  for (int i = tid; i < hidden * nf; i += kThreads) {
    const int j = i / nf, f = i - j * nf;
    sW1t[f * hidden + j] = w1[i];
  }
  for (int i = tid; i < hidden; i += kThreads) sB1[i] = b1 ? b1[i] : 0.f;
  for (int i = tid; i < nout * hidden; i += kThreads) {
    const int o = i / hidden, j = i - o * hidden;
    sW2t[j * nout + o] = w2[i];
  }
  for (int i = tid; i < nout; i += kThreads) sB2[i] = b2 ? b2[i] : 0.f;

  const int N = w * w;
  const int t0 = blockIdx.x * kTokPerBlock;
  const int den = w - 1;
  const int mod = 2 * den;
  // phase 1: features of (token, frequency) pairs
  for (int i = tid; i < kTokPerBlock * n_freq; i += kThreads) {
    const int tl = i / n_freq, k = i - tl * n_freq;
    const int t = min(t0 + tl, N - 1);
    const int iy = t / w, ix = t - iy * w;
    const int nx = 2 * ix - den, ny = 2 * iy - den;
    // exact phase: (2^k * n) mod 2(w-1), non-negative; |2^k n| < 2^23 for w <= 256
    const int px = ((nx * (1 << k)) % mod + mod) % mod;
    const int py = ((ny * (1 << k)) % mod + mod) % mod;
    const float ax = (float)px / (float)den;  // angle / pi, in [0, 2)
    const float ay = (float)py / (float)den;
    float* f = sF + tl * nf;
    f[k] = sinpif(ax);
    f[n_freq + k] = cospif(ax);
    f[2 * n_freq + k] = sinpif(ay);
    f[3 * n_freq + k] = cospif(ay);
  }
  __syncthreads();
  // phase 2: hidden layer, GELU with the exact erf form
  const float kInvSqrt2 = 0.70710678118654752440f;
  for (int i = tid; i < kTokPerBlock * hidden; i += kThreads) {
    const int tl = i / hidden, j = i - tl * hidden;
    const float* f = sF + tl * nf;
    float acc = sB1[j];
    for (int q = 0; q < nf; ++q) acc = fmaf(sW1t[q * hidden + j], f[q], acc);
    sH[tl * hidden + j] = 0.5f * acc * (1.f + erff(acc * kInvSqrt2));
  }
  __syncthreads();
  // phase 3: outputs; the first rank go to Q_p, the next rank to K_p
  for (int i = tid; i < kTokPerBlock * nout; i += kThreads) {
    const int tl = i / nout, o = i - tl * nout;
    const int t = t0 + tl;
    if (t >= N) continue;
    const float* h = sH + tl * hidden;
    float acc = sB2[o];
    for (int j = 0; j < hidden; ++j) acc = fmaf(sW2t[j * nout + o], h[j], acc);
    if (o < rank) store_out<OutT>(qp + (int64_t)t * rank + o, acc);
    else store_out<OutT>(kp + (int64_t)t * rank + (o - rank), acc);
  }
}

}  // namespace

size_t posgen_lds_bytes(const rib_mlp_t& mlp) {
  const size_t nf = 4 * (size_t)mlp.n_freq, nout = 2 * (size_t)mlp.rank, hd = mlp.hidden;
  return sizeof(float) * (nf * hd + hd + hd * nout + nout + kTokPerBlock * nf + kTokPerBlock * hd);
}

hipError_t launch_posgen(int w, const rib_mlp_t& mlp, rib_dtype_t out_dtype, void* q_p, void* k_p,
                         hipStream_t stream) {
  const int N = w * w;
  const int blocks = (N + kTokPerBlock - 1) / kTokPerBlock;
  const size_t lds = posgen_lds_bytes(mlp);
  if (out_dtype == RIB_F32) {
    hipLaunchKernelGGL(posgen_kernel<float>, dim3(blocks), dim3(kThreads), lds, stream, w, mlp.n_freq,
                       mlp.hidden, mlp.rank, mlp.w1, mlp.b1, mlp.w2, mlp.b2, (float*)q_p, (float*)k_p);
  } else {
    hipLaunchKernelGGL(posgen_kernel<bf16>, dim3(blocks), dim3(kThreads), lds, stream, w, mlp.n_freq,
                       mlp.hidden, mlp.rank, mlp.w1, mlp.b1, mlp.w2, mlp.b2, (bf16*)q_p, (bf16*)k_p);
  }
  return hipGetLastError();
}

}  // namespace rib
