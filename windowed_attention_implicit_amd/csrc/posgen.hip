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
// Design: one thread per token, weights staged once per block in LDS (every
// lane reads the same weight at the same time: an LDS broadcast). The phase
// 2^k * n / (w-1) is reduced exactly in integer arithmetic (mod 2(w-1)) before
// sinpi/cospi, so the highest frequencies keep full float32 accuracy. The
// output is tiny and computed once per window size.
#include "internal.hpp"

namespace rib {
namespace {

constexpr int kMaxFreq = 16;
constexpr int kMaxFeat = 4 * kMaxFreq;
constexpr int kMaxOut = 64;  // 2 * max rank

template <typename OutT>
__device__ __forceinline__ void store_out(OutT* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<bf16>(bf16* p, float v) { *p = f32_to_bf16(v); }

template <typename OutT>
__global__ __launch_bounds__(64) void posgen_kernel(int w, int n_freq, int hidden, int rank,
                                                    const float* __restrict__ w1, const float* __restrict__ b1,
                                                    const float* __restrict__ w2, const float* __restrict__ b2,
                                                    OutT* __restrict__ qp, OutT* __restrict__ kp) {
  extern __shared__ float smem[];
  const int nf = 4 * n_freq;
  const int nout = 2 * rank;
  float* sW1 = smem;                  // [hidden][nf]
  float* sB1 = sW1 + hidden * nf;     // [hidden]
  float* sW2 = sB1 + hidden;          // [nout][hidden]
  float* sB2 = sW2 + nout * hidden;   // [nout]
  for (int i = threadIdx.x; i < hidden * nf; i += blockDim.x) sW1[i] = w1[i];
  for (int i = threadIdx.x; i < hidden; i += blockDim.x) sB1[i] = b1 ? b1[i] : 0.f;
  for (int i = threadIdx.x; i < nout * hidden; i += blockDim.x) sW2[i] = w2[i];
  for (int i = threadIdx.x; i < nout; i += blockDim.x) sB2[i] = b2 ? b2[i] : 0.f;
  __syncthreads();

  const int N = w * w;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N) return;
  const int iy = t / w, ix = t - iy * w;
  const int den = w - 1;
  const int mod = 2 * den;
  const int nx = 2 * ix - den, ny = 2 * iy - den;

  float feat[kMaxFeat];
#pragma unroll
  for (int k = 0; k < kMaxFreq; ++k) {
    if (k < n_freq) {
      // exact phase: (2^k * n) mod 2(w-1), non-negative; |2^k n| < 2^23 for w <= 256
      int px = ((nx * (1 << k)) % mod + mod) % mod;
      int py = ((ny * (1 << k)) % mod + mod) % mod;
      float ax = (float)px / (float)den;  // angle / pi, in [0, 2)
      float ay = (float)py / (float)den;
      feat[k] = sinpif(ax);
      feat[n_freq + k] = cospif(ax);
      feat[2 * n_freq + k] = sinpif(ay);
      feat[3 * n_freq + k] = cospif(ay);
    }
  }

  float out[kMaxOut];
#pragma unroll
  for (int o = 0; o < kMaxOut; ++o) out[o] = (o < nout) ? sB2[o] : 0.f;

  const float kInvSqrt2 = 0.70710678118654752440f;
  for (int j = 0; j < hidden; ++j) {
    const float* wr = sW1 + j * nf;
    float acc = sB1[j];
#pragma unroll
    for (int i = 0; i < kMaxFeat; ++i)
      if (i < nf) acc = fmaf(wr[i], feat[i], acc);
    const float h = 0.5f * acc * (1.f + erff(acc * kInvSqrt2));
#pragma unroll
    for (int o = 0; o < kMaxOut; ++o)
      if (o < nout) out[o] = fmaf(sW2[o * hidden + j], h, out[o]);
  }
#pragma unroll
  for (int o = 0; o < kMaxOut; ++o) {
    if (o < rank) store_out<OutT>(qp + (int64_t)t * rank + o, out[o]);
    else if (o < nout) store_out<OutT>(kp + (int64_t)t * rank + (o - rank), out[o]);
  }
}

}  // namespace

hipError_t launch_posgen(int w, const rib_mlp_t& mlp, rib_dtype_t out_dtype, void* q_p, void* k_p,
                         hipStream_t stream) {
  const int N = w * w;
  const int threads = 64;
  const int blocks = (N + threads - 1) / threads;
  const size_t lds = sizeof(float) * ((size_t)mlp.hidden * 4 * mlp.n_freq + mlp.hidden +
                                      (size_t)2 * mlp.rank * mlp.hidden + 2 * mlp.rank);
  if (out_dtype == RIB_F32) {
    hipLaunchKernelGGL(posgen_kernel<float>, dim3(blocks), dim3(threads), lds, stream, w, mlp.n_freq,
                       mlp.hidden, mlp.rank, mlp.w1, mlp.b1, mlp.w2, mlp.b2, (float*)q_p, (float*)k_p);
  } else {
    hipLaunchKernelGGL(posgen_kernel<bf16>, dim3(blocks), dim3(threads), lds, stream, w, mlp.n_freq,
                       mlp.hidden, mlp.rank, mlp.w1, mlp.b1, mlp.w2, mlp.b2, (bf16*)q_p, (bf16*)k_p);
  }
  return hipGetLastError();
}

}  // namespace rib
