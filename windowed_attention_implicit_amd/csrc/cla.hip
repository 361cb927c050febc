// Convolutional local attention (CLA) gate for gfx950: G = sigmoid(PW_1x1(DW_3x3(X))) on a
// [B, H, W, C] map, the gating map that modulates the attention output (O' = O * G) in the
// pages' description of CLA (gist.science/paper/2603.06738, "Technical Summary" §2.B: depth-wise
// conv, point-wise conv and sigmoid; the German summary §2.B: O' = O (.) G; the Chinese summary
// §2.B: 3x3 depth-wise and 1x1 point-wise).
//
// bf16 kernel (persistent workgroups, one wave per 16 output channels):
//  * A tile is one row segment of 32 pixels with all C channels: in the map that is one
//    contiguous run, so the three halo rows (34 pixels each) load with 16-byte coalesced
//    reads and the gate tile stores the same way (staged through LDS). The next tile's halo
//    is loaded into registers while the current one is computed (the LDS-only barriers leave
//    those loads in flight). Each XCD walks its own contiguous band of tiles, so the rows a
//    tile shares with the tiles above and below it are L2 hits on that XCD.
//  * Depth-wise 3x3 on the vector unit in fp32: a thread owns two adjacent channels and
//    32 C / (2 threads) consecutive pixels (4 at C = 192); a 3 x 3 window of halo values slides
//    along them. Taps and biases come from a tap-major LDS table read per tile, which leaves
//    the registers for two workgroups per CU.
//  * Point-wise 1x1 on the matrix unit: G^T[out][px] = W_pw[out][:] . D[px][:] as
//    v_mfma_f32_16x16x32_bf16 over 16 outputs x 2 blocks of 16 pixels per wave (independent
//    accumulators, so consecutive MFMAs do not wait on each other). Each wave keeps its 16 rows
//    of W_pw as bf16 A fragments in registers for the whole launch; D (bf16) is read from LDS
//    as the B operand one K-step ahead of its use. With C/16 waves per workgroup (12 at
//    C = 192) three waves share each SIMD, so one wave's LDS latency hides behind another's
//    MFMAs.
//  * Sigmoid in fp32 on the accumulator, rounded once to bf16.
#include <algorithm>

#include "internal.hpp"

namespace rib {
namespace {

constexpr int kGatePx = 32;   // pixels per tile (one MFMA column block)
constexpr int kXcds = 8;      // accelerator dies; workgroups are dealt to them round-robin

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS operations, not for its
// global loads (the release fence of __syncthreads would also wait for the next tile's halo
// loads, which are meant to stay in flight across the barrier). The memory clobber keeps the
// compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float sigmoid_fast(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float sigmoid_exact(float z) { return 1.0f / (1.0f + expf(-z)); }

template <int CB>  // C = 32 CB channels; one wave per 16 output channels
__global__ __launch_bounds__(128 * CB) void cla_gate_bf16_kernel(GateArgs a) {
  constexpr int C = 32 * CB;
  constexpr int KS = C / 32;                 // MFMA K-steps (32 channels) of the point-wise conv
  constexpr int NT = 128 * CB;
  constexpr int HP = kGatePx + 2;            // halo row width in pixels
  constexpr int DROW = C + 8;                // padded LDS row (bf16) of D and of the staged gate
  static_assert(NT % (C / 2) == 0 && kGatePx % (NT / (C / 2)) == 0, "thread layout of the depth-wise stage");
  constexpr int kPxGroups = NT / (C / 2);    // pixel groups of the depth-wise stage
  constexpr int kPxPerThread = kGatePx / kPxGroups;
  __shared__ bf16 sX[3 * HP * C];            // halo rows y-1, y, y+1; later the staged gate tile
  __shared__ bf16 sD[kGatePx * DROW];        // depth-wise output, [px][C] (+ pad)
  __shared__ float sTap[20][C / 2];          // [9 taps of the even channel, 9 of the odd, 2 biases][pair]:
                                             // lanes (consecutive pairs) read consecutive words
  __shared__ float sBpw[C];                  // point-wise bias
  static_assert(3 * HP * C >= kGatePx * DROW, "the gate tile reuses the halo buffer");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  // point-wise weights of this wave's 16 output rows as 16x16x32 A fragments: lane l holds
  // row l % 16, channels 32 s + 8 (l / 16) + j
  const int l16 = lane & 15, quad = lane >> 4;
  bf16x8 wa[KS];
  {
    const float* wrow = a.w_pw + (int64_t)(16 * wave + l16) * C;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) wa[s][j] = f32_to_bf16(wrow[32 * s + 8 * quad + j]);
  }
  // biases and depth-wise taps live in LDS (re-read per tile) to keep registers for two
  // workgroups per CU
  for (int i = tid; i < C; i += NT) {
    sBpw[i] = a.b_pw ? a.b_pw[i] : 0.f;
    const int pr = i >> 1, e = i & 1;
#pragma unroll
    for (int k = 0; k < 9; ++k) sTap[9 * e + k][pr] = a.w_dw[i * 9 + k];
    sTap[18 + e][pr] = a.b_dw ? a.b_dw[i] : 0.f;
  }
  __syncthreads();
  const int cp = tid % (C / 2), pg = tid / (C / 2);

  const bf16* x = (const bf16*)a.x;
  bf16* gout = (bf16*)a.g;
  const int H = a.H, W = a.W;
  const int ntx = (W + kGatePx - 1) / kGatePx;
  const int ntiles = a.B * H * ntx;
  // halo of a tile: chunk i (16 bytes) of row r, pixel p, channel chunk k sits at sX + 8 i
  constexpr int kChunksPerPx = C / 8;
  constexpr int kHaloChunks = 3 * HP * kChunksPerPx;
  constexpr int kLoads = (kHaloChunks + NT - 1) / NT;
  u32x4 pre[kLoads];
  auto fetch = [&](int tile) {
    const int xt = tile % ntx, by = tile / ntx, y = by % H, x0 = xt * kGatePx;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int i = tid + j * NT;
      const int r = i / (HP * kChunksPerPx);
      const int rr = i - r * (HP * kChunksPerPx);
      const int p = rr / kChunksPerPx, k = rr - p * kChunksPerPx;
      const int yy = y + r - 1, xx = x0 + p - 1;
      pre[j] = u32x4(0u);
      if (i < kHaloChunks && yy >= 0 && yy < H && xx >= 0 && xx < W)
        pre[j] = *(const u32x4*)(x + ((int64_t)(by + r - 1) * W + xx) * C + 8 * k);
    }
  };
  // workgroup b runs on XCD b % 8 (round-robin dispatch); the grid is a multiple of 8
  const int xcd = blockIdx.x % kXcds, lw = blockIdx.x / kXcds, nw = gridDim.x / kXcds;
  const int band = (ntiles + kXcds - 1) / kXcds;
  const int t_end = min(ntiles, (xcd + 1) * band);
  const int t_first = xcd * band + lw;
  if (t_first < t_end) fetch(t_first);
  for (int tile = t_first; tile < t_end; tile += nw) {
    const int xt = tile % ntx;
    const int by = tile / ntx;               // b * H + y
    const int x0 = xt * kGatePx;
    // ---- halo rows (zero outside the map) from the registers into LDS; then start the next tile's
    lds_barrier();                            // the previous tile's gate tile has been copied out
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int i = tid + j * NT;
      if (i < kHaloChunks) *(u32x4*)&sX[8 * i] = pre[j];
    }
    lds_barrier();
    if (tile + nw < t_end) fetch(tile + nw);
    // ---- depth-wise 3x3 (fp32), rounded to bf16 into D; a 3 x 3 window of halo values slides
    // along the thread's pixels (three new LDS reads per pixel)
    {
      const int px0 = pg * kPxPerThread;
      float xw[3][3][2];
#pragma unroll
      for (int ky = 0; ky < 3; ++ky)
#pragma unroll
        for (int kx = 0; kx < 2; ++kx) {
          const bf16x2 xv = *(const bf16x2*)&sX[(ky * HP + px0 + kx) * C + 2 * cp];
          xw[ky][kx + 1][0] = (float)xv[0];
          xw[ky][kx + 1][1] = (float)xv[1];
        }
#pragma unroll
      for (int i = 0; i < kPxPerThread; ++i) {
        const int px = px0 + i;
#pragma unroll
        for (int ky = 0; ky < 3; ++ky) {
          const bf16x2 xv = *(const bf16x2*)&sX[(ky * HP + px + 2) * C + 2 * cp];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            xw[ky][0][e] = xw[ky][1][e];
            xw[ky][1][e] = xw[ky][2][e];
            xw[ky][2][e] = (float)xv[e];
          }
        }
        float d0 = sTap[18][cp], d1 = sTap[19][cp];
#pragma unroll
        for (int ky = 0; ky < 3; ++ky)
#pragma unroll
          for (int kx = 0; kx < 3; ++kx) {
            d0 = fmaf(sTap[3 * ky + kx][cp], xw[ky][kx][0], d0);
            d1 = fmaf(sTap[9 + 3 * ky + kx][cp], xw[ky][kx][1], d1);
          }
        bf16x2 dv;
        dv[0] = f32_to_bf16(d0);
        dv[1] = f32_to_bf16(d1);
        *(bf16x2*)&sD[px * DROW + 2 * cp] = dv;
      }
    }
    lds_barrier();
    // ---- point-wise 1x1 on MFMA: block pb = outputs 16 wave + [0, 16) x pixels 16 pb + [0, 16);
    // lane l holds outputs 4 (l / 16) + v of the block for pixel l % 16. The accumulators start
    // at the point-wise bias.
    f32x4 acc[2];
    {
      const f32x4 b4 = *(const f32x4*)&sBpw[16 * wave + 4 * quad];
      acc[0] = b4;
      acc[1] = b4;
    }
    auto bfrag = [&](int pb, int s) {
      return *(const bf16x8*)&sD[(16 * pb + l16) * DROW + 32 * s + 8 * quad];
    };
    bf16x8 bcur[2] = {bfrag(0, 0), bfrag(1, 0)};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 bnext[2];
      if (s + 1 < KS) {
        bnext[0] = bfrag(0, s + 1);
        bnext[1] = bfrag(1, s + 1);
      }
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
        acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[s], bcur[pb], acc[pb], 0, 0, 0);
      if (s + 1 < KS) {
        bcur[0] = bnext[0];
        bcur[1] = bnext[1];
      }
    }
    // ---- sigmoid; stage the gate tile [px][C] in the halo buffer (free since the last barrier)
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      bf16 o4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = f32_to_bf16(sigmoid_fast(acc[pb][i]));
      *(uint2*)&sX[(16 * pb + l16) * DROW + 16 * wave + 4 * quad] = *(const uint2*)o4;
    }
    lds_barrier();
    // ---- coalesced copy-out of the pixels inside the map
    const int npx = min(kGatePx, W - x0);
    bf16* gdst = gout + ((int64_t)by * W + x0) * C;
    for (int i = tid; i < npx * kChunksPerPx; i += NT) {
      const int p = i / kChunksPerPx, k = i - p * kChunksPerPx;
      *(u32x4*)(gdst + (int64_t)p * C + 8 * k) = *(const u32x4*)&sX[p * DROW + 8 * k];
    }
  }
}

// float32 gate: a workgroup per 32-pixel row segment; depth-wise into LDS, then one thread per
// (pixel, output channel) dot product over the C inputs. Correctness-sized work.
__global__ __launch_bounds__(256) void cla_gate_f32_kernel(GateArgs a) {
  extern __shared__ float sDf[];              // [kGatePx][C]
  const int C = a.C, H = a.H, W = a.W;
  const int ntx = (W + kGatePx - 1) / kGatePx;
  const int xt = blockIdx.x % ntx, by = blockIdx.x / ntx, y = by % H;
  const int x0 = xt * kGatePx;
  const float* x = (const float*)a.x;
  for (int i = threadIdx.x; i < kGatePx * C; i += 256) {
    const int px = i / C, c = i - px * C;
    const int xx = x0 + px;
    float d = a.b_dw ? a.b_dw[c] : 0.f;
    if (xx < W)
      for (int ky = 0; ky < 3; ++ky)
        for (int kx = 0; kx < 3; ++kx) {
          const int yy = y + ky - 1, xs = xx + kx - 1;
          if (yy >= 0 && yy < H && xs >= 0 && xs < W)
            d = fmaf(a.w_dw[c * 9 + 3 * ky + kx], x[((int64_t)(by + ky - 1) * W + xs) * C + c], d);
        }
    sDf[i] = d;
  }
  __syncthreads();
  float* g = (float*)a.g;
  for (int i = threadIdx.x; i < kGatePx * C; i += 256) {
    const int px = i / C, o = i - px * C;
    if (x0 + px >= W) continue;
    float z = a.b_pw ? a.b_pw[o] : 0.f;
    for (int c = 0; c < C; ++c) z = fmaf(a.w_pw[(int64_t)o * C + c], sDf[px * C + c], z);
    g[((int64_t)by * W + x0 + px) * C + o] = sigmoid_exact(z);
  }
}

template <int CB>
hipError_t launch_gate_cb(const GateArgs& a, int tiles, hipStream_t stream) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, cla_gate_bf16_kernel<CB>, 128 * CB, 0);
  if (e != hipSuccess) return e;
  const int64_t slots = (int64_t)std::max(cus, 1) * std::max(per_cu, 1);
  const int grid = (int)std::max<int64_t>(kXcds, std::min<int64_t>(tiles, slots) / kXcds * kXcds);
  hipLaunchKernelGGL(cla_gate_bf16_kernel<CB>, dim3(grid), dim3(128 * CB), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Up to 8 waves of 32 output channels: two waves per SIMD keep 256 VGPRs each for the
// register-resident point-wise weights.
bool cla_channels_supported(int C) { return C >= 32 && C <= 256 && C % 32 == 0; }

hipError_t launch_cla_gate(const GateArgs& a, int esize, hipStream_t stream) {
  const int ntx = (a.W + kGatePx - 1) / kGatePx;
  const int64_t tiles = (int64_t)a.B * a.H * ntx;
  if (tiles == 0) return hipSuccess;
  if (esize == 4) {
    hipLaunchKernelGGL(cla_gate_f32_kernel, dim3((unsigned)tiles), dim3(256), kGatePx * a.C * sizeof(float),
                       stream, a);
    return hipGetLastError();
  }
  switch (a.C / 32) {
    case 1: return launch_gate_cb<1>(a, (int)tiles, stream);
    case 2: return launch_gate_cb<2>(a, (int)tiles, stream);
    case 3: return launch_gate_cb<3>(a, (int)tiles, stream);
    case 4: return launch_gate_cb<4>(a, (int)tiles, stream);
    case 5: return launch_gate_cb<5>(a, (int)tiles, stream);
    case 6: return launch_gate_cb<6>(a, (int)tiles, stream);
    case 7: return launch_gate_cb<7>(a, (int)tiles, stream);
    case 8: return launch_gate_cb<8>(a, (int)tiles, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rib
