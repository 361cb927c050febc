// Convolutional local attention (CLA) gate for gfx950: G = sigmoid(PW_1x1(DW_3x3(X))) on a
// [B, H, W, C] map, the gating map that modulates the attention output (O' = O * G) in the
// pages' description of CLA (gist.science/paper/2603.06738, "Technical Summary" §2.B: depth-wise
// conv, point-wise conv and sigmoid; the German summary §2.B: O' = O (.) G; the Chinese summary
// §2.B: 3x3 depth-wise and 1x1 point-wise).
//
// bf16 kernel: a workgroup walks down a strip of row segments of 32 SEG pixels (one x segment,
// `rows` consecutive rows of one image) with SEG x CB waves (CB = C / 32; SEG = 2 where the LDS
// holds it, C <= 192, which gives one workgroup of 12 waves per CU at C = 192):
//  * Halo rows (32 SEG + 2 pixels x C channels, one contiguous run of the map) reach a ring of four
//    LDS rows by DMA (buffer_load ... lds), each row once per strip: rows y - 1, y, y + 1
//    serve output row y while row y + 2 is on its way. Pixels and rows outside the map
//    read as zeros through the buffer range check (the conv's zero padding).
//  * Depth-wise 3x3 on the vector unit in fp32: a thread owns two adjacent channels (taps and
//    bias in registers for the whole launch) and 8 consecutive pixels; a 3 x 3 window of halo
//    values slides along them. D (bf16) goes to LDS as [pixel][C], two rows' worth: the
//    depth-wise conv of row y + 1 runs between the same barriers as the point-wise conv of
//    row y (one barrier per row), so vector and matrix work overlap within each wave.
//  * Point-wise 1x1 on the matrix unit: G^T[out][px] = W_pw[out][:] . D[px][:] as
//    v_mfma_f32_16x16x32_bf16; wave v owns outputs 32 (v % CB) .. + 31 (two 16-row A blocks of
//    W_pw, bf16, in registers for the whole launch) for the 32 pixels 32 (v / CB) .. + 31 (two
//    16-column B blocks read from D), so D is read C / 32 times per row segment.
//  * Sigmoid in fp32 on the accumulator, rounded once to bf16. A lane's accumulators hold two
//    4-channel pieces of one pixel 16 channels apart; two lane swaps (v_permlane32_swap, then
//    v_permlane16_swap) regroup them into 8 consecutive channels per lane, stored as 16 bytes
//    straight to the map at the start of the next row's step (so the store's latency hides
//    behind that step) through a range-checked buffer store that drops pixels past the map's
//    edge: two store instructions per wave and row, each writing 16 whole 64-byte runs (four
//    8-byte stores of 32-byte runs cost a fifth of the step).
//  * The point-wise weights reach LDS once per workgroup by coalesced DMA (one float32 row per
//    instruction) before the first depth-wise conv, in the D buffers and the last ring slot, and
//    each wave reads its A fragments there: loading them per lane straight from global memory
//    (16 rows of 16-byte pieces per instruction, every row twice per workgroup) took a quarter
//    of the kernel's time on a 192-channel map.
#include <algorithm>

#include "internal.hpp"

namespace rib {
namespace {

constexpr int kGatePx = 32;   // pixels per wave's share of a row segment (two MFMA column blocks)

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS operations, not for its
// global traffic (the stores and the next halo row's DMA stay in flight across it). The memory
// clobber keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroup barrier after all of this wave's memory operations (halo DMA included) completed.
__device__ __forceinline__ void full_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroup barrier after all but this wave's last two memory operations completed: the row
// stores that follow the halo DMA the barrier waits for (memory operations complete in order).
__device__ __forceinline__ void barrier_after_dma_of_prev_step() {
  asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float sigmoid_fast(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float sigmoid_exact(float z) { return 1.0f / (1.0f + expf(-z)); }

__device__ __forceinline__ float bf_lo(unsigned u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf_hi(unsigned u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

template <int CB, int SEG>  // C = 32 CB channels; segments of 32 SEG pixels; SEG x CB waves
__global__ __launch_bounds__(64 * CB * SEG) void cla_gate_bf16_kernel(GateArgs a, int rows) {
  constexpr int C = 32 * CB;
  constexpr int NW = CB * SEG;                    // waves
  constexpr int NT = 64 * NW;
  constexpr int SPX = kGatePx * SEG;              // pixels per row segment
  constexpr int KS = CB;                          // MFMA K-steps (32 channels) of the point-wise conv
  constexpr int HP = SPX + 2;                     // halo row width in pixels
  constexpr int CPX = C / 8;                      // 16-byte chunks per pixel
  constexpr int kRowChunks = HP * CPX;
  constexpr int kRowInsts = (kRowChunks + 63) / 64;   // DMA instructions per halo row
  constexpr int kWaveInsts = (kRowInsts + NW - 1) / NW;
  constexpr int kRing = 4;
  constexpr int DROW = C + 8;                     // padded LDS row (bf16) of D
  constexpr int kPxPerThread = 8;                 // SPX pixels over the 4 SEG thread groups of a channel pair
  static_assert(NT == 4 * SEG * (C / 2), "two channels x 8 pixels per thread");
  __shared__ u32x4 sRing[kRing][kRowInsts * 64];
  __shared__ __align__(16) bf16 sD[2][SPX * DROW];   // two rows' D (double buffer)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l16 = lane & 15, quad = lane >> 4;
  const int og = wave % CB, sg = wave / CB;       // output group (32 channels) and 32-pixel half

  // strip: image b, x segment xt, rows [y0, y1)
  const int H = a.H, W = a.W;
  const int ntx = (W + SPX - 1) / SPX;
  const int nys = (H + rows - 1) / rows;
  const int col = blockIdx.x / nys, ys = blockIdx.x - col * nys;
  const int b = col / ntx, xt = col - b * ntx;
  const int x0 = xt * SPX, y0 = ys * rows, y1 = min(H, y0 + rows);
  const bf16* x = (const bf16*)a.x;
  bf16* gout = (bf16*)a.g;

  // halo row DMA: this wave's instructions i = wave + NW j; lane chunk c = 64 i + lane is halo
  // pixel hp = c / CPX (map pixel x0 - 1 + hp) and channel chunk c % CPX. The row's buffer
  // starts at map pixel bx = max(x0 - 1, 0) and ends at pixel min(W, x0 + SPX + 1): at x0 = 0 the
  // left halo pixel's offset is negative and, like pixels past W, fails the unsigned range check
  // (zeros).
  const int bx = x0 > 0 ? x0 - 1 : 0;
  unsigned doff[kWaveInsts];
#pragma unroll
  for (int j = 0; j < kWaveInsts; ++j) {
    const int c = 64 * (wave + NW * j) + lane;
    const int hp = c / CPX, k = c - hp * CPX;
    doff[j] = c < kRowChunks ? (unsigned)((x0 - 1 + hp - bx) * C * 2 + 16 * k) : 0x80000000u;
  }
  const int seg_bytes = (min(W, x0 + SPX + 1) - bx) * C * 2;
  auto dma_row = [&](int y) {
    const bool in = y >= 0 && y < H;
    const bf16* base = x + (((int64_t)b * H + (in ? y : 0)) * W + bx) * C;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), 0, in ? seg_bytes : 0, 0x00020000);
    u32x4* slot = sRing[(y - y0 + 1) & (kRing - 1)];
#pragma unroll
    for (int j = 0; j < kWaveInsts; ++j) {
      const int i = wave + NW * j;
      if (i < kRowInsts)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(slot + 64 * i), 16,
                                                 (int)doff[j], 0, 0, 0);
    }
  };

  // point-wise weights of this wave's 32 output rows as 16x16x32 A fragments: lane l holds row
  // 32 og + 16 ob + l % 16, channels 32 s + 8 (l / 16) + j; the bias of the lane's
  // accumulator rows 32 og + 16 ob + 4 (l / 16) + i
  bf16x8 wa[2][KS];   // filled in the prologue, from LDS
  f32x4 bias[2];
#pragma unroll
  for (int ob = 0; ob < 2; ++ob)
#pragma unroll
    for (int i = 0; i < 4; ++i) bias[ob][i] = a.b_pw ? a.b_pw[32 * og + 16 * ob + 4 * quad + i] : 0.f;
  // depth-wise taps and biases of the thread's channel pair
  const int cp = tid % (C / 2), pg = tid / (C / 2);
  float tap[2][9], bdw[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#pragma unroll
    for (int k = 0; k < 9; ++k) tap[e][k] = a.w_dw[(2 * cp + e) * 9 + k];
    bdw[e] = a.b_dw ? a.b_dw[2 * cp + e] : 0.f;
  }

  // depth-wise 3x3 (fp32) of output row y for the thread's 8 pixels into D buffer db; rows
  // y - 1 .. y + 1 sit in ring slots (y - y0) .. (y - y0 + 2) mod 4; a 3 x 3 window of halo
  // values slides along the pixels
  auto depthwise = [&](int y, int db) {
    const unsigned* rr[3];
#pragma unroll
    for (int ky = 0; ky < 3; ++ky) rr[ky] = (const unsigned*)sRing[(y + ky - y0) & (kRing - 1)] + cp;
    const int h0 = kPxPerThread * pg;   // halo pixel of the window's left column
    bf16* dst = sD[db] + h0 * DROW + 2 * cp;
    float xw[3][3][2];
#pragma unroll
    for (int ky = 0; ky < 3; ++ky)
#pragma unroll
      for (int kx = 0; kx < 2; ++kx) {
        const unsigned u = rr[ky][(h0 + kx) * (C / 2)];
        xw[ky][kx + 1][0] = bf_lo(u);
        xw[ky][kx + 1][1] = bf_hi(u);
      }
#pragma unroll
    for (int i = 0; i < kPxPerThread; ++i) {
#pragma unroll
      for (int ky = 0; ky < 3; ++ky) {
        const unsigned u = rr[ky][(h0 + i + 2) * (C / 2)];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          xw[ky][0][e] = xw[ky][1][e];
          xw[ky][1][e] = xw[ky][2][e];
        }
        xw[ky][2][0] = bf_lo(u);
        xw[ky][2][1] = bf_hi(u);
      }
      float d[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        d[e] = bdw[e];
#pragma unroll
        for (int ky = 0; ky < 3; ++ky)
#pragma unroll
          for (int kx = 0; kx < 3; ++kx) d[e] = fmaf(tap[e][3 * ky + kx], xw[ky][kx][e], d[e]);
      }
      bf16x2 dv;
      dv[0] = f32_to_bf16(d[0]);
      dv[1] = f32_to_bf16(d[1]);
      *(bf16x2*)(dst + i * DROW) = dv;
    }
  };

  // G of the previous row: per pixel block pb, 8 consecutive output channels 32 og + 8 (l / 16)
  // .. + 7 of pixel l % 16 per lane, stored at the start of the next step through a
  // range-checked buffer (pixels past W fall outside the row's range and are dropped), so every
  // wave issues exactly two stores per row (the barrier below counts on it), each writing whole
  // 64-byte runs of 16 pixels
  u32x4 gres[2];
  const int seg_px = min(W, x0 + SPX) - x0;
  auto store_row = [&](int y) {
    bf16* grow = gout + (((int64_t)b * H + y) * W + x0) * C;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(grow, 0, seg_px * C * 2, 0x00020000);
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const int px = 32 * sg + 16 * pb + l16;
      __builtin_amdgcn_raw_buffer_store_b128(gres[pb], rs, (px * C + 32 * og + 8 * quad) * 2, 0, 0);
    }
  };

  // Step y: the point-wise conv of row y (D buffer (y - y0) mod 2, formed in the previous step)
  // and the depth-wise conv of row y + 1 into the other buffer run between the same two barriers,
  // so each wave has matrix and vector work in flight together; row y + 3's DMA goes into the ring
  // slot of row y - 1 and row y - 1's gate is stored.
  // Prologue. The first depth-wise conv needs halo rows y0 - 1 .. y0 + 1 (ring slots 0 - 2); row
  // y0 + 2 (slot 3) is first read in step y0, and the D buffers are first written by the first
  // depth-wise conv. Until then the D buffers and ring slot 3 stage the point-wise weights: rounds
  // of kRoundRows float32 rows (whole 32-row output groups), one coalesced DMA instruction per
  // row, rows kWPitch bytes apart (16 bytes of padding spread the 16 rows of a fragment read over
  // the LDS banks), first in the D buffers, then in slot 3. The first round's weights go out
  // before the three halo rows and are waited for alone; the waves owning a round's rows read
  // their A fragments and round them to bf16. Row y0 + 2 goes out once the weights are read.
  {
    constexpr int kWPitch = 4 * C + 16;
    constexpr int kRowsA = (int)sizeof(sD) / kWPitch;
    constexpr int kRowsB = (int)sizeof(sRing[3]) / kWPitch;
    constexpr int kRoundRows = std::min(C, 32 * ((kRowsA + kRowsB) / 32));
    static_assert(kRoundRows >= 32, "a round holds at least one 32-row output group");
    // halo DMA instructions each wave issues after the first round's weights (three rows)
    constexpr int kMinHalo = std::min(63, 3 * (kRowInsts / NW));
    char* stage_a = (char*)sD;
    char* stage_b = (char*)sRing[3];
    auto stage_row = [&](int i) { return i < kRowsA ? stage_a + i * kWPitch : stage_b + (i - kRowsA) * kWPitch; };
    const __amdgpu_buffer_rsrc_t wrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.w_pw), 0, C * C * 4, 0x00020000);
#pragma unroll
    for (int r0 = 0; r0 < C; r0 += kRoundRows) {
      const int nr = std::min(kRoundRows, C - r0);
      for (int i = wave; i < nr; i += NW)
        if (lane < C / 4)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (__attribute__((address_space(3))) void*)stage_row(i), 16,
                                                   ((r0 + i) * C + 4 * lane) * 4, 0, 0, 0);
      if (r0 == 0) {
        // the halo rows follow the round's weights in issue order (the wait below counts on it)
        asm volatile("" ::: "memory");
        dma_row(y0 - 1);
        dma_row(y0);
        dma_row(y0 + 1);
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kMinHalo) : "memory");
      } else {
        full_barrier();
      }
      if (32 * og >= r0 && 32 * og < r0 + nr) {
#pragma unroll
        for (int ob = 0; ob < 2; ++ob) {
          const float* wrow = (const float*)stage_row(32 * og - r0 + 16 * ob + l16);
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const f32x4 w0 = *(const f32x4*)(wrow + 32 * s + 8 * quad);
            const f32x4 w1 = *(const f32x4*)(wrow + 32 * s + 8 * quad + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              wa[ob][s][j] = f32_to_bf16(w0[j]);
              wa[ob][s][4 + j] = f32_to_bf16(w1[j]);
            }
          }
        }
      }
      lds_barrier();
    }
  }
  // rows y0 - 1 .. y0 + 1 landed in every wave's part; row y0 + 2's DMA (at least kRowInsts / NW
  // instructions of each wave) may stay in flight until step y0
  if (y0 + 2 <= y1) {
    dma_row(y0 + 2);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(std::min(63, kRowInsts / NW)) : "memory");
  } else {
    full_barrier();
  }
  depthwise(y0, 0);
  for (int y = y0; y < y1; ++y) {
    // row y + 2 landed, D of row y complete, every wave past the previous step (ring slot of row
    // y - 1 and the other D buffer free). Row y + 2's DMA went out in step y - 1 before that
    // step's two stores, which from step y0 + 2 on may stay in flight.
    if (y >= y0 + 2) barrier_after_dma_of_prev_step();
    else full_barrier();
    if (y + 3 <= y1) dma_row(y + 3);
    // the stores must follow the DMA in issue order: the next step's barrier waits for all but
    // this wave's last two memory operations
    asm volatile("" ::: "memory");
    if (y > y0) store_row(y - 1);
    const int db = (y - y0) & 1;
    // ---- point-wise 1x1: block (ob, pb) = outputs 32 og + 16 ob + [0, 16) x pixels 32 sg + 16 pb +
    // [0, 16); lane l holds outputs 4 (l / 16) + i of the block for pixel l % 16
    f32x4 acc[2][2];
#pragma unroll
    for (int ob = 0; ob < 2; ++ob) acc[ob][0] = acc[ob][1] = bias[ob];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 bf[2];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
        bf[pb] = *(const bf16x8*)&sD[db][(32 * sg + 16 * pb + l16) * DROW + 32 * s + 8 * quad];
#pragma unroll
      for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int pb = 0; pb < 2; ++pb)
          acc[ob][pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ob][s], bf[pb], acc[ob][pb], 0, 0, 0);
    }
    if (y + 1 < y1) depthwise(y + 1, db ^ 1);
    // Lane l holds outputs 16 ob + 4 (l / 16) + 0..3 of pixel l % 16 (dwords lo, hi per ob).
    // Counting 16-lane rows, swapping rows 2, 3 of the ob = 0 dword with rows 0, 1 of the
    // ob = 1 dword (v_permlane32_swap), then the odd rows of the first result with the even rows
    // of the second (v_permlane16_swap), leaves row q with outputs 4 (2q) .. 4 (2q) + 3 in the
    // first result and 4 (2q + 1) .. + 3 in the second: 8 consecutive outputs per lane.
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      unsigned w[2][2];   // [ob][lo, hi]
#pragma unroll
      for (int ob = 0; ob < 2; ++ob) {
        bf16 o4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = f32_to_bf16(sigmoid_fast(acc[ob][pb][i]));
        const uint2 u = *(const uint2*)o4;
        w[ob][0] = u.x;
        w[ob][1] = u.y;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto r32 = __builtin_amdgcn_permlane32_swap(w[0][h], w[1][h], false, false);
        const auto r16 = __builtin_amdgcn_permlane16_swap(r32[0], r32[1], false, false);
        gres[pb][h] = r16[0];        // outputs 8 q + 2 h, + 1
        gres[pb][2 + h] = r16[1];    // outputs 8 q + 4 + 2 h, + 1
      }
    }
  }
  if (y1 > y0) store_row(y1 - 1);
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

// One round of one workgroup per CU: at C = 192 the ring and D buffers take 154 KB of the CU's
// 160 KB of LDS (SEG = 2), and at C = 224 and 256 (SEG = 1) more than half of it, so a second
// workgroup would not be resident at the same time.
template <int CB>
hipError_t launch_gate_cb(const GateArgs& a, hipStream_t stream) {
  constexpr int SEG = CB <= 6 ? 2 : 1;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // strips of `rows` rows: the fewest rows per strip whose strips all fit one round of resident
  // workgroups (each strip re-reads two halo rows, so longer strips waste less)
  const int64_t slots = std::max(cus, 1);
  const int64_t cols = (int64_t)a.B * ((a.W + kGatePx * SEG - 1) / (kGatePx * SEG));
  int rows = (int)std::max<int64_t>(1, (cols * a.H + slots - 1) / slots);
  while (rows < a.H && cols * ((a.H + rows - 1) / rows) > slots) ++rows;
  const int64_t grid = cols * ((a.H + rows - 1) / rows);
  hipLaunchKernelGGL((cla_gate_bf16_kernel<CB, SEG>), dim3((unsigned)grid), dim3(64 * CB * SEG), 0, stream, a, rows);
  return hipGetLastError();
}

}  // namespace

// One wave per 32 output channels, up to 8 (C = 256): the point-wise weights stay resident in
// registers (8 VGPRs per 32 input channels).
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
    case 1: return launch_gate_cb<1>(a, stream);
    case 2: return launch_gate_cb<2>(a, stream);
    case 3: return launch_gate_cb<3>(a, stream);
    case 4: return launch_gate_cb<4>(a, stream);
    case 5: return launch_gate_cb<5>(a, stream);
    case 6: return launch_gate_cb<6>(a, stream);
    case 7: return launch_gate_cb<7>(a, stream);
    case 8: return launch_gate_cb<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rib
