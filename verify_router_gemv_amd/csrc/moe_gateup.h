// Kernel 3: gate/up dequant-GEMV with SwiGLU.
#pragma once

#include "moe_gemv.h"

namespace moe {

// Gate/up: integer dot products of the 4-bit codes with the int8 digits of the layer input.
// Codes are unpacked once into bytes (even / odd elements of each 8-group) and kept in registers;
// each row routed to the expert then costs 24 v_dot4 per 32-weight block plus the fp32 fold
// s * step * (65536 A2 + 256 A1 + A0) + m * sum(x).
__device__ __forceinline__ float block_dot_q8(const uint32_t cw[8], const uint32_t xd[kXqWords], float step,
                                              float xsum, uint32_t sm, float acc) {
  int A[3] = {0, 0, 0};
#pragma unroll
  for (int dg = 0; dg < 3; ++dg)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      A[dg] = __builtin_amdgcn_sdot4(static_cast<int>(cw[2 * g]), static_cast<int>(xd[(dg * 4 + g) * 2]), A[dg], false);
      A[dg] = __builtin_amdgcn_sdot4(static_cast<int>(cw[2 * g + 1]), static_cast<int>(xd[(dg * 4 + g) * 2 + 1]),
                                     A[dg], false);
    }
  const float dot = fmaf(static_cast<float>(A[2]), 65536.f, fmaf(static_cast<float>(A[1]), 256.f, static_cast<float>(A[0])));
  const float sc = half_bits_to_float(sm), mn = half_bits_to_float(sm >> 16);
  return fmaf(sc * step, dot, fmaf(mn, xsum, acc));
}

__device__ __forceinline__ void unpack_bytes(const uint4 c, uint32_t cw[8]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cw[2 * i] = w[i] & 0x0F0F0F0Fu;
    cw[2 * i + 1] = (w[i] >> 4) & 0x0F0F0F0Fu;
  }
}

template <int G, int NB, int RW>
__global__ __launch_bounds__(kThreads) void gateup_kernel(Args a, int layer) {
  constexpr int RPI = 64 / G;
  constexpr int ROWS_W = RW * RPI;
  constexpr int ROWS_B = kWaves * ROWS_W;
  const int I = a.I, H = a.H, T = a.T;
  const int nblk = H / 32;
  const int tiles = (I + ROWS_B - 1) / ROWS_B;
  const int u = blockIdx.x / tiles, tile = blockIdx.x - u * tiles;
  const ExpertWork wk = load_work(a, layer, u);
  if (u >= wk.nu) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane % G, rs = lane / G;
  const moe_layer_weights W = get_weights(a, layer);
  const int row0 = tile * ROWS_B + wave * ROWS_W + rs;
  const size_t rq = static_cast<size_t>(H) / 2, rsm = static_cast<size_t>(H) / 32;

  uint4 cg[RW][NB], cu[RW][NB];
  uint32_t sg[RW][NB], su[RW][NB];
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    const size_t r = static_cast<size_t>(wk.e) * I + min(row0 + w * RPI, I - 1);  // rows past I: not stored
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = g + nb * G;
      cg[w][nb] = load_stream_u4(W.gate_q + r * rq + 16 * b);
      cu[w][nb] = load_stream_u4(W.up_q + r * rq + 16 * b);
      sg[w][nb] = load_stream_u32(W.gate_sm + r * rsm + b);
      su[w][nb] = load_stream_u32(W.up_sm + r * rsm + b);
    }
  }

  // Activation digits of one row: NB blocks x 24 words plus (step, block sum).
  uint32_t xd[NB][kXqWords];
  float xstep[NB], xsum[NB];
#define MOE_LOAD_ROW(R)                                                                      \
  {                                                                                          \
    const int t_ = work_row(wk, (R), T);                                                     \
    _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) {                                      \
      const size_t blk = static_cast<size_t>(t_) * nblk + g + nb * G;                        \
      const MOE_GLOBAL u32x4* src = (const MOE_GLOBAL u32x4*)(a.xq + blk * kXqWords);        \
      _Pragma("unroll") for (int q = 0; q < kXqWords / 4; ++q) {                             \
        const u32x4 v = src[q];                                                              \
        xd[nb][4 * q + 0] = v.x;                                                             \
        xd[nb][4 * q + 1] = v.y;                                                             \
        xd[nb][4 * q + 2] = v.z;                                                             \
        xd[nb][4 * q + 3] = v.w;                                                             \
      }                                                                                      \
      const f32x2 ss = *((const MOE_GLOBAL f32x2*)(a.xss + blk));                            \
      xstep[nb] = ss.x;                                                                      \
      xsum[nb] = ss.y;                                                                       \
    }                                                                                        \
  }
  MOE_LOAD_ROW(0)

  uint32_t wg[RW][NB][8], wu[RW][NB][8];
#pragma unroll
  for (int w = 0; w < RW; ++w)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      unpack_bytes(cg[w][nb], wg[w][nb]);
      unpack_bytes(cu[w][nb], wu[w][nb]);
    }

  for (int r = 0; r < wk.np; ++r) {
    float acc[2 * RW];
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      float ag = 0.f, au = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        ag = block_dot_q8(wg[w][nb], xd[nb], xstep[nb], xsum[nb], sg[w][nb], ag);
        au = block_dot_q8(wu[w][nb], xd[nb], xstep[nb], xsum[nb], su[w][nb], au);
      }
      acc[w] = ag;       // gate partials: acc[0 .. RW-1]
      acc[RW + w] = au;  // up partials:   acc[RW .. 2RW-1]
    }
    if (r + 1 < wk.np) MOE_LOAD_ROW(r + 1)  // uniform branch: the next row's digits, after this row's use
    float* hrow = a.hbuf + static_cast<size_t>(wk.p0 + r) * I;
    if constexpr (G == 64 && RW == 4) {
      float gsum, usum;
      reduce8_wave(acc, gsum, usum);
      const int R = lane >> 4;
      const int i = row0 + reduce8_slot(R);  // RPI == 1: row group w is row row0 + w
      if ((lane & 15) == 0 && i < I) hrow[i] = silu(gsum) * usum;
    } else {
#pragma unroll
      for (int w = 0; w < 2 * RW; ++w) acc[w] = group_sum<G>(acc[w]);
      if (g == 0) {
#pragma unroll
        for (int w = 0; w < RW; ++w) {
          const int i = row0 + w * RPI;
          if (i < I) hrow[i] = silu(acc[w]) * acc[RW + w];
        }
      }
    }
  }
#undef MOE_LOAD_ROW
}

}  // namespace moe
