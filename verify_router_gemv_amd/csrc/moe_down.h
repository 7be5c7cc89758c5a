// Kernel 4: down dequant-GEMV with the routing-weighted scatter-add.
#pragma once

#include "moe_gemv.h"

namespace moe {


template <int G, int NB, int RC, int RW>
__global__ __launch_bounds__(kThreads) void down_kernel(Args a, int layer) {
  constexpr int RPI = 64 / G;
  constexpr int ROWS_W = RW * RPI;
  constexpr int ROWS_B = kWaves * ROWS_W;
  extern __shared__ float hlds[];  // [xstage_i][I] when T > 1
  const int I = a.I, H = a.H, T = a.T;
  const int tiles = (H + ROWS_B - 1) / ROWS_B;
  const int u = blockIdx.x / tiles, tile = blockIdx.x - u * tiles;
  const ExpertWork wk = load_work(a, layer, u);
  if (u >= wk.nu) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane % G, rs = lane / G;
  const float* pw = a.pair_w + static_cast<size_t>(layer) * a.Pcap;
  const Ingress in = get_ingress(a);
  const moe_layer_weights W = get_weights(a, layer);
  float* __restrict__ xn = layer_output(a, in, layer);
  const int row0 = tile * ROWS_B + wave * ROWS_W + rs;
  const size_t rq = static_cast<size_t>(I) / 2, rsm = static_cast<size_t>(I) / 32;

  uint4 cd[RW][NB];
  uint32_t sd[RW][NB];
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    const size_t r = static_cast<size_t>(wk.e) * H + min(row0 + w * RPI, H - 1);  // rows past H: not stored
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = g + nb * G;
      cd[w][nb] = load_stream_u4(W.down_q + r * rq + 16 * b);
      sd[w][nb] = load_stream_u32(W.down_sm + r * rsm + b);
    }
  }

  const int xst = T > 1 ? a.xstage_i : MOE_ROUND_MAX_ROWS;
  for (int s0 = 0; s0 < wk.np; s0 += xst) {
    const int ns = min(xst, wk.np - s0);
    const float* src = a.hbuf + static_cast<size_t>(wk.p0 + s0) * I;
    if (T > 1) {
      __syncthreads();
      stage_rows(hlds, src, I, ns, [&](int r) { return r; });
      __syncthreads();
      src = hlds;
    }
    for (int c = 0; c < ns; c += RC) {
      int row_of[RC];
#pragma unroll
      for (int r = 0; r < RC; ++r) row_of[r] = min(c + r, ns - 1);
      float wpass[RC];
#pragma unroll
      for (int r = 0; r < RC; ++r) wpass[r] = pw[wk.p0 + s0 + min(c + r, ns - 1)];
      float xv[RC][NB][32], xs[RC][NB];
      if (T > 1) load_x<NB, RC, G, true>(src, I, row_of, ns - c, g, xv, xs);
      else load_x<NB, RC, G, false>(src, I, row_of, ns - c, g, xv, xs);
#pragma unroll
      for (int w = 0; w < RW; ++w)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) opaque(cd[w][nb]);
      float acc[RW][RC];
#pragma unroll
      for (int w = 0; w < RW; ++w) block_dots<NB, RC>(cd[w], sd[w], xv, xs, acc[w]);
#pragma unroll
      for (int w = 0; w < RW; ++w)
#pragma unroll
        for (int r = 0; r < RC; ++r) acc[w][r] = group_sum<G>(acc[w][r]);
      if (g == 0) {
#pragma unroll
        for (int r = 0; r < RC; ++r) {
          if (c + r >= ns) continue;
          const int slot = s0 + c + r;
          const int t = work_row(wk, slot, T);
          const float wgt = wpass[r];
#pragma unroll
          for (int w = 0; w < RW; ++w) {
            const int hr = row0 + w * RPI;
            if (hr < H) atomicAdd(xn + static_cast<size_t>(t) * H + hr, wgt * acc[w][r]);
          }
        }
      }
    }
  }
}

}  // namespace moe
