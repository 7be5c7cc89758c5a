// Kernel 4: down dequant-GEMV with the routing-weighted scatter-add.
#pragma once

#include "moe_gemv.h"

namespace moe {


// EXACT: store W_d h of each pair in its slot of ybuf (the combine kernel adds them in rank order)
// instead of adding the weighted product into the output with an atomic.
template <int G, int NB, int RC, int RW, bool EXACT, int FMT>
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
  const size_t rq = static_cast<size_t>(I) / 2, rsm = sm_row_words<FMT>(I);

  uint4 cd[RW][NB];
  BlockScale<FMT> sd[RW][NB];
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    const size_t r = static_cast<size_t>(wk.e) * H + min(row0 + w * RPI, H - 1);  // rows past H: not stored
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = g + nb * G;
      cd[w][nb] = load_stream_u4(W.down_q + r * rq + 16 * b);
      sd[w][nb].load(W.down_sm + r * rsm, b);
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
          if constexpr (EXACT) {
            float* y = a.ybuf + static_cast<size_t>(wk.p0 + slot) * H;
#pragma unroll
            for (int w = 0; w < RW; ++w) {
              const int hr = row0 + w * RPI;
              if (hr < H) y[hr] = acc[w][r];
            }
          } else {
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
}

// Exact mode: out[t][h] = (residual ? x[t][h] : 0) + sum over ranks j = 0..k-1, in that order, of
// p[t][j] * y[slot(t, j)][h]. Grid (T, ceil(H / 1024)) x 256 threads, four columns per thread.
static __global__ __launch_bounds__(kThreads) void combine_kernel(Args a, int layer) {
  const Ingress in = get_ingress(a);
  const float* __restrict__ x = layer_input(a, in, layer);
  float* __restrict__ xn = layer_output(a, in, layer);
  const int t = blockIdx.x, H = a.H, k = a.k;
  const int h = (blockIdx.y * kThreads + threadIdx.x) * 4;
  if (h >= H) return;
  const int32_t* slot_of = a.slot_of + static_cast<size_t>(layer) * a.Pcap + t * k;
  const float* pw = a.pair_w + static_cast<size_t>(layer) * a.Pcap;
  float4 acc = a.residual ? load_f4(x + static_cast<size_t>(t) * H + h) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int s = min(max(slot_of[j], 0), a.Pcap - 1);
    const float w = pw[s];
    const float4 y = load_f4(a.ybuf + static_cast<size_t>(s) * H + h);
    acc.x = fmaf(w, y.x, acc.x);
    acc.y = fmaf(w, y.y, acc.y);
    acc.z = fmaf(w, y.z, acc.z);
    acc.w = fmaf(w, y.w, acc.w);
  }
  *reinterpret_cast<float4*>(xn + static_cast<size_t>(t) * H + h) = acc;
}

}  // namespace moe
