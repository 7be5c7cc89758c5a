// Router logits, selection and the per-expert work records (kernels 1 and 2).
#pragma once

#include "moe_common.h"

namespace moe {

// ------------------------------------------------------------------------------------------
// Kernel 1: router logits (+ output seeding)
// ------------------------------------------------------------------------------------------

constexpr int kRouteExpertsPerBlock = kWaves;  // one expert per wave

// Grid: (ceil(E / 4), ceil(T / TC)). Each wave takes one expert and TC rows; every load of the
// wave (its router row and its TC activation rows) is issued before any arithmetic.
template <int NJ, int TC>  // NJ = H / 256: float4 chunks of a row per lane
__global__ __launch_bounds__(kThreads) void logits_kernel(Args a, int layer) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E, H = a.H;
  const Ingress in = get_ingress(a);
  const moe_layer_weights W = get_weights(a, layer);
  const float* __restrict__ x = layer_input(a, in, layer);
  float* __restrict__ xn = layer_output(a, in, layer);

  const int e = min(blockIdx.x * kRouteExpertsPerBlock + wave, E - 1);
  const int t0 = blockIdx.y * TC;
  float4 w[NJ], xv[TC][NJ];
  const float4* wr = reinterpret_cast<const float4*>(W.router_w + static_cast<size_t>(e) * H);
#pragma unroll
  for (int j = 0; j < NJ; ++j) w[j] = load_stream_f4(wr + lane + 64 * j);
#pragma unroll
  for (int r = 0; r < TC; ++r) {
    const float4* xr = reinterpret_cast<const float4*>(x + static_cast<size_t>(min(t0 + r, T - 1)) * H);
#pragma unroll
    for (int j = 0; j < NJ; ++j) xv[r][j] = load_f4(xr + lane + 64 * j);
  }
  const double bias = W.router_bias ? static_cast<double>(W.router_bias[e]) : 0.0;

  // Blocks of row-chunk 0 also seed this layer's output rows with the residual (deep stack) or
  // zeros, and write the layer input as int8 digits per 32-block for the gate/up kernel.
  if (blockIdx.y == 0) {
    const int n4 = T * H / 4;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    float4* xn4 = reinterpret_cast<float4*>(xn);
    for (int i = blockIdx.x * kThreads + tid; i < n4; i += gridDim.x * kThreads)
      xn4[i] = a.residual ? x4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    const int nblk = H / 32;
    for (int i = blockIdx.x * kThreads + tid; i < T * nblk; i += gridDim.x * kThreads)
      quantize_block(x + static_cast<size_t>(i) * 32, a.xq + static_cast<size_t>(i) * kXqWords, a.xss + i);
  }

  double acc[TC];
#pragma unroll
  for (int r = 0; r < TC; ++r) {
    acc[r] = 0.0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      acc[r] = fma(static_cast<double>(w[j].x), static_cast<double>(xv[r][j].x), acc[r]);
      acc[r] = fma(static_cast<double>(w[j].y), static_cast<double>(xv[r][j].y), acc[r]);
      acc[r] = fma(static_cast<double>(w[j].z), static_cast<double>(xv[r][j].z), acc[r]);
      acc[r] = fma(static_cast<double>(w[j].w), static_cast<double>(xv[r][j].w), acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < TC; ++r) acc[r] = wave_sum_f64(acc[r]);
  if (lane == 0 && blockIdx.x * kRouteExpertsPerBlock + wave < E) {
#pragma unroll
    for (int r = 0; r < TC; ++r)
      if (t0 + r < T) a.logits[static_cast<size_t>(t0 + r) * E + e] = acc[r] + bias;
  }
}

// ------------------------------------------------------------------------------------------
// Kernel 2: selection + worklist (one block)
// ------------------------------------------------------------------------------------------

struct SelectShared {
  int sel[MOE_ROUND_MAX_ROWS * MOE_ROUND_MAX_TOPK];     // [t][j] expert id
  float p[MOE_ROUND_MAX_ROWS * MOE_ROUND_MAX_TOPK];     // [t][j] routing weight
  unsigned long long mask[MOE_ROUND_MAX_EXPERTS];      // rows choosing expert e
  int uidx[MOE_ROUND_MAX_EXPERTS];                     // e -> unique index
  int uniq[MOE_ROUND_MAX_EXPERTS];
  int offs[MOE_ROUND_MAX_EXPERTS + 1];
  int pairs[MOE_ROUND_MAX_ROWS * MOE_ROUND_MAX_TOPK];   // by pair slot: t | j << 8
  int wsum[kSelectWaves];
  int nu;
};

// Top-k of one row on one wave. Each lane sorts its NPL (logit, id) keys once; then k rounds of a
// wave-wide unsigned max over the lanes' heads, the winning lane popping its head. Lane j records the
// j-th id and re-reads its exact fp64 logit for the softmax over the k selected logits.
template <int NPL>
__device__ __forceinline__ void select_row(const Args& a, SelectShared& s, int t) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  const double* zrow = a.logits + static_cast<size_t>(t) * E;
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    const double z = zrow[min(e, E - 1)];  // all loads issued together
    key[i] = e < E ? logit_key(z, e) : 0ull;  // 0 is below every real key
  }
#pragma unroll
  for (int pass = 0; pass < NPL; ++pass)
#pragma unroll
    for (int i = pass & 1; i + 1 < NPL; i += 2)
      if (key[i] < key[i + 1]) {
        const uint64_t tmp = key[i];
        key[i] = key[i + 1];
        key[i + 1] = tmp;
      }
  int myid = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t best = wave_max_u64(key[0]);
    const int e = key_expert(best);
    if (lane == (e & 63)) {
#pragma unroll
      for (int i = 0; i + 1 < NPL; ++i) key[i] = key[i + 1];
      key[NPL - 1] = 0ull;
    }
    if (lane == j) myid = e;
  }
  const double zj = zrow[lane < k ? myid : 0];
  const double z0 = __shfl(zj, 0, 64);  // rank 0 holds the largest selected logit
  const double ej = lane < k ? exp(zj - z0) : 0.0;
  const double sum = wave_sum_f64(ej);
  if (lane < k) {
    s.sel[t * k + lane] = myid;
    s.p[t * k + lane] = static_cast<float>(ej / sum);
  }
}

template <int NPL>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(Args a, int layer) {
  __shared__ SelectShared s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E, k = a.k, npairs = T * k;
  const Ingress in = get_ingress(a);

  for (int e = tid; e < E; e += kSelectThreads) s.mask[e] = 0ull;
  for (int t = wave; t < T; t += kSelectWaves) select_row<NPL>(a, s, t);
  __syncthreads();

  for (int idx = tid; idx < npairs; idx += kSelectThreads) atomicOr(&s.mask[s.sel[idx]], 1ull << (idx / k));
  __syncthreads();

  // Block-wide exclusive scan over experts (one per thread, E <= 512 < 1024) of
  // (rows choosing e, whether any row chose e).
  const unsigned long long m = tid < E ? s.mask[tid] : 0ull;
  const int c = __popcll(m), f = c > 0;
  const int packed = c | (f << 16);
  int incl = packed;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s.wsum[wave] = incl;
  __syncthreads();
  int wpre = 0, wtot = 0;
#pragma unroll
  for (int w = 0; w < kSelectWaves; ++w) {
    if (w < wave) wpre += s.wsum[w];
    wtot += s.wsum[w];
  }
  const int excl = incl - packed + wpre;
  const int u = excl >> 16, off0 = excl & 0xFFFF;
  const int nu = wtot >> 16;
  if (f) {
    s.uidx[tid] = u;
    s.uniq[u] = tid;
    s.offs[u] = off0;
  }
  if (tid == 0) {
    s.nu = nu;
    s.offs[nu] = npairs;
  }
  __syncthreads();
  for (int idx = tid; idx < npairs; idx += kSelectThreads) {
    const int t = idx / k, j = idx - t * k;
    const int e = s.sel[idx];
    const int pos = s.offs[s.uidx[e]] + __popcll(s.mask[e] & ((1ull << t) - 1ull));
    s.pairs[pos] = t | (j << 8);
  }
  __syncthreads();

  // Publish: per-expert records, the pair table, the caller's ids / routing weights.
  int32_t* rec = a.rec + static_cast<size_t>(layer) * a.Ucap * kRecWords;
  int32_t* uniq = a.uniq + static_cast<size_t>(layer) * a.Ucap;
  int32_t* offs = a.offs + static_cast<size_t>(layer) * (a.Ucap + 1);
  int32_t* pairs = a.pairs + static_cast<size_t>(layer) * a.Pcap;
  float* pw = a.pair_w + static_cast<size_t>(layer) * a.Pcap;
  for (int i = tid; i < nu * kRecWords; i += kSelectThreads) {
    const int uu = i / kRecWords, wd = i - uu * kRecWords;
    const int p0 = s.offs[uu], np = s.offs[uu + 1] - p0;
    int v = 0;
    if (wd == 0) v = s.uniq[uu];
    else if (wd == 1) v = p0;
    else if (wd == 2) v = np;
    else if (wd == 3) v = nu;
    else if (wd >= kRecRowWord && wd < kRecRowWord + MOE_ROUND_MAX_ROWS / 4) {
      const int r0 = (wd - kRecRowWord) * 4;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (r0 + b < np) v |= (s.pairs[p0 + r0 + b] & 0xFF) << (8 * b);
    }
    rec[i] = v;
  }
  for (int i = tid; i < nu; i += kSelectThreads) uniq[i] = s.uniq[i];
  for (int i = tid; i <= nu; i += kSelectThreads) offs[i] = s.offs[i];
  for (int i = tid; i < npairs; i += kSelectThreads) {
    const int pr = s.pairs[i];
    pairs[i] = pr;
    pw[i] = s.p[(pr & 0xFF) * k + (pr >> 8)];
    const size_t o = static_cast<size_t>(layer) * npairs + i;  // [L][T][k] with i = t*k + j
    if (in.ids) in.ids[o] = s.sel[i];
    if (in.route_w) in.route_w[o] = s.p[i];
  }
  if (tid == 0) a.n_unique[layer] = nu;
}

// Every GEMV block reads its expert's record and record 0 (whose unique count is always valid)
// in one round trip; values are clamped so nothing read back can index out of bounds.
struct ExpertWork {
  int e, p0, np, nu;
  int rows[MOE_ROUND_MAX_ROWS / 4];  // packed row ids, 4 per word
};

__device__ __forceinline__ ExpertWork load_work(const Args& a, int layer, int u) {
  const int32_t* rec = a.rec + static_cast<size_t>(layer) * a.Ucap * kRecWords;
  const int32_t* r = rec + static_cast<size_t>(min(u, a.Ucap - 1)) * kRecWords;
  ExpertWork w;
  const int nu = rec[3];
  w.e = r[0];
  w.p0 = r[1];
  w.np = r[2];
#pragma unroll
  for (int i = 0; i < MOE_ROUND_MAX_ROWS / 4; ++i) w.rows[i] = r[kRecRowWord + i];
  const int npairs = a.T * a.k;
  w.nu = min(max(nu, 0), a.Ucap);
  w.e = min(max(w.e, 0), a.E - 1);
  w.p0 = min(max(w.p0, 0), npairs);
  w.np = min(max(w.np, 0), npairs - w.p0);
  return w;
}

__device__ __forceinline__ int work_row(const ExpertWork& w, int r, int T) {
  // r is wave-uniform; select the packed word without dynamic register indexing
  int word = 0;
#pragma unroll
  for (int i = 0; i < MOE_ROUND_MAX_ROWS / 4; ++i)
    if (i == (r >> 2)) word = w.rows[i];
  return min((word >> (8 * (r & 3))) & 0xFF, T - 1);
}

}  // namespace moe
