// Prefill MoE: rounds of more than 64 rows, where the expert FFN is compute-bound.
//
// Per layer nine kernels, launched eagerly:
//   quant_rows_kernel   the layer input as 22-bit integers per row (three int8 digit planes) and
//                       per-32-block sums, for the int8 matrix cores
//   pf_logits_kernel    router GEMM on fp64 matrix cores (fp32 inputs, fp64 products and sums)
//   pf_topk_kernel      one wave per row: top-k, softmax over the selected, and the row's bit in
//                       each chosen expert's row mask
//   pf_scan_kernel      one block: rows per expert, their offsets, the unique list and the
//                       64-pair work items
//   pf_scatter_kernel   counting sort of the (row, rank) pairs by expert (ascending expert, rows
//                       ascending within one); the caller's ids and routing weights
//   pf_gateup_kernel    per work item and 64 rows of I: silu(W_g x) * (W_u x) as an int8 GEMM
//   quant_rows_kernel   the SwiGLU rows as digits
//   pf_down_kernel      per work item and 128 rows of H: W_d h per pair, into a slot buffer
//   pf_combine_kernel   each row adds its k products in rank order (and the residual)
//
// The infero README, "Beyond plain text decode", routes prefill through a counting sort followed
// by a GEMM per expert; its "Design notes" run batched projections straight off the quantised
// weights on integer matrix instructions, one instruction per 32-weight block, with the block
// scales applied in float afterwards. Here the activations are 22-bit integers split into three
// int8 planes, so the int32 block products are exact and the fp32 fold keeps the round within the
// fp32-accumulation tolerance of the decode path; the block minimum's term sum_b m * sum(x) runs
// on fp32 matrix instructions.
#pragma once

#include "moe_common.h"
#include "moe_gemv.h"
#include "moe_route.h"

namespace moe {
namespace pf {

constexpr int kTile = 64;                 // GEMM tile: 64 (row, rank) pairs by 64 or 128 weight rows
constexpr int kGemmThreads = 512;         // GEMM blocks: 8 waves, each 32 weight rows x 32 pairs of one matrix
constexpr int kGemmWaves = kGemmThreads / 64;
constexpr float kQMax = 4194303.0f;       // 2^22 - 1: 32 * 15 * kQMax < 2^31 (int32 block dots)
constexpr int kStepBlocks = 4;            // 32-blocks of the reduction per pipeline step
// LDS per GEMM block: two buffers of [block][plane][half][pair][4] digit words.
constexpr int kStageWords = kStepBlocks * 3 * 2 * kTile * 4;
constexpr int kGemmLds = 2 * kStageWords * 4;

struct PfArgs {
  Ingress in;
  moe_layer_weights w;
  float* xbuf0;          // [Tp][H] layer outputs between layers (L > 1)
  float* xbuf1;
  double* logits;        // [Tp][E]
  uint32_t* xq;          // [Tp][H/32][kXqWords] digits of the layer input
  float* xstep;          // [Tp] its per-row step
  float* xsum;           // [Tp][H/32] block sums divided by the step
  unsigned long long* mask;  // [E][W] rows choosing expert e, 64 per word
  int32_t* wpre;         // [E][W] rows of expert e in the words before
  int32_t* sel;          // [Tp][k] expert ids
  float* selp;           // [Tp][k] routing weights
  int32_t* n_unique;     // [L]
  int32_t* uniq;         // [L][E]
  int32_t* offs;         // [L][E + 1]
  int32_t* eoff;         // [E] first pair slot of expert e
  int32_t* pairs;        // [L][Pcap] t | j << 16, grouped by expert
  float* pair_w;         // [Pcap]
  int32_t* slot_of;      // [Pcap] pair slot of (t, j) at t * k + j
  int4* items;           // [Icap] (expert, first pair slot, pairs, 0)
  int32_t* n_items;      // [1]
  float* hbuf;           // [Pcap][I] SwiGLU rows by pair slot
  uint32_t* hq;          // [Pcap][I/32][kXqWords]
  float* hstep;          // [Pcap]
  float* hsum;           // [Pcap][I/32]
  float* ybuf;           // [Pcap][H] W_d h by pair slot
  int32_t H, I, E, L, T, k, residual, Pcap, Icap, W;
};

__device__ __forceinline__ const float* pf_layer_input(const PfArgs& a, int layer) {
  if (layer == 0) return a.in.hidden;
  return ((layer - 1) & 1) ? a.xbuf1 : a.xbuf0;
}
__device__ __forceinline__ float* pf_layer_output(const PfArgs& a, int layer) {
  if (layer == a.L - 1) return a.in.out;
  return (layer & 1) ? a.xbuf1 : a.xbuf0;
}

// ------------------------------------------------------------------------------------------
// Rows as digits: one wave per row of K floats. q = rint(x / step) with step = max|x| / kQMax over
// the row, split into balanced base-256 digits d0, d1 in [-128, 127] and d2 (|d2| <= 64), stored
// per 32-block in the gate/up digit layout (words [plane][group of 8][even/odd], the even word
// holding elements 8g+0,2,4,6, the odd one 8g+1,3,5,7: the order of the weight nibbles). The
// block sums (of x, in fp32) are stored divided by the step. Grid: ceil(n / 4) x 256 threads.
// zero_words / zero: words of `zero` cleared by the grid on the side (the layer's row masks).
// ------------------------------------------------------------------------------------------
static __global__ __launch_bounds__(kThreads) void quant_rows_kernel(const float* __restrict__ src, int K, int n,
                                                                   uint32_t* dig, float* step_out, float* bsum,
                                                                   unsigned long long* zero, int zero_words) {
  const int lane = threadIdx.x & 63;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < zero_words; i += gridDim.x * kThreads) zero[i] = 0ull;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= n) return;  // whole waves leave together
  const float* x = src + static_cast<size_t>(row) * K;
  const int n4 = K / 4;  // float4 chunks; chunk c = lane + 64 j is elements 4c..4c+3 of block c / 8
  uint32_t mx = 0;
  for (int c = lane; c < n4; c += 64) {
    const float4 v = load_f4(x + 4 * c);
    const float m4 = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    mx = max(mx, __builtin_bit_cast(uint32_t, m4));  // non-negative floats order as integers
  }
  const float rmax = __builtin_bit_cast(float, wave_max_u32(mx));
  const float step = rmax / kQMax;
  const float inv = rmax > 0.f ? kQMax / rmax : 0.f;
  const float sinv = rmax > 0.f ? 1.f / step : 0.f;
  if (lane == 0) step_out[row] = step;
  uint32_t* drow = dig + static_cast<size_t>(row) * (K / 32) * kXqWords;
  for (int c0 = 0; c0 < n4; c0 += 64) {  // K / 4 is a multiple of 8: a block's 8 lanes are all in or out
    const int c = c0 + lane;
    const bool in = c < n4;
    const float4 v = load_f4(x + 4 * min(c, n4 - 1));
    float sum = (v.x + v.y) + (v.z + v.w);
    sum += dpp_f32<kDppXor1>(sum);
    sum += dpp_f32<kDppXor2>(sum);
    sum += dpp_f32<kDppHalfMirror>(sum);  // the 8 lanes of this block
    const float e[4] = {v.x, v.y, v.z, v.w};
    int d[3][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = static_cast<int>(rintf(e[i] * inv));
      q = max(-static_cast<int>(kQMax), min(static_cast<int>(kQMax), q));
      const int d0 = ((q + 128) & 255) - 128;
      const int q1 = (q - d0) >> 8;
      const int d1 = ((q1 + 128) & 255) - 128;
      d[0][i] = d0;
      d[1][i] = d1;
      d[2][i] = (q1 - d1) >> 8;
    }
    if (in) {
      const int b = c >> 3, sub = c & 7;
      // elements 4*sub + i: group sub / 2, even word for i = 0, 2 and odd for i = 1, 3, bytes
      // 2*(sub % 2) + i / 2 of the word
      uint16_t* base = reinterpret_cast<uint16_t*>(drow + static_cast<size_t>(b) * kXqWords);
      const int g = sub >> 1, half = sub & 1;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        base[((p * 4 + g) * 2 + 0) * 2 + half] = static_cast<uint16_t>((d[p][0] & 0xFF) | ((d[p][2] & 0xFF) << 8));
        base[((p * 4 + g) * 2 + 1) * 2 + half] = static_cast<uint16_t>((d[p][1] & 0xFF) | ((d[p][3] & 0xFF) << 8));
      }
      if (sub == 0) bsum[static_cast<size_t>(row) * (K / 32) + b] = sum * sinv;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Router logits on fp64 matrix cores: z[t][e] = sum_h Wr[e][h] x[t][h] + b[e]. Every fp32 x fp32
// product is exact in fp64 and the sums are fp64, as in the decode path. v_mfma_f64_16x16x4f64:
// A = 16 experts x 4 terms, B = 4 terms x 16 rows; lane l supplies A row / B column l % 16 and term
// l / 16, and D register i of lane l holds row l/16 + 4i (an expert) of column l % 16 (a token row;
// measured: unlike the fp32 form's rows 4(l/16)+i, the fp64 form interleaves its rows). A float4
// per lane feeds four instructions: instruction i takes elements h0 + 4(l/16) + i, the same on both
// sides. Grid: (ceil(E / 16), ceil(T / 64)); wave w takes rows 16w..16w+15 of the block's 64.
// ------------------------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));

static __global__ __launch_bounds__(kThreads) void pf_logits_kernel(PfArgs a, int layer) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int E = a.E, T = a.T, H = a.H;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 64 + wave * 16;
  const float* x = pf_layer_input(a, layer);
  const float* wr = a.w.router_w + static_cast<size_t>(min(e0 + c, E - 1)) * H + 4 * q;
  const float* xr = x + static_cast<size_t>(min(t0 + c, T - 1)) * H + 4 * q;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
  for (int h0 = 0; h0 < H; h0 += 16) {  // H / 16 is a multiple of 16
    const float4 wv = load_stream_f4(wr + h0);
    const float4 xv = load_f4(xr + h0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(wv.x), static_cast<double>(xv.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(wv.y), static_cast<double>(xv.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(wv.z), static_cast<double>(xv.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(wv.w), static_cast<double>(xv.w), acc, 0, 0, 0);
  }
  const int t = t0 + c;
  if (t < T) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + q + 4 * i;
      if (e < E) {
        const double b = a.w.router_bias ? static_cast<double>(a.w.router_bias[e]) : 0.0;
        a.logits[static_cast<size_t>(t) * E + e] = acc[i] + b;
      }
    }
  }
}

// The same product with the reduction split over the block's four waves (for rounds too small to
// fill the chip with one wave per 16 x 16 tile): grid (ceil(E / 16), ceil(T / 16)); wave w sums
// h in [w H / 4, (w + 1) H / 4) and wave 0 adds the four partial sums in wave order.
static __global__ __launch_bounds__(kThreads) void pf_logits_splitk_kernel(PfArgs a, int layer) {
  __shared__ f64x4 part[kWaves - 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int E = a.E, T = a.T, H = a.H;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  const int hq = H / kWaves;  // a multiple of 64
  const float* x = pf_layer_input(a, layer);
  const float* wr = a.w.router_w + static_cast<size_t>(min(e0 + c, E - 1)) * H + wave * hq + 4 * q;
  const float* xr = x + static_cast<size_t>(min(t0 + c, T - 1)) * H + wave * hq + 4 * q;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
  for (int h0 = 0; h0 < hq; h0 += 16) {
    const float4 wv = load_stream_f4(wr + h0);
    const float4 xv = load_f4(xr + h0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(wv.x), static_cast<double>(xv.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(wv.y), static_cast<double>(xv.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(wv.z), static_cast<double>(xv.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(wv.w), static_cast<double>(xv.w), acc, 0, 0, 0);
  }
  if (wave > 0) part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) acc += part[w][lane];
  const int t = t0 + c;
  if (t < T) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + q + 4 * i;
      if (e < E) {
        const double b = a.w.router_bias ? static_cast<double>(a.w.router_bias[e]) : 0.0;
        a.logits[static_cast<size_t>(t) * E + e] = acc[i] + b;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Top-k per row (one wave each, the decode path's routine), then the row's bit in the mask of
// each chosen expert. Grid: ceil(T / 4) x 256 threads.
// ------------------------------------------------------------------------------------------
template <int NPL>
__global__ __launch_bounds__(kThreads) void pf_topk_kernel(PfArgs a, int layer) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int k = a.k;
  int id;
  float p;
  topk_row<NPL>(a.logits + static_cast<size_t>(t) * a.E, a.E, k, id, p);
  if (lane < k) {
    a.sel[t * k + lane] = id;
    a.selp[t * k + lane] = p;
    atomicOr(a.mask + static_cast<size_t>(id) * a.W + (t >> 6), 1ull << (t & 63));
  }
}

// ------------------------------------------------------------------------------------------
// Counting sort by expert. pf_scan_kernel (one block of 1024 threads): thread e < E counts expert
// e's rows word by word (recording the count before each word), and a block scan turns the counts
// into pair offsets, unique indices and work-item offsets. pf_scatter_kernel (one thread per pair)
// then puts (row t, rank j) at its expert's offset plus the rows of that expert below t (the words
// before, then the bits below t in t's word): slots are grouped by ascending expert with rows
// ascending inside, as in the decode worklist.
// ------------------------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

static __global__ __launch_bounds__(kScanThreads) void pf_scan_kernel(PfArgs a, int layer) {
  __shared__ unsigned long long s_scan[kScanThreads];
  const int tid = threadIdx.x, E = a.E, W = a.W;
  const int npairs = a.T * a.k;
  int cnt = 0;
  if (tid < E) {
    const unsigned long long* m = a.mask + static_cast<size_t>(tid) * W;
    int32_t* wp = a.wpre + static_cast<size_t>(tid) * W;
    int w = 0;
    for (; w + 8 <= W; w += 8) {  // eight loads in flight
      unsigned long long v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = m[w + j];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        wp[w + j] = cnt;
        cnt += __popcll(v[j]);
      }
    }
    for (; w < W; ++w) {
      wp[w] = cnt;
      cnt += __popcll(m[w]);
    }
  }
  // Packed inclusive scan: pairs (bits 0-23), work items (24-43), unique experts (44-63).
  const int ni = (cnt + kTile - 1) / kTile;
  const unsigned long long v = static_cast<unsigned long long>(cnt) | (static_cast<unsigned long long>(ni) << 24) |
                               (static_cast<unsigned long long>(cnt > 0) << 44);
  s_scan[tid] = v;
  __syncthreads();
  for (int d = 1; d < kScanThreads; d <<= 1) {
    const unsigned long long add = tid >= d ? s_scan[tid - d] : 0ull;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  const unsigned long long excl = s_scan[tid] - v;
  const unsigned long long all = s_scan[kScanThreads - 1];
  const int p0 = static_cast<int>(excl & 0xFFFFFF), i0 = static_cast<int>((excl >> 24) & 0xFFFFF);
  const int u = static_cast<int>(excl >> 44);
  const int nu = static_cast<int>(all >> 44), nitems = static_cast<int>((all >> 24) & 0xFFFFF);
  int32_t* uniq = a.uniq + static_cast<size_t>(layer) * E;
  int32_t* offs = a.offs + static_cast<size_t>(layer) * (E + 1);
  if (tid < E) {
    a.eoff[tid] = p0;
    if (cnt > 0) {
      uniq[u] = tid;
      offs[u] = p0;
      for (int g = 0; g < ni; ++g) a.items[i0 + g] = make_int4(tid, p0 + g * kTile, min(kTile, cnt - g * kTile), 0);
    }
  }
  if (tid == 0) {
    offs[nu] = npairs;
    a.n_unique[layer] = nu;
    *a.n_items = nitems;
  }
}

// Grid: ceil(T * k / 256) x 256 threads, one (row, rank) pair each.
static __global__ __launch_bounds__(kThreads) void pf_scatter_kernel(PfArgs a, int layer) {
  const int npairs = a.T * a.k;
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= npairs) return;
  const int t = idx / a.k, j = idx - t * a.k;
  const int e = a.sel[idx];
  const float p = a.selp[idx];
  const size_t mw = static_cast<size_t>(e) * a.W + (t >> 6);
  const int pos = min(a.eoff[e] + a.wpre[mw] + __popcll(a.mask[mw] & ((1ull << (t & 63)) - 1ull)), npairs - 1);
  a.pairs[static_cast<size_t>(layer) * a.Pcap + pos] = t | (j << 16);
  a.pair_w[pos] = p;
  a.slot_of[idx] = pos;
  const size_t o = static_cast<size_t>(layer) * npairs + idx;  // [L][T][k]
  if (a.in.ids) a.in.ids[o] = e;
  if (a.in.route_w) a.in.route_w[o] = p;
}

// ------------------------------------------------------------------------------------------
// GEMM tiles on v_mfma_i32_32x32x32_i8, one 32-weight block per instruction (the full-rate int8
// form on gfx950; the 16x16x32 form runs at half rate). A = 32 pair rows' digits of one plane,
// B = 32 weight rows' 4-bit codes as bytes; lane l supplies A row / B column l % 32 and elements
// 16(l/32)..+15 (the even elements of each 8-group, then the odd ones: the order both the weight
// nibbles and the stored digits have), and D register i of lane l holds row 8(i/4) + 4(l/32) + i%4
// (a pair) of column l % 32 (a weight row), so a lane's block scale is one value. The three digit
// planes chain through the accumulator, high plane first (D = (D << 8) + A_p B), which forms
// P = P0 + 256 P1 + 65536 P2 exactly in wrapping int32 (the sum fits); the fold is acc += s * P. The
// minimum's term sum_b m_b * sum(x)_b / step runs on v_mfma_f32_32x32x2f32 into the same
// accumulators (A = the pairs' block sums, B = the rows' minima, two blocks per instruction; the
// same D layout), and each pair's step multiplies its total at the end.
//
// Block tile: 64 pairs by 64 rows of gate and of up (gate/up) or by 128 rows (down), eight waves
// of 32 rows x 32 pairs of one matrix each (at most 128 VGPRs: four waves per SIMD). The 64 pairs'
// digits of each 4-block step go through LDS (double-buffered, one barrier per step) in
// [block][plane][half][pair][16 bytes] order, so a lane reads its 16 bytes next to its
// neighbours'. The next step's digits are loaded into registers while the current step computes
// and written to LDS after it: LDS DMA loads would make the compiler wait for them before the
// step's first LDS read, as it cannot tell the two buffers apart. Pairs past the item's last
// repeat it.
// ------------------------------------------------------------------------------------------
typedef int32_t i32x4v __attribute__((ext_vector_type(4)));
typedef int32_t i32x16v __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// The digits of blocks kb0..kb0+3 of the 64 pairs are 24 chunks (block, plane, half) of 16 bytes
// per pair; wave w moves chunks 3w..3w+2 with lane l taking pair l (from its digit row `src`).
constexpr int kChunksPerWave = 24 / kGemmWaves;
__device__ __forceinline__ void fetch_step(const uint32_t* src, int kb0, u32x4 (&v)[kChunksPerWave]) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int n = 0; n < kChunksPerWave; ++n) {
    const int ins = wave * kChunksPerWave + n;  // (bs * 3 + p) * 2 + h
    const int h = ins & 1, p = (ins >> 1) % 3, bs = (ins >> 1) / 3;
    v[n] = *reinterpret_cast<const u32x4*>(src + static_cast<size_t>(kb0 + bs) * kXqWords + p * 8 + 4 * h);
  }
}
__device__ __forceinline__ void store_step(const u32x4 (&v)[kChunksPerWave], uint32_t* buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int n = 0; n < kChunksPerWave; ++n)
    *reinterpret_cast<u32x4*>(buf + ((wave * kChunksPerWave + n) * kTile + lane) * 4) = v[n];
}

// 16 code bytes (elements 16h..16h+15 of a block) from its 8 packed bytes, in the digit order.
__device__ __forceinline__ i32x4v codes16(uint2 w) {
  return i32x4v{static_cast<int32_t>(w.x & 0x0F0F0F0Fu), static_cast<int32_t>((w.x >> 4) & 0x0F0F0F0Fu),
                static_cast<int32_t>(w.y & 0x0F0F0F0Fu), static_cast<int32_t>((w.y >> 4) & 0x0F0F0F0Fu)};
}

// A lane's 8-byte code halves of blocks kb0..kb0+3 (half l / 32 of each): lane (c, h) loads blocks
// kb0 + 2h and kb0 + 2h + 1 of row c whole (so the 32 lanes of a half-wave read 32 rows' 64 bytes in
// two 16-byte loads per lane), then the two half-waves trade the halves the other needs.
// Ordinary cached loads: a line is touched by the two steps that share it, and items of one
// expert re-read its rows.
struct StepCodes {
  u32x4 p, q;  // blocks kb0 + 2h and kb0 + 2h + 1 of this lane's row, as loaded
  uint4 smw;   // Q4B32: the scale/min words of blocks kb0..kb0+3; Q4S256: the record of their
               // super-block (a step of 4 blocks never crosses one)
};
template <int FMT>
__device__ __forceinline__ void load_step_codes(const uint8_t* row, const uint32_t* smrow, int kb0, StepCodes& w) {
  const int h = (threadIdx.x & 63) >> 5;
  w.p = *reinterpret_cast<const u32x4*>(row + 16 * (kb0 + 2 * h));
  w.q = *reinterpret_cast<const u32x4*>(row + 16 * (kb0 + 2 * h + 1));
  w.smw = *reinterpret_cast<const uint4*>(smrow + (FMT == kFmtQ4S256 ? 4 * (kb0 >> 3) : kb0));
}
// Scale and minimum of block kb0 + bs from a step's words (bs may differ between lanes).
template <int FMT>
__device__ __forceinline__ float step_scale(const uint4& smw, int kb0, int bs) {
  if constexpr (FMT == kFmtQ4S256) {
    BlockScale<kFmtQ4S256> b;
    b.r = smw;
    b.j = (kb0 & 7) + bs;
    return b.scale();
  } else {
    return half_bits_to_float(bs == 0 ? smw.x : bs == 1 ? smw.y : bs == 2 ? smw.z : smw.w);
  }
}
template <int FMT>
__device__ __forceinline__ float step_min(const uint4& smw, int kb0, int bs) {
  if constexpr (FMT == kFmtQ4S256) {
    BlockScale<kFmtQ4S256> b;
    b.r = smw;
    b.j = (kb0 & 7) + bs;
    return b.minv();
  } else {  // bs is 0/1 or 2/3 by half-wave: a select, not an indexed register
    const uint32_t hm = 0u - static_cast<uint32_t>(bs & 1);
    const uint32_t w = bs < 2 ? (smw.x ^ ((smw.x ^ smw.y) & hm)) : (smw.z ^ ((smw.z ^ smw.w) & hm));
    return half_bits_to_float(w >> 16);
  }
}
__device__ __forceinline__ void trade_halves(const StepCodes& w, uint2 (&cw)[kStepBlocks]) {
  // before: low half-wave p = block kb0 (lo, hi words), upper half-wave p = block kb0 + 2
  uint32_t p0 = w.p.x, p1 = w.p.y, p2 = w.p.z, p3 = w.p.w, q0 = w.q.x, q1 = w.q.y, q2 = w.q.z, q3 = w.q.w;
  permlane32_swap(p0, p2);  // low: (p0, p2) = kb0 lo, kb0 + 2 lo; upper: kb0 hi, kb0 + 2 hi
  permlane32_swap(p1, p3);
  permlane32_swap(q0, q2);
  permlane32_swap(q1, q3);
  cw[0] = make_uint2(p0, p1);
  cw[1] = make_uint2(q0, q1);
  cw[2] = make_uint2(p2, p3);
  cw[3] = make_uint2(q2, q3);
}

// Work unit of GEMM block `bid` of `nb` (a multiple of 8): consecutive units (the tiles of one
// work item) go to one XCD, whose L2 then holds that item's digit rows once.
__device__ __forceinline__ int xcd_unit(int bid, int nb) { return (bid & 7) * (nb >> 3) + (bid >> 3); }

// One wave's 32 weight rows (starting at codes0 / sm0 in each of NM matrices) against 32 of the
// block's 64 staged pairs (half ph). src: this lane's staging source row (pair lane % 64); xs: the
// block sums of pair 32 ph + lane % 32. live = false (no pair of this half exists): the wave only
// stages and waits. acc[m][i]: D element i, in units of the pair's step.
template <int NM, int FMT>
__device__ __forceinline__ void gemm_rows(const uint8_t* const* codes0, const uint32_t* const* sm0, int K,
                                          const uint32_t* src, const float* xs, int ph, bool live, uint32_t* lds,
                                          f32x16 (&acc)[NM]) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const int nblk = K / 32, nstep = nblk / kStepBlocks;
  const size_t rsm = sm_row_words<FMT>(K);
  live = __builtin_amdgcn_readfirstlane(static_cast<int>(live)) != 0;  // one value per wave
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;
  u32x4 nxt[kChunksPerWave];
  StepCodes cur_w[NM], nxt_w[NM];
  float x2[2], nx2[2];
  if (live) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
      load_step_codes<FMT>(codes0[m] + static_cast<size_t>(c) * (K / 2), sm0[m] + c * rsm, 0, cur_w[m]);
    x2[0] = xs[h];
    x2[1] = xs[2 + h];
  }
  fetch_step(src, 0, nxt);
  store_step(nxt, lds);
  __syncthreads();
  for (int st = 0; st < nstep; ++st) {
    const int kb0 = st * kStepBlocks;
    const uint32_t* cur = lds + (st & 1) * kStageWords;
    const bool more = st + 1 < nstep;
    // The next step's codes, scale/min words, block sums and digits are loaded while this step
    // computes (its own arrived during the previous step).
    if (live && more) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
        load_step_codes<FMT>(codes0[m] + static_cast<size_t>(c) * (K / 2), sm0[m] + c * rsm, kb0 + kStepBlocks,
                             nxt_w[m]);
      nx2[0] = xs[kb0 + kStepBlocks + h];
      nx2[1] = xs[kb0 + kStepBlocks + 2 + h];
    }
    if (more) fetch_step(src, kb0 + kStepBlocks, nxt);
    if (live) {
      uint2 cw[NM][kStepBlocks];
#pragma unroll
      for (int m = 0; m < NM; ++m) trade_halves(cur_w[m], cw[m]);
#pragma unroll
      for (int bs = 0; bs < kStepBlocks; ++bs) {
        i32x4v ap[3];
#pragma unroll
        for (int p = 0; p < 3; ++p)
          ap[p] = *reinterpret_cast<const i32x4v*>(cur + (((bs * 3 + p) * 2 + h) * kTile + 32 * ph + c) * 4);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const i32x4v b = codes16(cw[m][bs]);
          const float sc = step_scale<FMT>(cur_w[m].smw, kb0, bs);
          const i32x16v z = {};
          i32x16v d = __builtin_amdgcn_mfma_i32_32x32x32_i8(ap[2], b, z, 0, 0, 0);
          d = __builtin_amdgcn_mfma_i32_32x32x32_i8(ap[1], b, d << 8, 0, 0, 0);
          d = __builtin_amdgcn_mfma_i32_32x32x32_i8(ap[0], b, d << 8, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[m][i] = fmaf(sc, static_cast<float>(d[i]), acc[m][i]);
        }
      }
      // The minimum's term of the 4 blocks (instruction j takes blocks kb0 + 2j + l / 32), after the
      // folds: the next step's integer products then cover its latency before acc is needed again.
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const float m0 = step_min<FMT>(cur_w[m].smw, kb0, h);
        const float m1 = step_min<FMT>(cur_w[m].smw, kb0, 2 + h);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(x2[0], m0, acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x2f32(x2[1], m1, acc[m], 0, 0, 0);
      }
    }
    if (more) store_step(nxt, lds + ((st + 1) & 1) * kStageWords);  // read two steps ago
    __syncthreads();  // step st read by every wave; step st + 1 staged
    if (live && more) {
#pragma unroll
      for (int m = 0; m < NM; ++m) cur_w[m] = nxt_w[m];
      x2[0] = nx2[0];
      x2[1] = nx2[1];
    }
  }
}

// Pair (within the block's 64) of D element i for this lane.
__device__ __forceinline__ int d_pair(int ph, int i) {
  return 32 * ph + 8 * (i >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (i & 3);
}

// Gate/up: work unit = (item, 64 rows of I). Waves 0-3 take gate, 4-7 up (rows 32 (w & 1)..,
// pairs 32 ((w >> 1) & 1)..); the up waves hand their sums to the gate waves through LDS, which
// write silu(g) * v of the block's rows for the item's pairs into hbuf (by pair slot).
template <int FMT>
__global__ __launch_bounds__(kGemmThreads) void pf_gateup_kernel(PfArgs a, int layer) {
  extern __shared__ uint32_t lds[];
  const int I = a.I, H = a.H;
  const int tiles = I / kTile;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int it = unit / tiles, i0 = (unit - it * tiles) * kTile;
  if (it >= *a.n_items) return;  // whole blocks leave together
  const int4 item = a.items[it];
  const int e = item.x, p0 = item.y, np = item.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mt = wave >> 2, rh = wave & 1, ph = (wave >> 1) & 1;
  const int32_t* pairs = a.pairs + static_cast<size_t>(layer) * a.Pcap;
  __shared__ float s_step[kTile];  // the item's pairs' steps, for the epilogue
  const int tsrc = pairs[p0 + min(lane, np - 1)] & 0xFFFF;                  // staging: pair lane
  if (wave == 0) s_step[lane] = a.xstep[tsrc];  // visible after the GEMM's first barrier
  const int tsum = pairs[p0 + min(32 * ph + (lane & 31), np - 1)] & 0xFFFF;  // block sums: A row
  const uint32_t* src = a.xq + static_cast<size_t>(tsrc) * (H / 32) * kXqWords;
  const float* xs = a.xsum + static_cast<size_t>(tsum) * (H / 32);
  const size_t row = static_cast<size_t>(e) * I + i0 + 32 * rh;  // the wave's first weight row
  const uint8_t* codes[1] = {(mt ? a.w.up_q : a.w.gate_q) + row * (H / 2)};
  const uint32_t* sm[1] = {(mt ? a.w.up_sm : a.w.gate_sm) + row * sm_row_words<FMT>(H)};
  f32x16 acc[1];
  gemm_rows<1, FMT>(codes, sm, H, src, xs, ph, 32 * ph < np, lds, acc);
  // The staging buffers are free (the GEMM ends on a barrier): up sums [rh][ph][i][lane].
  float* xch = reinterpret_cast<float*>(lds) + ((rh * 2 + ph) * 16) * 64 + lane;
  if (mt == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) xch[i * 64] = acc[0][i];
  }
  __syncthreads();
  if (mt == 0) {
    const int col = i0 + 32 * rh + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int pr = d_pair(ph, i);
      const float step = s_step[pr];
      if (pr < np) a.hbuf[static_cast<size_t>(p0 + pr) * I + col] = silu(step * acc[0][i]) * (step * xch[i * 64]);
    }
  }
}

// Down: work unit = (item, 128 rows of H); wave w takes rows 32 (w & 3).. and pairs 32 (w >> 2)...
// Writes W_d h of the block's rows for the item's pairs into ybuf (by pair slot).
constexpr int kDownRows = 128;
template <int FMT>
__global__ __launch_bounds__(kGemmThreads) void pf_down_kernel(PfArgs a, int layer) {
  extern __shared__ uint32_t lds[];
  const int I = a.I, H = a.H;
  const int tiles = H / kDownRows;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int it = unit / tiles, h0 = (unit - it * tiles) * kDownRows;
  if (it >= *a.n_items) return;
  const int4 item = a.items[it];
  const int e = item.x, p0 = item.y, np = item.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rq = wave & 3, ph = wave >> 2;
  __shared__ float s_step[kTile];
  const uint32_t* src = a.hq + static_cast<size_t>(p0 + min(lane, np - 1)) * (I / 32) * kXqWords;
  if (wave == 0) s_step[lane] = a.hstep[p0 + min(lane, np - 1)];  // visible after the first barrier
  const float* xs = a.hsum + static_cast<size_t>(p0 + min(32 * ph + (lane & 31), np - 1)) * (I / 32);
  const size_t row = static_cast<size_t>(e) * H + h0 + 32 * rq;
  const uint8_t* codes[1] = {a.w.down_q + row * (I / 2)};
  const uint32_t* sm[1] = {a.w.down_sm + row * sm_row_words<FMT>(I)};
  f32x16 acc[1];
  gemm_rows<1, FMT>(codes, sm, I, src, xs, ph, 32 * ph < np, lds, acc);
  const int col = h0 + 32 * rq + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int pr = d_pair(ph, i);
    const float step = s_step[pr];
    if (pr < np) a.ybuf[static_cast<size_t>(p0 + pr) * H + col] = step * acc[0][i];
  }
}

// out[t][h] = (residual ? x[t][h] : 0) + sum over ranks j = 0..k-1, in that order, of
// p[t][j] * y[slot(t, j)][h]. Grid (T, ceil(H / 1024)) x 256 threads, four columns per thread.
static __global__ __launch_bounds__(kThreads) void pf_combine_kernel(PfArgs a, int layer) {
  const float* __restrict__ x = pf_layer_input(a, layer);
  float* __restrict__ xn = pf_layer_output(a, layer);
  const int t = blockIdx.x, H = a.H, k = a.k;
  const int h = (blockIdx.y * kThreads + threadIdx.x) * 4;
  if (h >= H) return;
  float4 acc = a.residual ? load_f4(x + static_cast<size_t>(t) * H + h) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int s = min(max(a.slot_of[t * k + j], 0), a.Pcap - 1);
    const float w = a.pair_w[s];
    const float4 y = load_f4(a.ybuf + static_cast<size_t>(s) * H + h);
    acc.x = fmaf(w, y.x, acc.x);
    acc.y = fmaf(w, y.y, acc.y);
    acc.z = fmaf(w, y.z, acc.z);
    acc.w = fmaf(w, y.w, acc.w);
  }
  *reinterpret_cast<float4*>(xn + static_cast<size_t>(t) * H + h) = acc;
}

}  // namespace pf
}  // namespace moe
