// Prefill MoE: rounds of more than 64 rows, where the expert FFN is compute-bound.
//
// Per layer nine kernels, launched eagerly:
//   quant_rows_kernel   the layer input, scaled per row by a power of two, as pairs of fp16 values
//                       (hi + lo) and per-32-block sums, for the fp16 matrix cores
//   pf_logits_kernel    router GEMM on fp64 matrix cores (fp32 inputs, fp64 products and sums)
//   pf_topk_kernel      one wave per row: top-k, softmax over the selected, and the row's bit in
//                       each chosen expert's row mask
//   pf_scan_kernel      one block: rows per expert, their offsets, the unique list and the
//                       64-pair work items
//   pf_scatter_kernel   counting sort of the (row, rank) pairs by expert (ascending expert, rows
//                       ascending within one); the caller's ids and routing weights
//   pf_gateup_kernel    per work item and 64 rows of I: silu(W_g x) * (W_u x) as an fp16 GEMM
//   quant_rows_kernel   the SwiGLU rows as fp16 pairs
//   pf_down_kernel      per work item and 128 rows of H: W_d h per pair, into a slot buffer
//   pf_combine_kernel   each row adds its k products in rank order (and the residual)
//
// The infero README, "Beyond plain text decode", routes prefill through a counting sort followed
// by a GEMM per expert; its "Design notes" run batched projections straight off the quantised
// weights on matrix instructions, per 32-weight block, with the block scales applied in float
// afterwards. Here each activation is split into two fp16 values, hi + lo, after a power-of-two
// scaling of its row, which keeps 22 significant bits; the 4-bit codes are exact in fp16, so each
// block product is an fp32 sum of exact products and the fp32 fold keeps the round within the
// fp32-accumulation tolerance of the decode path. The block minimum's term sum_b m * sum(x) runs
// on fp32 matrix instructions.
#pragma once

#include "moe_common.h"
#include "moe_gemv.h"
#include "moe_route.h"

namespace moe {
namespace pf {

constexpr int kTile = 64;                 // GEMM tile: 64 (row, rank) pairs by 64 or 128 weight rows
constexpr int kGemmThreads = 512;         // down GEMM blocks: 8 waves, each 32 weight rows x 32 pairs
constexpr int kRowExp = 14;               // scaled rows: |x / step| < 2^14, well inside fp16's range
constexpr int kPfWords = 32;              // words per 32-block of a row: [hi/lo][group of 8][4 words]
constexpr int kStepBlocks = 4;            // 32-blocks of the reduction per pipeline step
constexpr int kStepChunks = kStepBlocks * 8;  // 16-byte chunks of one row per step: (block, plane, group)
// A row is stored as steps of 4 blocks: the blocks' 32 chunks, then their 4 sums (blocks 0, 2, 1, 3).
constexpr int kStepWords = kStepChunks * 4 + 4;
__host__ __device__ constexpr int pf_row_words(int K) { return K / (32 * kStepBlocks) * kStepWords; }
// LDS per GEMM block: two buffers of [pair][step words]. The 4 words of sums keep both the 16-byte
// writes (one pair's chunks across a half-wave) and the 16-byte reads (one chunk of 32 consecutive
// pairs) free of bank conflicts.
constexpr int kPairStride = kStepWords;
constexpr int kStageWords = kTile * kPairStride;
constexpr int kGemmLds = 2 * kStageWords * 4;

struct PfArgs {
  Ingress in;
  moe_layer_weights w;
  float* xbuf0;          // [Tp][H] layer outputs between layers (L > 1)
  float* xbuf1;
  double* logits;        // [Tp][E]
  uint32_t* xq;          // [Tp][pf_row_words(H)] fp16 pairs and block sums of the layer input
  float* xstep;          // [Tp] its per-row step (a power of two)
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
  uint32_t* hq;          // [Pcap][pf_row_words(I)]
  float* hstep;          // [Pcap]
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
// Rows as fp16 pairs: one wave per row of K floats. The row is scaled by step = 2^(e - kRowExp),
// where max|x| < 2^e, so |x / step| < 2^14 (an exact scaling); each scaled value v becomes
// hi = fp16(v) and lo = fp16(v - hi), both rounded to nearest (v - hi is exact in fp32), which
// leaves |v - hi - lo| <= 2^-22 |v| + 2^-25. Stored per 32-block as [plane hi, lo][group g of 8]
// [word j = 0..3], word j holding elements 8g + j (low half) and 8g + 4 + j (high half): the order
// in which a weight code word's nibbles unpack; each 4 blocks are followed by their sums of v (fp32).
// Grid: ceil(n / 4) x 256 threads. zero_words / zero: words of `zero` cleared by the grid on the
// side (the layer's row masks).
// ------------------------------------------------------------------------------------------
static __global__ __launch_bounds__(kThreads) void quant_rows_kernel(const float* __restrict__ src, int K, int n,
                                                                   uint32_t* dig, float* step_out,
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
  int ex = 0;
  frexpf(rmax, &ex);       // rmax < 2^ex
  ex = max(ex, -100);      // keeps step a normal float
  const float step = rmax > 0.f ? ldexpf(1.f, ex - kRowExp) : 1.f;
  const float inv = rmax > 0.f ? ldexpf(1.f, kRowExp - ex) : 0.f;
  if (lane == 0) step_out[row] = step;
  uint32_t* drow = dig + static_cast<size_t>(row) * pf_row_words(K);
  for (int c0 = 0; c0 < n4; c0 += 64) {  // K / 4 is a multiple of 8: a block's 8 lanes are all in or out
    const int c = c0 + lane;
    const bool in = c < n4;
    const float4 v = load_f4(x + 4 * min(c, n4 - 1));
    const float e[4] = {v.x * inv, v.y * inv, v.z * inv, v.w * inv};
    float sum = (e[0] + e[1]) + (e[2] + e[3]);
    sum += dpp_f32<kDppXor1>(sum);
    sum += dpp_f32<kDppXor2>(sum);
    sum += dpp_f32<kDppHalfMirror>(sum);  // the 8 lanes of this block
    // Elements 4 sub + i of the block (sub = lane % 8) are word i of group sub / 2 in each plane:
    // the low half for even sub, the high half for odd. Lanes 2m and 2m + 1 trade halves, so the
    // even lane stores the group's 4 hi-plane words and the odd lane its 4 lo-plane words.
    const int half = lane & 1;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 hi = static_cast<_Float16>(e[i]);
      const _Float16 lo = static_cast<_Float16>(e[i] - static_cast<float>(hi));
      const uint32_t hb = __builtin_bit_cast(uint16_t, hi), lb = __builtin_bit_cast(uint16_t, lo);
      const uint32_t got = dpp_u32<kDppXor1>(half ? hb : lb);  // the partner's hi (to an even lane) or lo
      w[i] = half ? (got | (lb << 16)) : (hb | (got << 16));
    }
    if (in) {
      const int b = c >> 3, g = (c & 7) >> 1;
      uint32_t* step_w = drow + (b >> 2) * kStepWords;
      *reinterpret_cast<uint4*>(step_w + (b & 3) * kPfWords + (half * 4 + g) * 4) = make_uint4(w[0], w[1], w[2], w[3]);
      if ((c & 7) == 0) reinterpret_cast<float*>(step_w)[kStepChunks * 4 + (b & 1) * 2 + ((b >> 1) & 1)] = sum;
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
// sides.
// ------------------------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));

// Large rounds: a block computes 32 experts x 32 rows, its four waves splitting the reduction in
// quarters (wave w sums h in [w H / 4, (w + 1) H / 4)), each wave holding the four 16 x 16 tiles of
// the block's output; wave 0 adds the quarters in wave order. Four loads (two router rows' and two
// input rows' float4 per lane) feed sixteen matrix instructions, twice the work per loaded byte of
// a 16 x 16 tile. Grid: (ceil(E / 32), ceil(T / 32)).
static __global__ __launch_bounds__(kThreads) void pf_logits_kernel(PfArgs a, int layer) {
  __shared__ f64x4 part[kWaves - 1][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int E = a.E, T = a.T, H = a.H;
  const int e0 = blockIdx.x * 32, t0 = blockIdx.y * 32;
  const int hq = H / kWaves;  // a multiple of 64
  const float* x = pf_layer_input(a, layer);
  const float* wr0 = a.w.router_w + static_cast<size_t>(min(e0 + c, E - 1)) * H + wave * hq + 4 * q;
  const float* wr1 = a.w.router_w + static_cast<size_t>(min(e0 + 16 + c, E - 1)) * H + wave * hq + 4 * q;
  const float* xr0 = x + static_cast<size_t>(min(t0 + c, T - 1)) * H + wave * hq + 4 * q;
  const float* xr1 = x + static_cast<size_t>(min(t0 + 16 + c, T - 1)) * H + wave * hq + 4 * q;
  f64x4 acc[4] = {};  // [expert half * 2 + row half]
#pragma unroll 4
  for (int h0 = 0; h0 < hq; h0 += 16) {
    const float4 w0 = load_stream_f4(wr0 + h0), w1 = load_stream_f4(wr1 + h0);
    const float4 x0 = load_f4(xr0 + h0), x1 = load_f4(xr1 + h0);
    const float wv[2][4] = {{w0.x, w0.y, w0.z, w0.w}, {w1.x, w1.y, w1.z, w1.w}};
    const float xv[2][4] = {{x0.x, x0.y, x0.z, x0.w}, {x1.x, x1.y, x1.z, x1.w}};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(wv[b >> 1][j]), static_cast<double>(xv[b & 1][j]),
                                                      acc[b], 0, 0, 0);
  }
  if (wave > 0) {
#pragma unroll
    for (int b = 0; b < 4; ++b) part[wave - 1][b][lane] = acc[b];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] += part[w][b][lane];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int t = t0 + 16 * (b & 1) + c;
    if (t < T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + 16 * (b >> 1) + q + 4 * i;
        if (e < E) {
          const double bias = a.w.router_bias ? static_cast<double>(a.w.router_bias[e]) : 0.0;
          a.logits[static_cast<size_t>(t) * E + e] = acc[b][i] + bias;
        }
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
  topk_row<NPL, kWaves>(a.logits + static_cast<size_t>(t) * a.E, a.E, k, id, p);
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
// GEMM tiles on v_mfma_f32_32x32x16_f16, two instructions per 32-weight block and plane. A = 32
// pair rows' fp16 values of one plane, B = 32 weight rows' 4-bit codes as exact fp16 values; lane
// l supplies A row / B column l % 32 and 8 elements of the instruction's 16, and D register i of
// lane l holds row 8(i/4) + 4(l/32) + i%4 (a pair) of column l % 32 (a weight row), so a lane's
// block scale is one value. Instruction s of a block takes group 2(l/32) + s of it in both
// operands (in the order of the unpacked code nibbles), which covers the block's 32 elements. The
// block's four products (lo plane first, then hi) sum in the matrix core's fp32 accumulator and
// the fold is acc += s * P. The minimum's term sum_b m_b * sum(x)_b / step runs on
// v_mfma_f32_32x32x2f32 into the same accumulators (A = the pairs' block sums, B = the rows'
// minima, two blocks per instruction; the same D layout; the sums come with the staged values),
// and each pair's step multiplies its total at the end.
//
// Block tile: 64 pairs by 64 rows of gate and of up (gate/up) or by 128 rows (down). Down has
// eight waves of 32 rows x 32 pairs (at most 128 VGPRs: four waves per SIMD). Gate/up has four
// waves of 32 rows x 64 pairs, as two 32-pair tiles that share every unpacked code word (at most
// 256 VGPRs: two waves per SIMD). The 64 pairs' values of each 4-block step go through LDS
// (double-buffered, one barrier per step). A step of a pair's row is 528 contiguous bytes, and a
// half-wave loads its 512 bytes of values whole, so a load instruction touches 8 cache lines
// rather than one per lane (one more load per wave takes its pairs' sums). The next step's values are loaded
// into registers while the current step computes
// and written to LDS after it: LDS DMA loads would make the compiler wait for them before the
// step's first LDS read, as it cannot tell the two buffers apart. Pairs past the item's last
// repeat it.
// ------------------------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Step st of the 64 pairs' rows: 32 chunks (block, plane, group) of 16 bytes per pair, then the
// chunk of block sums. With NW waves per block, wave w stages pairs P w.. P w + P - 1 (P = 64 / NW):
// load n moves pair P w + 2n + l / 32, whose row starts at word offs[n] of `base`, with lane l
// taking chunk l % 32; the last load takes the sums of pair P w + l % P (row offset soff), which
// lanes 0..P-1 store.
template <int NW>
struct Staging {
  static constexpr int kPairs = kTile / NW;      // pairs staged per wave
  static constexpr int kLoads = kPairs / 2;      // 512-byte loads per wave and step (two pairs each)
  __device__ static __forceinline__ int pair(int n) {
    return (threadIdx.x >> 6) * kPairs + 2 * n + ((threadIdx.x & 63) >> 5);
  }
  __device__ static __forceinline__ void fetch(const uint32_t* base, const uint32_t (&offs)[kLoads], uint32_t soff,
                                               int st, u32x4 (&v)[kLoads + 1]) {
    const uint32_t j = threadIdx.x & 31, sw = static_cast<uint32_t>(st) * kStepWords;
#pragma unroll
    for (int n = 0; n < kLoads; ++n) v[n] = *reinterpret_cast<const u32x4*>(base + (offs[n] + sw + 4 * j));
    v[kLoads] = *reinterpret_cast<const u32x4*>(base + (soff + sw + kStepChunks * 4));
  }
  __device__ static __forceinline__ void store(const u32x4 (&v)[kLoads + 1], uint32_t* buf) {
    const int lane = threadIdx.x & 63, j = lane & 31;
#pragma unroll
    for (int n = 0; n < kLoads; ++n) *reinterpret_cast<u32x4*>(buf + pair(n) * kPairStride + 4 * j) = v[n];
    if (lane < kPairs)
      *reinterpret_cast<u32x4*>(buf + ((threadIdx.x >> 6) * kPairs + lane) * kPairStride + kStepChunks * 4) = v[kLoads];
  }
};

// The 8 codes of one code word (a group of 8 weights, nibble j = element j) as fp16 values in the
// order elements j, 4 + j for j = 0..3: each nibble pair goes into the mantissas of 1024.0 (fp16
// 0x6400, whose unit in the last place is 1), and 1024 is subtracted exactly.
// `magic` holds 0x64006400 in a register, so that mask-and-insert is one v_and_or_b32 (a VOP3 form,
// which takes no second literal).
__device__ __forceinline__ f16x8 codes8(uint32_t w, uint32_t magic) {
  const f16x2 off = {static_cast<_Float16>(1024.f), static_cast<_Float16>(1024.f)};
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2 v = __builtin_bit_cast(f16x2, ((w >> (4 * j)) & 0x000F000Fu) | magic) - off;
    r[2 * j] = v[0];
    r[2 * j + 1] = v[1];
  }
  return r;
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
// work item) go to one XCD, whose L2 then holds that item's activation rows once.
__device__ __forceinline__ int xcd_unit(int bid, int nb) { return (bid & 7) * (nb >> 3) + (bid >> 3); }

// One wave's 32 weight rows (codes0 / sm0) against NT 32-pair tiles of the block's 64 staged
// pairs, halves ph0 .. ph0 + NT - 1 (the block has 8 / NT waves); two tiles share every unpacked
// code word. base + src: this lane's pair's row (pair lane % 64, as a word offset below 2^32).
// ntiles: how many of the NT tiles hold pairs (0 for a wave of one empty tile: it only stages and
// waits). acc[t][i]: D element i of tile t, in units of the pair's step.
template <int FMT, int NT>
__device__ __forceinline__ void gemm_rows(const uint8_t* codes0, const uint32_t* sm0, int K, const uint32_t* base,
                                          uint32_t src, int ph0, int ntiles, uint32_t* lds, f32x16 (&acc)[NT]) {
  using S = Staging<8 / NT>;
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const int nblk = K / 32, nstep = nblk / kStepBlocks;
  const size_t rsm = sm_row_words<FMT>(K);
  ntiles = __builtin_amdgcn_readfirstlane(ntiles);  // one value per wave
  const bool live = ntiles > 0;
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));  // kept in a VGPR (see codes8)
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  // The rows this lane stages: those of pairs S::pair(n), whose lanes hold them as `src`.
  uint32_t srcs[S::kLoads];
#pragma unroll
  for (int n = 0; n < S::kLoads; ++n) srcs[n] = __shfl(src, S::pair(n));
  const uint32_t ssrc = __shfl(src, (threadIdx.x >> 6) * S::kPairs + (lane & (S::kPairs - 1)));
  u32x4 nxt[S::kLoads + 1];
  StepCodes cur_w, nxt_w;
  if (live) load_step_codes<FMT>(codes0 + static_cast<size_t>(c) * (K / 2), sm0 + c * rsm, 0, cur_w);
  S::fetch(base, srcs, ssrc, 0, nxt);
  S::store(nxt, lds);
  __syncthreads();
  for (int st = 0; st < nstep; ++st) {
    const int kb0 = st * kStepBlocks;
    const uint32_t* cur = lds + (st & 1) * kStageWords;
    const bool more = st + 1 < nstep;
    // The next step's codes, scale/min words and staged values are loaded while this step
    // computes (its own arrived during the previous step).
    if (live && more)
      load_step_codes<FMT>(codes0 + static_cast<size_t>(c) * (K / 2), sm0 + c * rsm, kb0 + kStepBlocks, nxt_w);
    if (more) S::fetch(base, srcs, ssrc, st + 1, nxt);
    if (live) {
      uint2 cw[kStepBlocks];
      trade_halves(cur_w, cw);
      const uint32_t* prow[NT];
      float2 x2[NT];  // the step's block sums of the tile's pairs (blocks kb0 + h, kb0 + 2 + h)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        prow[t] = cur + (32 * (ph0 + t) + c) * kPairStride;
        x2[t] = *reinterpret_cast<const float2*>(prow[t] + kStepChunks * 4 + 2 * h);
      }
#pragma unroll
      for (int bs = 0; bs < kStepBlocks; ++bs) {
        const f16x8 b0 = codes8(cw[bs].x, magic), b1 = codes8(cw[bs].y, magic);
        const float sc = step_scale<FMT>(cur_w.smw, kb0, bs);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (NT > 1) {
            if (t >= ntiles) break;
          }
          f16x8 ap[2][2];  // [plane][instruction]: group 2h + s of the block
#pragma unroll
          for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int q = 0; q < 2; ++q)
              ap[p][q] = *reinterpret_cast<const f16x8*>(prow[t] + ((bs * 2 + p) * 4 + 2 * h + q) * 4);
          const f32x16 z = {};
          f32x16 d = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap[1][0], b0, z, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap[1][1], b1, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap[0][0], b0, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap[0][1], b1, d, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[t][i] = fmaf(sc, d[i], acc[t][i]);
        }
      }
      // The minimum's term of the 4 blocks (instruction j takes blocks kb0 + 2j + l / 32), after
      // the folds: the next step's products then cover its latency before acc is needed again.
      const float m0 = step_min<FMT>(cur_w.smw, kb0, h), m1 = step_min<FMT>(cur_w.smw, kb0, 2 + h);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (NT > 1) {
          if (t >= ntiles) break;
        }
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(x2[t].x, m0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(x2[t].y, m1, acc[t], 0, 0, 0);
      }
    }
    if (more) S::store(nxt, lds + ((st + 1) & 1) * kStageWords);  // read two steps ago
    __syncthreads();  // step st read by every wave; step st + 1 staged
    if (live && more) cur_w = nxt_w;
  }
}

// Pair (within the block's 64) of D element i of pair half ph for this lane.
__device__ __forceinline__ int d_pair(int ph, int i) {
  return 32 * ph + 8 * (i >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (i & 3);
}

// Gate/up: work unit = (item, 64 rows of I), 8 / NT waves. NT = 2 (the form launched): waves 0-1
// take gate, 2-3 up (rows 32 (w & 1)..), each against all 64 pairs as two tiles. NT = 1: waves 0-3
// gate, 4-7 up (rows 32 (w & 1).., pairs 32 ((w >> 1) & 1)..). The up waves hand their sums to the
// gate waves through LDS, which write silu(g) * v of the block's rows for the item's pairs into
// hbuf (by pair slot).
template <int FMT, int NT>
__global__ __launch_bounds__(64 * 8 / NT) __attribute__((amdgpu_waves_per_eu(4 / NT))) void pf_gateup_kernel(
    PfArgs a, int layer) {
  extern __shared__ uint32_t lds[];
  const int I = a.I, H = a.H;
  const int tiles = I / kTile;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int it = unit / tiles, i0 = (unit - it * tiles) * kTile;
  if (it >= *a.n_items) return;  // whole blocks leave together
  const int4 item = a.items[it];
  const int e = item.x, p0 = item.y, np = item.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mt = NT == 2 ? wave >> 1 : wave >> 2, rh = wave & 1, ph0 = NT == 2 ? 0 : (wave >> 1) & 1;
  const int ntiles = NT == 2 ? (np > 32 ? 2 : 1) : (32 * ph0 < np ? 1 : 0);
  const int32_t* pairs = a.pairs + static_cast<size_t>(layer) * a.Pcap;
  __shared__ float s_step[kTile];  // the item's pairs' steps, for the epilogue
  const int tsrc = pairs[p0 + min(lane, np - 1)] & 0xFFFF;  // staging: pair lane
  if (wave == 0) s_step[lane] = a.xstep[tsrc];  // visible after the GEMM's first barrier
  const uint32_t src = static_cast<uint32_t>(tsrc) * static_cast<uint32_t>(pf_row_words(H));
  const size_t row = static_cast<size_t>(e) * I + i0 + 32 * rh;  // the wave's first weight row
  const uint8_t* codes = (mt ? a.w.up_q : a.w.gate_q) + row * (H / 2);
  const uint32_t* sm = (mt ? a.w.up_sm : a.w.gate_sm) + row * sm_row_words<FMT>(H);
  f32x16 acc[NT];
  gemm_rows<FMT, NT>(codes, sm, H, a.xq, src, ph0, ntiles, lds, acc);
  // The staging buffers are free (the GEMM ends on a barrier): up sums [rh][pair half][i][lane].
  float* xch = reinterpret_cast<float*>(lds) + lane;
  if (mt == 1) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) xch[((rh * 2 + ph0 + t) * 16 + i) * 64] = acc[t][i];
  }
  __syncthreads();
  if (mt == 0) {
    const int col = i0 + 32 * rh + (lane & 31);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pr = d_pair(ph0 + t, i);
        const float step = s_step[pr];
        if (pr < np)
          a.hbuf[static_cast<size_t>(p0 + pr) * I + col] =
              silu(step * acc[t][i]) * (step * xch[((rh * 2 + ph0 + t) * 16 + i) * 64]);
      }
  }
}
constexpr int kGateupTiles = 2;  // tiles per gate/up wave: 4 waves of 32 rows x 64 pairs
constexpr int kGateupThreads = 64 * 8 / kGateupTiles;

// Down: work unit = (item, 128 rows of H), 8 waves; wave w takes rows 32 (w & 3).. and pairs
// 32 (w >> 2)... (Down's reduction is 4 steps at I = 512; with two tiles per wave and so two waves
// per SIMD it was slower.) Writes W_d h of the block's rows for the item's pairs into ybuf (by pair
// slot).
constexpr int kDownRows = 128;
template <int FMT>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(4))) void pf_down_kernel(PfArgs a, int layer) {
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
  const uint32_t src = static_cast<uint32_t>(p0 + min(lane, np - 1)) * static_cast<uint32_t>(pf_row_words(I));
  if (wave == 0) s_step[lane] = a.hstep[p0 + min(lane, np - 1)];  // visible after the first barrier
  const size_t row = static_cast<size_t>(e) * H + h0 + 32 * rq;
  const uint8_t* codes = a.w.down_q + row * (I / 2);
  const uint32_t* sm = a.w.down_sm + row * sm_row_words<FMT>(I);
  f32x16 acc[1];
  gemm_rows<FMT, 1>(codes, sm, I, a.hq, src, ph, 32 * ph < np ? 1 : 0, lds, acc);
  const int col = h0 + 32 * rq + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int pr = d_pair(ph, i);
    const float step = s_step[pr];
    if (pr < np) a.ybuf[static_cast<size_t>(p0 + pr) * H + col] = step * acc[0][i];
  }
}

// Down for I <= kDown32MaxI (NSTEP = I / 128 steps): work unit = (item, pair half, 256 rows of H),
// 8 waves, wave w taking rows 32 w.. against the half's (up to) 32 pairs. The block copies those
// pairs' whole rows into LDS once (70 KB at I = 512, so two blocks share a CU and one block's copy
// overlaps the other's compute; a row's words in order, consecutive lanes reading consecutive 16
// bytes of one row), then each wave runs its NSTEP steps with no barrier, its codes loaded two steps
// ahead; the step loop is unrolled, so the code registers rotate without copies. Per unit of work
// this copies the rows half as often as pf_down_kernel. Each pair's row is padded to a stride of
// 4 words mod 32, so the 16-byte reads of 32 consecutive pairs are free of bank conflicts.
constexpr int kDown32Rows = 256;
constexpr int kDown32MaxI = 512;
__host__ __device__ constexpr int down32_stride(int I) { return pf_row_words(I) + (36 - pf_row_words(I) % 32) % 32; }
__host__ __device__ constexpr int down32_lds(int I) { return 32 * down32_stride(I) * 4; }
template <int FMT, int NSTEP>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(4))) void pf_down32_kernel(PfArgs a, int layer) {
  extern __shared__ uint32_t lds[];
  constexpr int I = NSTEP * 32 * kStepBlocks;
  constexpr int RW = pf_row_words(I), PS = down32_stride(I), RQ = RW / 4;
  constexpr int kCopies = (32 * RQ + kGemmThreads - 1) / kGemmThreads;
  const int H = a.H;
  const int tiles = H / kDown32Rows;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int it = unit / (2 * tiles), rem = unit - it * 2 * tiles, half = rem / tiles;
  const int h0 = (rem - half * tiles) * kDown32Rows;
  if (it >= *a.n_items) return;  // whole blocks leave together
  const int4 item = a.items[it];
  const int e = item.x, q0 = item.y + 32 * half, nq = min(32, item.z - 32 * half);
  if (nq <= 0) return;           // an item of at most 32 pairs has no second half
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 31, h = lane >> 5;
  __shared__ float s_step[32];
  if (tid < 32) s_step[tid] = a.hstep[q0 + min(tid, nq - 1)];
  // The wave's weight rows and the first two steps' codes, issued before the copy.
  const size_t row = static_cast<size_t>(e) * H + h0 + 32 * wave + c;
  const uint8_t* codes = a.w.down_q + row * (I / 2);
  const uint32_t* sm = a.w.down_sm + row * sm_row_words<FMT>(I);
  StepCodes w[NSTEP];
#pragma unroll
  for (int st = 0; st < (NSTEP < 2 ? NSTEP : 2); ++st) load_step_codes<FMT>(codes, sm, st * kStepBlocks, w[st]);
  // The half's 32 pair rows (pairs past nq repeat the last): 16-byte chunk q is chunk q % RQ of pair q / RQ.
  {
    u32x4 v[kCopies];
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int q = min(tid + i * kGemmThreads, 32 * RQ - 1);
      const int pr = q / RQ, r = q - pr * RQ;
      v[i] = *reinterpret_cast<const u32x4*>(a.hq + static_cast<size_t>(q0 + min(pr, nq - 1)) * RW + 4 * r);
    }
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int q = tid + i * kGemmThreads;
      if (q < 32 * RQ) {
        const int pr = q / RQ, r = q - pr * RQ;
        *reinterpret_cast<u32x4*>(lds + pr * PS + 4 * r) = v[i];
      }
    }
  }
  __syncthreads();
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));  // kept in a VGPR (see codes8)
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const uint32_t* prow0 = lds + c * PS;
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    if (st + 2 < NSTEP) load_step_codes<FMT>(codes, sm, (st + 2) * kStepBlocks, w[st + 2]);
    const int kb0 = st * kStepBlocks;
    const uint32_t* prow = prow0 + st * kStepWords;
    const float2 x2 = *reinterpret_cast<const float2*>(prow + kStepChunks * 4 + 2 * h);
    uint2 cw[kStepBlocks];
    trade_halves(w[st], cw);
#pragma unroll
    for (int bs = 0; bs < kStepBlocks; ++bs) {
      const f16x8 b0 = codes8(cw[bs].x, magic), b1 = codes8(cw[bs].y, magic);
      const float sc = step_scale<FMT>(w[st].smw, kb0, bs);
      f16x8 ap[2][2];  // [plane][instruction]: group 2h + s of the block
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          ap[p][q] = *reinterpret_cast<const f16x8*>(prow + ((bs * 2 + p) * 4 + 2 * h + q) * 4);
      const f32x16 z = {};
      f32x16 d = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap[1][0], b0, z, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap[1][1], b1, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap[0][0], b0, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap[0][1], b1, d, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = fmaf(sc, d[i], acc[i]);
    }
    const float m0 = step_min<FMT>(w[st].smw, kb0, h), m1 = step_min<FMT>(w[st].smw, kb0, 2 + h);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x2.x, m0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x2.y, m1, acc, 0, 0, 0);
  }
  const int col = h0 + 32 * wave + c;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int pr = d_pair(0, i);
    const float step = s_step[pr];
    if (pr < nq) a.ybuf[static_cast<size_t>(q0 + pr) * H + col] = step * acc[i];
  }
}

// out[t][h] = (residual ? x[t][h] : 0) + sum over ranks j = 0..k-1, in that order, of
// p[t][j] * y[slot(t, j)][h]. Grid (T, ceil(H / 1024)) x 256 threads, four columns per thread.
static __global__ __launch_bounds__(kThreads) void pf_combine_kernel(PfArgs a, int layer) {
  const float* x = pf_layer_input(a, layer);  // may be xn itself (the caller's hidden == out)
  float* xn = pf_layer_output(a, layer);
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
