// Prefill MoE: rounds of more than 64 rows, where the expert FFN is compute-bound.
//
// Per layer eight kernels, launched eagerly:
//   quant_rows_kernel   the layer input as 22-bit integers per row (three int8 digit planes) and
//                       per-32-block sums, for the int8 matrix cores
//   pf_logits_kernel    router GEMM on fp64 matrix cores (fp32 inputs, fp64 products and sums)
//   pf_topk_kernel      one wave per row: top-k, softmax over the selected, and the row's bit in
//                       each chosen expert's row mask
//   pf_scan_kernel      one block: counting sort of the (row, rank) pairs by expert (ascending
//                       expert, rows ascending within one), 64-row work items, the caller's ids
//   pf_gateup_kernel    per work item and 64 rows of I: silu(W_g x) * (W_u x) as an int8 GEMM
//   quant_rows_kernel   the SwiGLU rows as digits
//   pf_down_kernel      per work item and 64 rows of H: W_d h per pair, into a slot buffer
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
#include "moe_route.h"

namespace moe {
namespace pf {

constexpr int kTile = 64;                 // GEMM tile: 64 weight rows x 64 (row, rank) pairs
constexpr float kQMax = 4194303.0f;       // 2^22 - 1: 32 * 15 * kQMax < 2^31 (int32 block dots)
constexpr int kStepBlocks = 4;            // 32-blocks of the reduction per pipeline step
// LDS per GEMM block: two buffers of [block][plane][group][column][even, odd] digit words.
constexpr int kStageWords = kStepBlocks * 3 * 4 * kTile * 2;
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
  for (int h0 = 0; h0 < H; h0 += 16) {
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
// Counting sort by expert, one block of 1024 threads. Thread e < E counts expert e's rows word by
// word (recording the count before each word), a block scan turns counts into pair offsets, unique
// indices and work-item offsets, and each (row t, rank j) pair lands at its expert's offset plus
// the rows of that expert below t (the words before, then the bits below t in t's word): slots
// are grouped by ascending expert with rows ascending inside, as in the decode worklist.
// ------------------------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

static __global__ __launch_bounds__(kScanThreads) void pf_scan_kernel(PfArgs a, int layer) {
  __shared__ unsigned long long s_scan[kScanThreads];
  __shared__ int s_off[MOE_ROUND_MAX_EXPERTS];
  const int tid = threadIdx.x, E = a.E, W = a.W, T = a.T, k = a.k;
  const int npairs = T * k;
  int cnt = 0;
  if (tid < E) {
    const unsigned long long* m = a.mask + static_cast<size_t>(tid) * W;
    int32_t* wp = a.wpre + static_cast<size_t>(tid) * W;
    for (int w = 0; w < W; ++w) {
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
    s_off[tid] = p0;
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
  __threadfence_block();
  __syncthreads();  // wpre and s_off written
  int32_t* pairs = a.pairs + static_cast<size_t>(layer) * a.Pcap;
  for (int idx = tid; idx < npairs; idx += kScanThreads) {
    const int t = idx / k, j = idx - t * k;
    const int e = a.sel[idx];
    const size_t mw = static_cast<size_t>(e) * W + (t >> 6);
    const int pos = min(s_off[e] + a.wpre[mw] + __popcll(a.mask[mw] & ((1ull << (t & 63)) - 1ull)), npairs - 1);
    const float p = a.selp[idx];
    pairs[pos] = t | (j << 16);
    a.pair_w[pos] = p;
    a.slot_of[idx] = pos;
    const size_t o = static_cast<size_t>(layer) * npairs + idx;  // [L][T][k]
    if (a.in.ids) a.in.ids[o] = e;
    if (a.in.route_w) a.in.route_w[o] = p;
  }
}

// ------------------------------------------------------------------------------------------
// GEMM tiles on v_mfma_i32_16x16x32_i8, one 32-weight block per instruction: A = 16 weight rows'
// 4-bit codes as bytes (even elements of each 8-group, then the odd ones: the digit order), B = one
// digit plane of 16 pair rows; lane l supplies A row / B column l % 16 and elements 8(l/16)..+7, and
// D lane l holds rows 4(l/16)..+3 of column l % 16. Per block and (A, B) tile the three plane
// products combine exactly in int32 (P = P0 + 256 P1 + 65536 P2, with wrapping shifts: the sum
// fits) and fold into fp32 as acc += s * P. The minimum's term sum_b m_b * sum(x)_b / step runs
// on v_mfma_f32_16x16x4f32 into the same accumulators (A = 16 rows' m over 4 blocks, B = the block
// sums; the same D layout), and the row's step multiplies the total at the end.
//
// The 64 pair rows' digits of each 4-block step are gathered into LDS (double-buffered, one
// barrier per step) in [block][plane][group][column][even, odd] order, so the 16 lanes of a group
// read 16 consecutive 8-byte words. Columns past the item's pairs repeat its last pair.
// ------------------------------------------------------------------------------------------
typedef int32_t i32x4v __attribute__((ext_vector_type(4)));

// Stage the digits of blocks kb0..kb0+3 of the 64 source rows into LDS: 96 wave-instructions of a
// 4-byte gather each (word `half` of group q, plane p, block bs of column c), split over 4 waves.
__device__ __forceinline__ void stage_step(const uint32_t* const* rows, int kb0, uint32_t* buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane & 1;  // lane l moves word `half` of column 32 ch + l / 2
#pragma unroll
  for (int n = 0; n < 24; ++n) {
    const int ins = wave * 24 + n;           // 0..95: (bs, p, q, column half)
    const int ch = ins & 1, q = (ins >> 1) & 3, p = (ins >> 3) % 3, bs = (ins >> 3) / 3;
    const uint32_t* src = rows[ch] + static_cast<size_t>(kb0 + bs) * kXqWords + p * 8 + 2 * q + half;
    uint32_t* dst = buf + ((((bs * 3 + p) * 4 + q) * kTile) + 32 * ch) * 2;
    __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void*)src, (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
  }
}

// Combine the three plane products of one D element and fold it with the row's block scale.
__device__ __forceinline__ float fold3(int p0, int p1, int p2, float s, float acc) {
  const uint32_t v = static_cast<uint32_t>(p0) + (static_cast<uint32_t>(p1) << 8) + (static_cast<uint32_t>(p2) << 16);
  return fmaf(s, static_cast<float>(static_cast<int32_t>(v)), acc);
}

// Byte codes of one 32-bit code word (8 weights) in the digit order.
__device__ __forceinline__ long codes8(uint32_t w) {
  const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
  return static_cast<long>(static_cast<uint64_t>(ev) | (static_cast<uint64_t>(od) << 32));
}

// 4x4 transpose of dwords across the four 16-lane groups: before, group g holds words 0..3 of
// block g; after, group g holds word g of blocks 0..3.
__device__ __forceinline__ void transpose4(uint4& v) {
  permlane32_swap(v.x, v.z);
  permlane32_swap(v.y, v.w);
  permlane16_swap(v.x, v.y);
  permlane16_swap(v.z, v.w);
}

// Work unit of GEMM block `bid` of `nb` (a multiple of 8): consecutive units (the tiles of one
// work item) go to one XCD, whose L2 then holds that item's digit rows once.
__device__ __forceinline__ int xcd_unit(int bid, int nb) { return (bid & 7) * (nb >> 3) + (bid >> 3); }

// One wave's 16 consecutive weight rows of NM matrices against the 64 staged columns. codes0 /
// sm0: the code and scale/min rows of the wave's first row in each matrix. acc[m][c4][i]: D row
// 4(l/16)+i (weight row), column 16 c4 + l % 16 (pair), in units of the column's step. Each
// pipeline step also stages the next step's digits.
template <int NM>
__device__ __forceinline__ void gemm_rows(const uint8_t* const* codes0, const uint32_t* const* sm0, int K,
                                          const uint32_t* const* src_rows, const float* const* xs_rows,
                                          uint32_t* lds, f32x4 (&acc)[NM][4]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int nblk = K / 32, nstep = nblk / kStepBlocks;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) acc[m][c4] = f32x4{0.f, 0.f, 0.f, 0.f};
  stage_step(src_rows, 0, lds);
  __syncthreads();
  for (int st = 0; st < nstep; ++st) {
    const int kb0 = st * kStepBlocks;
    uint32_t* cur = lds + (st & 1) * kStageWords;
    if (st + 1 < nstep) stage_step(src_rows, kb0 + kStepBlocks, lds + ((st + 1) & 1) * kStageWords);
    // A: lane (r, q) loads block kb0 + q of row r; after the transpose it holds word q of blocks
    // kb0..kb0+3. Scales of the D rows 4q..4q+3 for the 4 blocks; the minimum of (row r, block q).
    uint4 cw[NM];
    float s[NM][kStepBlocks][4];
    float mq[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      cw[m] = load_stream_u4(codes0[m] + static_cast<size_t>(r) * (K / 2) + 16 * (kb0 + q));
      mq[m] = half_bits_to_float(load_stream_u32(sm0[m] + static_cast<size_t>(r) * nblk + kb0 + q) >> 16);
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(sm0[m] + static_cast<size_t>(4 * q + i) * nblk + kb0);
        s[m][0][i] = half_bits_to_float(w4.x);
        s[m][1][i] = half_bits_to_float(w4.y);
        s[m][2][i] = half_bits_to_float(w4.z);
        s[m][3][i] = half_bits_to_float(w4.w);
      }
      transpose4(cw[m]);
    }
    // The minimum's term of the 4 blocks, into the accumulators.
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const float xs = xs_rows[c4][kb0 + q];
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m][c4] = __builtin_amdgcn_mfma_f32_16x16x4f32(mq[m], xs, acc[m][c4], 0, 0, 0);
    }
#pragma unroll
    for (int bs = 0; bs < kStepBlocks; ++bs) {
      long a8[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint32_t word = bs == 0 ? cw[m].x : bs == 1 ? cw[m].y : bs == 2 ? cw[m].z : cw[m].w;
        a8[m] = codes8(word);
      }
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        long b8[3];
#pragma unroll
        for (int p = 0; p < 3; ++p)
          b8[p] = *reinterpret_cast<const long*>(cur + ((((bs * 3 + p) * 4 + q) * kTile) + 16 * c4 + r) * 2);
        const i32x4v z = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const i32x4v d0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a8[m], b8[0], z, 0, 0, 0);
          const i32x4v d1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a8[m], b8[1], z, 0, 0, 0);
          const i32x4v d2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a8[m], b8[2], z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][c4][i] = fold3(d0[i], d1[i], d2[i], s[m][bs][i], acc[m][c4][i]);
        }
      }
    }
    __syncthreads();  // step st read by every wave; step st + 1 staged
  }
}

// Gate/up: work unit = (item, 64 rows of I). Wave w takes rows i0 + 16w .. +15 of both gate and
// up, and writes silu(g) * v of its rows for the item's pairs into hbuf (by pair slot).
static __global__ __launch_bounds__(kThreads) void pf_gateup_kernel(PfArgs a, int layer) {
  extern __shared__ uint32_t lds[];
  const int I = a.I, H = a.H;
  const int tiles = I / kTile;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int it = unit / tiles, i0 = (unit - it * tiles) * kTile;
  if (it >= *a.n_items) return;  // whole blocks leave together
  const int4 item = a.items[it];
  const int e = item.x, p0 = item.y, np = item.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 15, q = lane >> 4;
  const int32_t* pairs = a.pairs + static_cast<size_t>(layer) * a.Pcap;
  // Source rows of the staged columns: the staging lanes need columns lane / 2 and 32 + lane / 2;
  // the accumulation lanes need the block sums of columns 16 c4 + r.
  const uint32_t* src[2];
#pragma unroll
  for (int ch = 0; ch < 2; ++ch) {
    const int t = pairs[p0 + min(32 * ch + (lane >> 1), np - 1)] & 0xFFFF;
    src[ch] = a.xq + static_cast<size_t>(t) * (H / 32) * kXqWords;
  }
  const float* xs[4];
  int tcol[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) {
    tcol[c4] = pairs[p0 + min(16 * c4 + r, np - 1)] & 0xFFFF;
    xs[c4] = a.xsum + static_cast<size_t>(tcol[c4]) * (H / 32);
  }
  const size_t row = static_cast<size_t>(e) * I + i0 + 16 * wave;  // the wave's first row
  const uint8_t* codes[2] = {a.w.gate_q + row * (H / 2), a.w.up_q + row * (H / 2)};
  const uint32_t* sm[2] = {a.w.gate_sm + row * (H / 32), a.w.up_sm + row * (H / 32)};
  f32x4 acc[2][4];
  gemm_rows<2>(codes, sm, H, src, xs, lds, acc);
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) {
    const int c = 16 * c4 + r;
    const float step = a.xstep[tcol[c4]];
    float4 h;
    h.x = silu(step * acc[0][c4][0]) * (step * acc[1][c4][0]);
    h.y = silu(step * acc[0][c4][1]) * (step * acc[1][c4][1]);
    h.z = silu(step * acc[0][c4][2]) * (step * acc[1][c4][2]);
    h.w = silu(step * acc[0][c4][3]) * (step * acc[1][c4][3]);
    if (c < np)
      *reinterpret_cast<float4*>(a.hbuf + static_cast<size_t>(p0 + c) * I + i0 + 16 * wave + 4 * q) = h;
  }
}

// Down: work unit = (item, 64 rows of H). Wave w takes rows h0 + 16w .. +15 of W_d and writes
// W_d h of its rows for the item's pairs into ybuf (by pair slot).
static __global__ __launch_bounds__(kThreads) void pf_down_kernel(PfArgs a, int layer) {
  extern __shared__ uint32_t lds[];
  const int I = a.I, H = a.H;
  const int tiles = H / kTile;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int it = unit / tiles, h0 = (unit - it * tiles) * kTile;
  if (it >= *a.n_items) return;
  const int4 item = a.items[it];
  const int e = item.x, p0 = item.y, np = item.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 15, q = lane >> 4;
  const uint32_t* src[2];
#pragma unroll
  for (int ch = 0; ch < 2; ++ch)
    src[ch] = a.hq + static_cast<size_t>(p0 + min(32 * ch + (lane >> 1), np - 1)) * (I / 32) * kXqWords;
  const float* xs[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) xs[c4] = a.hsum + static_cast<size_t>(p0 + min(16 * c4 + r, np - 1)) * (I / 32);
  const size_t row = static_cast<size_t>(e) * H + h0 + 16 * wave;  // the wave's first row
  const uint8_t* codes[1] = {a.w.down_q + row * (I / 2)};
  const uint32_t* sm[1] = {a.w.down_sm + row * (I / 32)};
  f32x4 acc[1][4];
  gemm_rows<1>(codes, sm, I, src, xs, lds, acc);
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) {
    const int c = 16 * c4 + r;
    const float step = a.hstep[p0 + min(c, np - 1)];
    const float4 y = make_float4(step * acc[0][c4][0], step * acc[0][c4][1], step * acc[0][c4][2], step * acc[0][c4][3]);
    if (c < np) *reinterpret_cast<float4*>(a.ybuf + static_cast<size_t>(p0 + c) * H + h0 + 16 * wave + 4 * q) = y;
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
