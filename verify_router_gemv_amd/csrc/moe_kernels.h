// Device code of the MoE decode/verify round (gfx950, wave64). Included once, by moe_round.hip.
//
// Per layer four kernels:
//   logits_kernel  router GEMV z[t][e] = sum_h Wr[e][h] x[t][h] + b[e]: fp32 inputs, fp64 products
//                  and sums; also seeds the layer's output rows (residual x, or zeros).
//   select_kernel  one block: per-row top-k (k rounds of a wave-wide max over (logit, id) keys),
//                  softmax over the k selected logits, the union of the rows' experts and a counting
//                  sort of the (row, rank) pairs by expert; it writes one 128-byte record per unique
//                  expert (id, pair offset, row count, unique count, packed row ids).
//   gateup_kernel  streams one unique expert's 4-bit gate and up rows once for all rows routed to
//                  it, dequantising in registers, and writes silu(g) * v per (row, rank) pair.
//   down_kernel    streams the unique experts' 4-bit down rows and scatter-adds routing weight x
//                  (W_d h) into the output rows.
// Everything a GEMV block needs before its weight stream is in its expert's record, so it waits
// for one dependent global round trip; every other load is issued up front, never inside a loop
// whose trip count depends on the data (such loops serialise memory latency).
//
// Page references: "How AlphaInfer makes local decoding fast" section 2 (a decode round is one
// forward pass over 1-8 rows, replayed as a captured graph, per-request data is ingress) and
// section 3.1 (extra verified rows add the bytes of experts only they chose, so the union is read
// once); infero README "Beyond plain text decode" (top-k routing at decode, counting sort into
// per-expert work), "Layout" figure (the SwiGLU expert), "Design notes" (block weights consumed
// in place; a float GEMV decoding one weight per thread runs far below the memory bound, so each
// lane here decodes 32-weight blocks from 16-byte loads).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_round.h"

namespace moe {

constexpr int kThreads = 256;   // 4 waves per block
constexpr int kWaves = kThreads / 64;
constexpr int kSelectThreads = 1024;  // the select kernel's single block: 16 waves, one row each
constexpr int kSelectWaves = kSelectThreads / 64;

// Per-unique-expert record: [0] expert id, [1] first pair slot, [2] rows routed to the expert,
// [3] number of unique experts of the layer, [4..19] the rows' ids, one byte each, in slot order.
constexpr int kRecWords = 32;
constexpr int kRecRowWord = 4;
// A 32-block of activations as three signed int8 digits of a 24-bit integer: x ~ step * (d2*65536 +
// d1*256 + d0). Words [digit d][group g of 8][even/odd]: the even word packs elements 8g+0,2,4,6, the
// odd word 8g+1,3,5,7, matching the nibble order of a weight code word.
constexpr int kXqWords = 24;
constexpr float kXqMax = 8355711.0f;  // 127*65536 + 127*256 + 127
constexpr int kXStageMax = 8;        // activation rows staged in LDS at a time (T > 1) ...
constexpr int kXStageBytes = 65536;  // ... within 64 KB of LDS

// Per-run pointers. Eager launches carry them by value; graph replays read them from a fixed
// device copy (written when they change), so a captured graph is never rebuilt.
struct Ingress {
  const float* hidden;  // [T][H]
  float* out;           // [T][H]
  int32_t* ids;         // [L][T][k] or null
  float* route_w;       // [L][T][k] or null
};

struct Args {
  const Ingress* ing;              // graph mode: device ingress; eager mode: null
  Ingress in;                      // eager mode ingress
  const moe_layer_weights* wtab;   // graph mode: device table [L]; eager mode: null
  moe_layer_weights w;             // eager mode: this layer's weights
  float* xbuf0;
  float* xbuf1;
  double* logits;     // [T_max][E]
  int32_t* n_unique;  // [L]
  int32_t* uniq;      // [L][Ucap]
  int32_t* offs;      // [L][Ucap + 1]
  int32_t* pairs;     // [L][Pcap]  t | (j << 8)
  float* pair_w;      // [L][Pcap]
  int32_t* rec;       // [L][Ucap][kRecWords] per-unique-expert records
  float* hbuf;        // [Pcap][I]
  uint32_t* xq;       // [T_max][H/32][kXqWords] int8 digits of the layer input, per 32-block
  float2* xss;        // [T_max][H/32] (digit step, block sum) of the layer input
  int32_t H, I, E, L, T, k, residual, Ucap, Pcap;
  int32_t xstage_h, xstage_i;  // activation rows staged in LDS at a time (gate/up: rows of H, down: of I)
};

__device__ __forceinline__ Ingress get_ingress(const Args& a) { return a.ing ? *a.ing : a.in; }
__device__ __forceinline__ moe_layer_weights get_weights(const Args& a, int layer) {
  return a.wtab ? a.wtab[layer] : a.w;
}
__device__ __forceinline__ const float* layer_input(const Args& a, const Ingress& in, int layer) {
  if (layer == 0) return in.hidden;
  return ((layer - 1) & 1) ? a.xbuf1 : a.xbuf0;
}
__device__ __forceinline__ float* layer_output(const Args& a, const Ingress& in, int layer) {
  if (layer == a.L - 1) return in.out;
  return (layer & 1) ? a.xbuf1 : a.xbuf0;
}

// ------------------------------------------------------------------------------------------
// Cross-lane reductions on VALU only: DPP inside 16-lane rows, gfx950 permlane swaps across rows.
// ------------------------------------------------------------------------------------------

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp_u32<CTRL>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  return __builtin_bit_cast(double, dpp_u64<CTRL>(__builtin_bit_cast(uint64_t, v)));
}

// gfx950 lane swaps, written as inline asm: the compiler's two-result builtins for these were
// observed to wire both results to one register when the inputs differ (sum s[0] + s[1] compiled
// to s[0] + s[0]). Both operands are read and written: v_permlane32_swap exchanges lanes 32-63 of
// `a` with lanes 0-31 of `b`; v_permlane16_swap exchanges the odd 16-lane rows of `a` with the
// even rows of `b`. The s_nop covers the VALU-write -> swap-read hazard.
__device__ __forceinline__ void permlane32_swap(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Exchange with the lane 16 (X16) or 32 (X32) apart: returns the partner's value.
template <bool X32>
__device__ __forceinline__ uint32_t swap_partner_u32(uint32_t v) {
  uint32_t a = v, b = v;
  if constexpr (X32) {
    permlane32_swap(a, b);  // a: [lo half, lo half], b: [hi half, hi half]
    return (__lane_id() < 32) ? b : a;
  } else {
    permlane16_swap(a, b);  // a: rows [r0, r0, r2, r2], b: rows [r1, r1, r3, r3]
    return ((__lane_id() >> 4) & 1) ? a : b;
  }
}
template <bool X32>
__device__ __forceinline__ float swap_partner_f32(float v) {
  return __builtin_bit_cast(float, swap_partner_u32<X32>(__builtin_bit_cast(uint32_t, v)));
}
template <bool X32>
__device__ __forceinline__ uint64_t swap_partner_u64(uint64_t v) {
  const uint32_t lo = swap_partner_u32<X32>(static_cast<uint32_t>(v));
  const uint32_t hi = swap_partner_u32<X32>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
template <bool X32>
__device__ __forceinline__ double swap_partner_f64(double v) {
  return __builtin_bit_cast(double, swap_partner_u64<X32>(__builtin_bit_cast(uint64_t, v)));
}

// Sum over groups of G consecutive lanes (G a power of two <= 64); every lane gets its group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_f32<kDppXor1>(v);
  if constexpr (G >= 4) v += dpp_f32<kDppXor2>(v);
  if constexpr (G >= 8) v += dpp_f32<kDppHalfMirror>(v);
  if constexpr (G >= 16) v += dpp_f32<kDppMirror>(v);
  if constexpr (G >= 32) v += swap_partner_f32<false>(v);
  if constexpr (G >= 64) v += swap_partner_f32<true>(v);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  v += swap_partner_f64<false>(v);
  v += swap_partner_f64<true>(v);
  return v;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp_u64<kDppXor1>(v));
  v = umax64(v, dpp_u64<kDppXor2>(v));
  v = umax64(v, dpp_u64<kDppHalfMirror>(v));
  v = umax64(v, dpp_u64<kDppMirror>(v));
  v = umax64(v, swap_partner_u64<false>(v));
  v = umax64(v, swap_partner_u64<true>(v));
  return v;
}

// Full sums over 64 lanes of 8 values at once (a transposed butterfly): the xor-32 and xor-16
// levels pair values through the permlane swaps, so each level halves the registers instead of
// repeating per value; the last four levels run inside 16-lane rows. Afterwards every lane of row
// R (lanes 16R..16R+15) holds in `lo` the total of v[{0,2,1,3}[R]] and in `hi` of v[{4,6,5,7}[R]].
__device__ __forceinline__ float pair_sum32(float a, float b) {
  uint32_t x = __builtin_bit_cast(uint32_t, a), y = __builtin_bit_cast(uint32_t, b);
  permlane32_swap(x, y);  // x: [a lo, b lo], y: [a hi, b hi]
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float pair_sum16(float a, float b) {
  uint32_t x = __builtin_bit_cast(uint32_t, a), y = __builtin_bit_cast(uint32_t, b);
  permlane16_swap(x, y);  // x: rows [a0, b0, a2, b2], y: rows [a1, b1, a3, b3]
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ void reduce8_wave(const float v[8], float& lo, float& hi) {
  const float s01 = pair_sum32(v[0], v[1]), s23 = pair_sum32(v[2], v[3]);
  const float s45 = pair_sum32(v[4], v[5]), s67 = pair_sum32(v[6], v[7]);
  lo = group_sum<16>(pair_sum16(s01, s23));
  hi = group_sum<16>(pair_sum16(s45, s67));
}
__device__ __forceinline__ int reduce8_slot(int row) { return (row == 1) ? 2 : (row == 2 ? 1 : row); }

// ------------------------------------------------------------------------------------------
// Small helpers
// ------------------------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define MOE_GLOBAL __attribute__((address_space(1)))

// Streaming (non-temporal) loads through global (not flat) addressing: weights are read once per
// round; keep them from evicting the small reused data (activations, logits, records).
// Every load in the kernels below is unconditional with a clamped, in-bounds address: a load under
// a divergent branch is followed by its own wait, which would serialise the memory latency.
__device__ __forceinline__ uint4 load_stream_u4(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const MOE_GLOBAL u32x4*)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t load_stream_u32(const uint32_t* p) {
  return __builtin_nontemporal_load((const MOE_GLOBAL uint32_t*)(p));
}
__device__ __forceinline__ float4 load_stream_f4(const void* p) {
  const f32x4 v = __builtin_nontemporal_load((const MOE_GLOBAL f32x4*)(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load_f4(const void* p) {
  const f32x4 v = *((const MOE_GLOBAL f32x4*)(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xFFFFu)));
}

// Single-instruction byte -> float conversions (v_cvt_f32_ubyte0..3).
#define MOE_CVT_UBYTE(N)                                                            \
  __device__ __forceinline__ float cvt_ubyte##N(uint32_t v) {                       \
    float r;                                                                        \
    asm("v_cvt_f32_ubyte" #N " %0, %1" : "=v"(r) : "v"(v));                         \
    return r;                                                                       \
  }
MOE_CVT_UBYTE(0)
MOE_CVT_UBYTE(1)
MOE_CVT_UBYTE(2)
MOE_CVT_UBYTE(3)
#undef MOE_CVT_UBYTE

// 32 codes of one block (16 bytes, byte j = element 2j | element 2j+1 << 4) -> floats in order,
// 11 VALU instructions per 8 codes.
__device__ __forceinline__ void unpack_block(const uint4 c, float q[32]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = w[i] & 0x0F0F0F0Fu;         // elements 8i+0, +2, +4, +6
    const uint32_t hi = (w[i] >> 4) & 0x0F0F0F0Fu;  // elements 8i+1, +3, +5, +7
    q[8 * i + 0] = cvt_ubyte0(lo);
    q[8 * i + 1] = cvt_ubyte0(hi);
    q[8 * i + 2] = cvt_ubyte1(lo);
    q[8 * i + 3] = cvt_ubyte1(hi);
    q[8 * i + 4] = cvt_ubyte2(lo);
    q[8 * i + 5] = cvt_ubyte2(hi);
    q[8 * i + 6] = cvt_ubyte3(lo);
    q[8 * i + 7] = cvt_ubyte3(hi);
  }
}

__device__ __forceinline__ float dot32(const float q[32], const float x[32]) {
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    d0 = fmaf(q[i], x[i], d0);
    d1 = fmaf(q[i + 1], x[i + 1], d1);
  }
  return d0 + d1;
}

// Make a value opaque to the optimiser so per-pass unpacking is not hoisted out of the pass loop
// (hoisting keeps every unpacked code live across the loop and multiplies register use).
__device__ __forceinline__ void opaque(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Order-preserving 64-bit key of a logit with the expert id in the low 9 bits, so one unsigned
// max picks the largest logit and, among logits equal to 2^-43 relative, the lower id.
__device__ __forceinline__ uint64_t logit_key(double z, int e) {
  if (!(z == z)) z = -INFINITY;  // NaN ranks lowest
  uint64_t b = __builtin_bit_cast(uint64_t, z);
  b = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return (b & ~0x1FFull) | static_cast<uint64_t>(511 - e);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return 511 - static_cast<int>(key & 0x1FFull); }


// Digits of one 32-block (see kXqWords). The integer q = rint(x / step) with step = max|x| / kXqMax
// is split into balanced base-256 digits d0, d1, d2 in [-127, 127]; the block sum is kept in fp32.
__device__ __forceinline__ void quantize_block(const float* src, uint32_t* dst, float2* ss) {
  float v[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 f = load_f4(src + 4 * q);
    v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
  }
  float mx = 0.f, sum = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) { mx = fmaxf(mx, fabsf(v[i])); sum += v[i]; }
  const float inv = mx > 0.f ? kXqMax / mx : 0.f;
  uint32_t d[3][8];  // digit planes, 4 bytes per word in element order 0..31
#pragma unroll
  for (int w = 0; w < 8; ++w) { d[0][w] = 0u; d[1][w] = 0u; d[2][w] = 0u; }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int q = static_cast<int>(rintf(v[i] * inv));
    q = max(-static_cast<int>(kXqMax), min(static_cast<int>(kXqMax), q));
    const int d0 = ((q + 128) & 255) - 128;
    const int q1 = (q - d0) >> 8;
    const int d1 = ((q1 + 128) & 255) - 128;
    const int d2 = (q1 - d1) >> 8;
    const int w = i >> 2, sh = 8 * (i & 3);
    d[0][w] |= (static_cast<uint32_t>(d0) & 0xFFu) << sh;
    d[1][w] |= (static_cast<uint32_t>(d1) & 0xFFu) << sh;
    d[2][w] |= (static_cast<uint32_t>(d2) & 0xFFu) << sh;
  }
  // regroup each 8-element group into even (0,2,4,6) and odd (1,3,5,7) words
#pragma unroll
  for (int dg = 0; dg < 3; ++dg)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t a0 = d[dg][2 * g], a1 = d[dg][2 * g + 1];  // bytes of elements 8g..8g+3, 8g+4..8g+7
      const uint32_t even = __builtin_amdgcn_perm(a1, a0, 0x06040200u);  // bytes e0 e2 | e4 e6
      const uint32_t odd = __builtin_amdgcn_perm(a1, a0, 0x07050301u);   // bytes e1 e3 | e5 e7
      dst[(dg * 4 + g) * 2 + 0] = even;
      dst[(dg * 4 + g) * 2 + 1] = odd;
    }
  *ss = make_float2(mx / kXqMax, sum);
}

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

// ------------------------------------------------------------------------------------------
// Kernels 3 and 4: dequant-GEMV tiles
// ------------------------------------------------------------------------------------------
//
// Lane layout: G lanes share one weight row, each owning NB of its 32-weight blocks (block
// b = g + nb*G); a wave covers 64/G rows per load and RW such row groups (for gate/up: of both
// matrices). Codes (16 B) and the scale/min word (4 B) of each block are loaded once into
// registers. The activation rows routed to the expert are processed RC at a time from registers:
// for T == 1 loaded directly, otherwise staged kXStage rows at a time in LDS. Per block the dot
// product is s * sum(q*x) + m * sum(x).

// Load RC activation rows' segments for this lane, from LDS rows (FROM_LDS) or global rows.
template <int NB, int RC, int G, bool FROM_LDS>
__device__ __forceinline__ void load_x(const float* src, int row_stride, const int* row_of, int nlive, int g,
                                       float xv[RC][NB][32], float xs[RC][NB]) {
#pragma unroll
  for (int r = 0; r < RC; ++r) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const size_t off = static_cast<size_t>(row_of[r]) * row_stride + 32 * (g + nb * G);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float4 v;
        if constexpr (FROM_LDS) {
          const f32x4 t = *((const __attribute__((address_space(3))) f32x4*)(src + off) + q);
          v = make_float4(t.x, t.y, t.z, t.w);
        } else {
          v = load_f4(src + off + 4 * q);  // row_of[] is always a valid row
        }
        xv[r][nb][4 * q + 0] = v.x;
        xv[r][nb][4 * q + 1] = v.y;
        xv[r][nb][4 * q + 2] = v.z;
        xv[r][nb][4 * q + 3] = v.w;
      }
    }
  }
  // zero the rows past the live count after every load has been issued
#pragma unroll
  for (int r = 0; r < RC; ++r) {
    const bool live = r < nlive;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        xv[r][nb][q] = live ? xv[r][nb][q] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 32; q += 4) sum += (xv[r][nb][q] + xv[r][nb][q + 1]) + (xv[r][nb][q + 2] + xv[r][nb][q + 3]);
      xs[r][nb] = sum;
    }
  }
}

template <int NB, int RC>
__device__ __forceinline__ void block_dots(const uint4 c[NB], const uint32_t sm[NB], const float xv[RC][NB][32],
                                           const float xs[RC][NB], float acc[RC]) {
#pragma unroll
  for (int r = 0; r < RC; ++r) acc[r] = 0.f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float q[32];
    unpack_block(c[nb], q);
    const float sc = half_bits_to_float(sm[nb]), mn = half_bits_to_float(sm[nb] >> 16);
#pragma unroll
    for (int r = 0; r < RC; ++r) acc[r] = fmaf(mn, xs[r][nb], fmaf(sc, dot32(q, xv[r][nb]), acc[r]));
  }
}

// Cooperative copy of up to `n` rows (row ids from `rowid(r)`) of length K into LDS.
template <typename RowFn>
__device__ __forceinline__ void stage_rows(float* lds, const float* src, int K, int n, RowFn rowid) {
  const int k4 = K / 4;
  float4* d4 = reinterpret_cast<float4*>(lds);
  for (int idx = threadIdx.x; idx < n * k4; idx += kThreads) {
    const int r = idx / k4, c4 = idx - r * k4;
    d4[idx] = reinterpret_cast<const float4*>(src + static_cast<size_t>(rowid(r)) * K)[c4];
  }
}

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

// ------------------------------------------------------------------------------------------
// Kernel selection
// ------------------------------------------------------------------------------------------

using KernelFn = void (*)(Args, int);

constexpr int rows_per_lane_group(int NB) { return NB == 1 ? 4 : (NB == 2 ? 2 : 1); }

template <int G, int NB, int RC>
struct GemvPick {
  static constexpr int RW = rows_per_lane_group(NB);
  static KernelFn gateup() { return gateup_kernel<G, NB, RW>; }
  static KernelFn down() { return down_kernel<G, NB, RC, RW>; }
  static constexpr int rows_per_block() { return kWaves * RW * (64 / G); }
};

template <int G, int NB>
inline bool pick_rc(int RC, bool up, KernelFn* fn, int* rows) {
  if (up) {  // gate/up walks the expert's rows one at a time; no pass width
    *fn = GemvPick<G, NB, 1>::gateup();
    *rows = GemvPick<G, NB, 1>::rows_per_block();
    return true;
  }
  switch (RC) {
#define MOE_RC(R)                                 \
  case R:                                         \
    *fn = GemvPick<G, NB, R>::down();             \
    *rows = GemvPick<G, NB, R>::rows_per_block(); \
    return true;
    MOE_RC(1) MOE_RC(2) MOE_RC(4)
#undef MOE_RC
  }
  return false;
}

template <int G>
inline bool pick_nb(int NB, int RC, bool up, KernelFn* fn, int* rows) {
  switch (NB) {
    case 1: return pick_rc<G, 1>(RC, up, fn, rows);
    case 2: return pick_rc<G, 2>(RC, up, fn, rows);
    case 3: return pick_rc<G, 3>(RC, up, fn, rows);
    case 4: return pick_rc<G, 4>(RC, up, fn, rows);
  }
  return false;
}

// Each lane split G is instantiated in its own translation unit (moe_gemv_g<G>.hip) so the
// library builds in parallel.
bool pick_gemv_g4(int NB, int RC, bool up, KernelFn* fn, int* rows);
bool pick_gemv_g8(int NB, int RC, bool up, KernelFn* fn, int* rows);
bool pick_gemv_g16(int NB, int RC, bool up, KernelFn* fn, int* rows);
bool pick_gemv_g32(int NB, int RC, bool up, KernelFn* fn, int* rows);
bool pick_gemv_g64(int NB, int RC, bool up, KernelFn* fn, int* rows);

inline bool pick_gemv(int G, int NB, int RC, bool up, KernelFn* fn, int* rows) {
  switch (G) {
    case 4: return pick_gemv_g4(NB, RC, up, fn, rows);
    case 8: return pick_gemv_g8(NB, RC, up, fn, rows);
    case 16: return pick_gemv_g16(NB, RC, up, fn, rows);
    case 32: return pick_gemv_g32(NB, RC, up, fn, rows);
    case 64: return pick_gemv_g64(NB, RC, up, fn, rows);
  }
  return false;
}

// Router rows per wave: one at T == 1, two otherwise.
inline int logits_rows(int T) { return T == 1 ? 1 : 2; }

template <int TC>
inline KernelFn pick_logits_tc(int H) {
  switch (H / 256) {
#define MOE_NJ(N) \
  case N: return logits_kernel<N, TC>;
    MOE_NJ(1) MOE_NJ(2) MOE_NJ(3) MOE_NJ(4) MOE_NJ(6) MOE_NJ(8) MOE_NJ(12) MOE_NJ(16) MOE_NJ(24) MOE_NJ(32)
#undef MOE_NJ
  }
  return nullptr;
}

inline KernelFn pick_logits(int H, int T) { return logits_rows(T) == 1 ? pick_logits_tc<1>(H) : pick_logits_tc<2>(H); }

inline KernelFn pick_select(int E) {
  if (E <= 64) return select_kernel<1>;
  if (E <= 128) return select_kernel<2>;
  if (E <= 256) return select_kernel<4>;
  return select_kernel<8>;
}

// Rows of one expert processed per register pass, by round width.
inline int rows_per_pass(int T) { return T == 1 ? 1 : 2; }

}  // namespace moe
