// Device code of the MoE decode/verify round (gfx950, wave64): shared definitions.
//
// Per layer four kernels:
//   logits_kernel  router GEMV z[t][e] = sum_h Wr[e][h] x[t][h] + b[e]: fp32 inputs, fp64 products
//                  and sums; its extra blocks write the input's int8 digits and seed the output rows
//                  with the residual (the gate/up kernel zeroes them when there is none).
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

#include "moe_round.h"

namespace moe {

constexpr int kThreads = 256;   // 4 waves per block
constexpr int kWaves = kThreads / 64;
constexpr int kSelectThreads = 1024;  // the select kernel's single block: 16 waves, one row each
constexpr int kSelectWaves = kSelectThreads / 64;

// Per-work-item record (an item is one expert and up to rg of its rows): [0] expert id, [1] first
// pair slot, [2] rows of the item, [3] number of items of the layer, [4..19] the rows' ids, one byte
// each, in slot order.
constexpr int kRecWords = 32;
constexpr int kRecRowWord = 4;
// A 32-block of activations as three signed int8 digits of a 24-bit integer: x ~ step * (d2*65536 +
// d1*256 + d0). Words [digit d][group g of 8][even/odd]: the even word packs elements 8g+0,2,4,6, the
// odd word 8g+1,3,5,7, matching the nibble order of a weight code word.
constexpr int kXqWords = 24;
// Rounds of at least this many rows are "wide": gate/up stages the input digits in LDS, and both
// GEMVs may use their matrix-core tiles.
constexpr int kWideRows = 16;
constexpr float kXqMax = 8355711.0f;  // 127*65536 + 127*256 + 127
constexpr int kXStageMax = 8;        // SwiGLU rows the down kernel stages in LDS as digits at a time ...
constexpr int kXStageBytes = 65536;  // ... within 64 KB of LDS

// Per-run pointers. Eager launches carry them by value; graph replays read them from a fixed
// device copy (written when they change), so a captured graph is never rebuilt for a new request.
struct Ingress {
  const float* hidden;  // [T][H]
  float* out;           // [T][H]
  int32_t* ids;         // [L][T][k] or null
  float* route_w;       // [L][T][k] or null
};

struct Args {
  const Ingress* ing;              // graph mode: device ingress; eager mode: null
  Ingress in;                      // eager mode ingress
  moe_layer_weights w;             // this layer's weights (a graph node's parameters in graph mode)
  float* xall;        // layer outputs before the last: slot s at xall + s * xstride
  int32_t xslots;     // 2 (slots reused alternately) or L - 1 (every layer's input kept)
  int32_t xstride;    // floats per slot (T_max * H)
  double* logits;     // [T_max][E]
  int32_t* n_unique;  // [L]
  int32_t* uniq;      // [L][Ucap]
  int32_t* offs;      // [L][Ucap + 1]
  int32_t* pairs;     // [L][Pcap]  t | (j << 8)
  float* pair_w;      // [L][Pcap]
  int32_t* rec;       // [L][Icap][kRecWords] per-work-item records
  float* hbuf;        // [Pcap][I]
  float* ybuf;        // exact mode: [Pcap][H] down products W_d h per pair slot
  int32_t* slot_of;   // [L][Pcap] pair slot of (row t, rank j) at t * k + j
  int32_t* tsel;      // [Pcap] wide rounds: expert ids by (row, rank) from the top-k kernel
  float* tp;          // [Pcap] and their routing weights
  uint32_t* xq;       // [T_max][H/32][kXqWords] int8 digits of the layer input, per 32-block
  float2* xss;        // [T_max][H/32] (digit step, block sum) of the layer input
  int32_t H, I, E, L, T, k, residual, Ucap, Pcap;
  int32_t Icap;       // record slots per layer (work items <= pairs)
  int32_t rg;         // rows per work item at most (this launch)
  int32_t xstage_h;  // gate/up: rows of input digits staged in LDS at a time (T > 1)
  int32_t xstage_i;  // down: SwiGLU rows staged in LDS (as digits) at a time
  int32_t mfma_rows;  // gate/up: experts with at least this many rows use the matrix-core tile (0: never)
  int32_t exact;      // fixed-order combine (the logits kernel does not seed the output)
  int32_t prefetch;   // touch the next kernel's weight lines (see touch_lines)
  const float* router_next;  // the next layer's router matrix (null on the last layer)
  const moe_expert_ref* etab;  // table mode: this layer's [E] expert pointers (null: the w arrays)
  const uint32_t* resident;    // tail skip: this layer's residency bits [ceil(E/32)] (null: off)
  int32_t skip_j;              // tail skip: 0-based rank from which a missed expert's pair is a tail pair
  int32_t* n_skipped;          // [L] experts the tail skip left out
};

// Words of device memory that no kernel writes while they are read (changed only between kernels,
// in stream order), through the constant address space: scalar loads, whose wait is not the
// vector-memory counter's, so no vector load waits for them (nor they for a vector load).
template <int N>
__device__ __forceinline__ void load_const_words(const void* p, uint64_t (&w)[N]) {
  const __attribute__((address_space(4))) uint64_t* q = (const __attribute__((address_space(4))) uint64_t*)(p);
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] = q[i];
}

// The ingress pointers (graph mode: from the device buffer, by scalar loads).
__device__ __forceinline__ Ingress get_ingress(const Args& a) {
  if (!a.ing) return a.in;
  uint64_t w[4];
  load_const_words(a.ing, w);
  Ingress in;
  in.hidden = reinterpret_cast<const float*>(w[0]);
  in.out = reinterpret_cast<float*>(w[1]);
  in.ids = reinterpret_cast<int32_t*>(w[2]);
  in.route_w = reinterpret_cast<float*>(w[3]);
  return in;
}
// A layer's weight pointers are always kernel arguments (so every weight address is known without a
// load); graph replays pick up new weights through their nodes' parameters, not a device table.
__device__ __forceinline__ const moe_layer_weights& get_weights(const Args& a, int) { return a.w; }
__device__ __forceinline__ const float* layer_input(const Args& a, const Ingress& in, int layer) {
  if (layer == 0) return in.hidden;
  return a.xall + static_cast<size_t>((layer - 1) % a.xslots) * a.xstride;
}
__device__ __forceinline__ float* layer_output(const Args& a, const Ingress& in, int layer) {
  if (layer == a.L - 1) return in.out;
  return a.xall + static_cast<size_t>(layer % a.xslots) * a.xstride;
}

// ------------------------------------------------------------------------------------------
// Cross-lane reductions on VALU only: DPP inside 16-lane rows, gfx950 permlane swaps across rows.
// ------------------------------------------------------------------------------------------

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kDppRor8 = 0x128;       // lane i <-> i ^ 8 within 16 (a rotation by 8)

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

// Both 32-bit halves of two fp64 values through one lane swap (X32: lanes 32 apart, else 16).
template <bool X32>
__device__ __forceinline__ void swap_f64(double& a, double& b) {
  const uint64_t ua = __builtin_bit_cast(uint64_t, a), ub = __builtin_bit_cast(uint64_t, b);
  uint32_t al = static_cast<uint32_t>(ua), ah = static_cast<uint32_t>(ua >> 32);
  uint32_t bl = static_cast<uint32_t>(ub), bh = static_cast<uint32_t>(ub >> 32);
  if constexpr (X32) {
    permlane32_swap(al, bl);
    permlane32_swap(ah, bh);
  } else {
    permlane16_swap(al, bl);
    permlane16_swap(ah, bh);
  }
  a = __builtin_bit_cast(double, (static_cast<uint64_t>(ah) << 32) | al);
  b = __builtin_bit_cast(double, (static_cast<uint64_t>(bh) << 32) | bl);
}

// Wave sums of R rows at once (R = 1, 2, 4 or 8 values per lane). The levels over lane bits 5, 4
// and 3 first halve the rows each lane carries: lanes with the bit clear keep the lower half of
// their rows, lanes with it set the upper half, and one lane swap (or DPP rotation) hands each lane
// its partner's values for the rows it keeps. Once a lane carries a single row, the remaining
// levels add its partners' copies. Every row goes through the same tree whatever R (partners 32,
// 16 and 8 lanes apart, then lane i with 7 - i within 8, then 2 and 1 apart; fp addition being
// commutative, either operand order gives the same bits), so a row's sum does not depend on the
// rows summed beside it. Lane l returns the sum of row l / (64 / R).
template <int R>
__device__ __forceinline__ double wave_sums_f64(const double (&v)[R]) {
  static_assert(R == 1 || R == 2 || R == 4 || R == 8, "1, 2, 4 or 8 rows");
  constexpr int R1 = R > 1 ? R / 2 : 1, R2 = R1 > 1 ? R1 / 2 : 1;
  double s1[R1], s2[R2];
#pragma unroll
  for (int i = 0; i < R1; ++i) {
    double a = v[i], b = v[R > 1 ? i + R1 : i];
    swap_f64<true>(a, b);  // lanes 0-31: their own a and lane + 32's a; lanes 32-63: the b's
    s1[i] = a + b;
  }
#pragma unroll
  for (int i = 0; i < R2; ++i) {
    double a = s1[i], b = s1[R1 > 1 ? i + R2 : i];
    swap_f64<false>(a, b);  // the same over 16-lane rows: even rows keep a, odd rows b
    s2[i] = a + b;
  }
  double s;
  if constexpr (R2 > 1) {
    const bool up = (__lane_id() & 8) != 0;
    s = (up ? s2[1] : s2[0]) + dpp_f64<kDppRor8>(up ? s2[0] : s2[1]);
  } else {
    s = s2[0] + dpp_f64<kDppRor8>(s2[0]);
  }
  s += dpp_f64<kDppHalfMirror>(s);
  s += dpp_f64<kDppXor2>(s);
  s += dpp_f64<kDppXor1>(s);
  return s;
}

// Wave-wide maximum left in every lane, on VALU only (no round trip through scalar registers):
// DPP inside each 16-lane row, then the two permlane swaps, whose two outputs together hold both
// partners of a level, so the maximum of the pair needs no lane select.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppHalfMirror>(v));
  v = max(v, dpp_u32<kDppMirror>(v));
  uint32_t a = v, b = v;
  permlane16_swap(a, b);  // a: rows [r0, r0, r2, r2], b: rows [r1, r1, r3, r3]
  v = max(a, b);
  a = v;
  b = v;
  permlane32_swap(a, b);  // a: [lo half, lo half], b: [hi half, hi half]
  return max(a, b);
}

// Number of bits of the wave mask m set below this lane.
__device__ __forceinline__ int mbcnt64(uint64_t m) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
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
#define MOE_LDS __attribute__((address_space(3)))

// Global-address-space views of device pointers the compiler cannot place by itself (those that
// may come from the ingress buffer): loads, stores and atomics through them are global operations,
// counted by the vector-memory counter alone. Generic (flat) ones also count against the
// LDS / scalar-load counter, so every later LDS read or kernel-argument load would wait for them
// to complete (an atomic's or a store's full round trip).
template <typename T>
__device__ __forceinline__ MOE_GLOBAL T* gptr(T* p) {
  return (MOE_GLOBAL T*)p;
}
__device__ __forceinline__ void atomic_add_global(MOE_GLOBAL float* p, float v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A word that no kernel writes while this one runs, by a scalar load (its own counter, so it waits
// for no vector-memory operation).
__device__ __forceinline__ float load_const_f32(const float* p) {
  return *(const __attribute__((address_space(4))) float*)p;
}

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

// Make a value opaque to the optimiser so per-pass unpacking is not hoisted out of the pass loop
// (hoisting keeps every unpacked code live across the loop and multiplies register use).
__device__ __forceinline__ void opaque(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Load one word of every 64-byte line of [p, p + bytes) (bytes a positive multiple of 4), spread
// over the block's threads (at most N lines per thread). Plain loads (not the streaming ones) so the
// lines are kept in L2: a kernel reads, a few microseconds early, lines that the next kernel's block
// with the same index will read, and blocks with equal indices of consecutive launches run on the
// same XCD (one L2). The words are kept apart and only consumed by keep_live at the end of the
// block's work: any earlier use would make the wave wait for them, and (the memory counter being in
// order) for every load issued before them.
template <int N>
struct Touched {
  uint32_t v[N];
};
template <int N>
__device__ __forceinline__ Touched<N> touch_lines(const void* p, size_t bytes, int tid, int nthreads) {
  const uint8_t* b = static_cast<const uint8_t*>(p);
  Touched<N> t;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const size_t off = (static_cast<size_t>(i) * nthreads + tid) * 64;
    t.v[i] = *(const MOE_GLOBAL uint32_t*)(b + (off < bytes ? off : bytes - 4));
  }
  return t;
}
// Marks the words as used without storing them (the wave waits for them here).
template <int N>
__device__ __forceinline__ void keep_live(const Touched<N>& t) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(t.v[i]));
}

// Order-preserving 64-bit key of a logit with the expert id in the low 9 bits, so one unsigned
// max picks the largest logit and, among logits equal to 2^-43 relative, the lower id.
__device__ __forceinline__ uint64_t logit_key(double z, int e) {
  if (!(z == z)) z = -INFINITY;  // NaN ranks lowest
  uint64_t b = __builtin_bit_cast(uint64_t, z);
  b = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return (b & ~0x1FFull) | static_cast<uint64_t>(511 - e);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return 511 - static_cast<int>(key & 0x1FFull); }


// Digits of two 32-blocks by one wave (see kXqWords): lanes 0-31 take block qb, lanes 32-63 block
// qb + 1, one element per lane. The integer q = rint(x / step) with step = max|x| / kXqMax is split
// into balanced base-256 digits d0, d1, d2 in [-127, 127], each lane storing its three digit bytes
// at their places in the even / odd words; the block sum is kept in fp32. Blocks at or past nq are
// skipped (their lanes still take part in the reductions, on a clamped block). seed: if not null,
// each element is also copied there (the residual the layer's output rows start from).
__device__ __forceinline__ void quantize_block_pair(const float* x, uint32_t* xq, float2* xss, int qb, int nq,
                                                    MOE_GLOBAL float* seed) {
  const int lane = threadIdx.x & 63, e = lane & 31;
  const int b = qb + (lane >> 5);
  const float v = gptr(x)[static_cast<size_t>(min(b, nq - 1)) * 32 + e];
  float mx = fabsf(v), sum = v;
  mx = fmaxf(mx, dpp_f32<kDppXor1>(mx));
  sum += dpp_f32<kDppXor1>(sum);
  mx = fmaxf(mx, dpp_f32<kDppXor2>(mx));
  sum += dpp_f32<kDppXor2>(sum);
  mx = fmaxf(mx, dpp_f32<kDppHalfMirror>(mx));
  sum += dpp_f32<kDppHalfMirror>(sum);
  mx = fmaxf(mx, dpp_f32<kDppMirror>(mx));
  sum += dpp_f32<kDppMirror>(sum);
  mx = fmaxf(mx, swap_partner_f32<false>(mx));  // the other 16-lane row of this half
  sum += swap_partner_f32<false>(sum);
  const float inv = mx > 0.f ? kXqMax / mx : 0.f;
  int q = static_cast<int>(rintf(v * inv));
  q = max(-static_cast<int>(kXqMax), min(static_cast<int>(kXqMax), q));
  const int d0 = ((q + 128) & 255) - 128;
  const int q1 = (q - d0) >> 8;
  const int d1 = ((q1 + 128) & 255) - 128;
  const int d2 = (q1 - d1) >> 8;
  if (b < nq) {
    if (seed) seed[static_cast<size_t>(b) * 32 + e] = v;
    // element e = 8g + i sits in word (plane * 4 + g) * 2 + (i & 1), byte i >> 1
    uint8_t* dst = reinterpret_cast<uint8_t*>(xq + static_cast<size_t>(b) * kXqWords);
    const int g = e >> 3, i = e & 7;
    const int off = ((g * 2 + (i & 1)) * 4) + (i >> 1);
    dst[off] = static_cast<uint8_t>(d0 & 0xFF);
    dst[32 + off] = static_cast<uint8_t>(d1 & 0xFF);
    dst[64 + off] = static_cast<uint8_t>(d2 & 0xFF);
    if (e == 0) xss[b] = make_float2(mx / kXqMax, sum);
  }
}

}  // namespace moe
