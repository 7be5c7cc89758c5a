// Shared pieces of the dequant-GEMV kernels (lane layout, weight formats).
#pragma once

#include "moe_route.h"

namespace moe {

// ------------------------------------------------------------------------------------------
// Kernels 3 and 4: dequant-GEMV tiles
// ------------------------------------------------------------------------------------------
//
// Lane layout: G lanes share one weight row, each owning NB of its 32-weight blocks (block
// b = g + nb*G; when G * NB exceeds the row's K/32 blocks, the slots past the end load the row's
// last block and are masked to add zero); a wave covers 64/G rows per load and RW such row groups (for gate/up: of both
// matrices). Codes (16 B) and the block's scale/minimum source of each block are loaded once into
// registers. The activation rows (the layer input for gate/up, the SwiGLU rows for down) are
// int8 digits per 32-block; per block the dot product is s * step * (integer dot) + m * sum(x).

// ------------------------------------------------------------------------------------------
// Weight formats: where a 32-weight block's scale s and minimum m come from (w = s*q + m).
//   kFmtQ4B32:  one word per block, fp16 s (low half) and fp16 m (high half);
//               a row has K/32 words.
//   kFmtQ4S256: one 16-byte record per 256-weight super-block: word 0 holds fp16 d (low) and
//               fp16 dmin (high); words 1..3 a 96-bit string of eight 12-bit fields, field j
//               (bits 12j..12j+11) the 6-bit scale sc_j and 6-bit minimum m_j of sub-block j;
//               s = d*sc_j and m = -dmin*m_j (both exact in fp32); a row has K/64 words.
// The codes are the same in both.
// ------------------------------------------------------------------------------------------
constexpr int kFmtQ4B32 = 0, kFmtQ4S256 = 1;

template <int FMT>
__host__ __device__ constexpr size_t sm_row_words(size_t K) { return FMT == kFmtQ4S256 ? K / 64 : K / 32; }

// One expert's matrices: from the layer's contiguous [E][..] arrays, or, in table mode, from the
// expert's table entry (one dependent load; e is uniform over the block, so the entry's address is).
struct ExpertPtrs {
  const uint8_t* gq;
  const uint32_t* gs;
  const uint8_t* uq;
  const uint32_t* us;
  const uint8_t* dq;
  const uint32_t* ds;
};

template <int FMT>
__device__ __forceinline__ ExpertPtrs expert_ptrs(const Args& a, int e) {
  e = __builtin_amdgcn_readfirstlane(e);
  ExpertPtrs p;
  if (a.etab) {
    // Scalar loads (the table changes only between kernels, in stream order): the weight
    // addresses then do not wait for vector loads issued before them.
    uint64_t w[6];
    load_const_words(a.etab + e, w);
    p.gq = reinterpret_cast<const uint8_t*>(w[0]);
    p.gs = reinterpret_cast<const uint32_t*>(w[1]);
    p.uq = reinterpret_cast<const uint8_t*>(w[2]);
    p.us = reinterpret_cast<const uint32_t*>(w[3]);
    p.dq = reinterpret_cast<const uint8_t*>(w[4]);
    p.ds = reinterpret_cast<const uint32_t*>(w[5]);
    return p;
  }
  const size_t H = a.H, I = a.I, ex = static_cast<size_t>(e);
  p.gq = a.w.gate_q + ex * I * (H / 2);
  p.gs = a.w.gate_sm + ex * I * sm_row_words<FMT>(H);
  p.uq = a.w.up_q + ex * I * (H / 2);
  p.us = a.w.up_sm + ex * I * sm_row_words<FMT>(H);
  p.dq = a.w.down_q + ex * H * (I / 2);
  p.ds = a.w.down_sm + ex * H * sm_row_words<FMT>(I);
  return p;
}

template <int FMT>
struct BlockScale;

template <>
struct BlockScale<kFmtQ4B32> {
  uint32_t w;
  __device__ __forceinline__ void load(const uint32_t* sm_row, int b) { w = load_stream_u32(sm_row + b); }
  // An idle block slot of a padded lane split: scale and minimum 0, so the block adds nothing.
  __device__ __forceinline__ void mask(bool live) { w = live ? w : 0u; }
  __device__ __forceinline__ float scale() const { return half_bits_to_float(w); }
  __device__ __forceinline__ float minv() const { return half_bits_to_float(w >> 16); }
};

template <>
struct BlockScale<kFmtQ4S256> {
  uint4 r;  // the super-block's record
  int j;    // sub-block of this 32-weight block
  __device__ __forceinline__ void load(const uint32_t* sm_row, int b) {
    r = load_stream_u4(sm_row + 4 * (b >> 3));
    j = b & 7;
  }
  __device__ __forceinline__ void mask(bool live) { r.x = live ? r.x : 0u; }  // d = dmin = 0
  __device__ __forceinline__ uint32_t field() const {
    const uint64_t lo = static_cast<uint64_t>(r.y) | (static_cast<uint64_t>(r.z) << 32);  // bits 0..63
    const uint64_t hi = static_cast<uint64_t>(r.z) | (static_cast<uint64_t>(r.w) << 32);  // bits 32..95
    const uint64_t v = j < 5 ? (lo >> (12 * j)) : (hi >> (12 * j - 32));
    return static_cast<uint32_t>(v) & 0xFFFu;
  }
  __device__ __forceinline__ float scale() const {
    return half_bits_to_float(r.x) * static_cast<float>(field() & 63u);
  }
  __device__ __forceinline__ float minv() const {
    return -half_bits_to_float(r.x >> 16) * static_cast<float>(field() >> 6);
  }
};

}  // namespace moe
