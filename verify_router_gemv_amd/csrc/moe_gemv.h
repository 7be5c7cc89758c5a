// Shared pieces of the dequant-GEMV kernels (lane layout, activation loads, LDS staging).
#pragma once

#include "moe_route.h"

namespace moe {

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

template <int FMT>
struct BlockScale;

template <>
struct BlockScale<kFmtQ4B32> {
  uint32_t w;
  __device__ __forceinline__ void load(const uint32_t* sm_row, int b) { w = load_stream_u32(sm_row + b); }
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

template <int NB, int RC, typename BS>
__device__ __forceinline__ void block_dots(const uint4 c[NB], const BS sm[NB], const float xv[RC][NB][32],
                                           const float xs[RC][NB], float acc[RC]) {
#pragma unroll
  for (int r = 0; r < RC; ++r) acc[r] = 0.f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float q[32];
    unpack_block(c[nb], q);
    const float sc = sm[nb].scale(), mn = sm[nb].minv();
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

}  // namespace moe
