// Kernel 3: gate/up dequant-GEMV with SwiGLU.
#pragma once

#include "moe_gemv.h"

namespace moe {

// Gate/up: integer dot products of the 4-bit codes with the int8 digits of the layer input.
// Codes unpack into bytes (even / odd elements of each 8-group, two VALU per word); each row
// routed to the expert then costs 24 v_dot4 per 32-weight block plus the fp32 fold
// s * step * (65536 A2 + 256 A1 + A0) + m * sum(x). A0 + 256 A1 is formed as an integer: each
// plane's sum is at most 32 * 15 * 127 in magnitude, so it stays below 2^24 and converts exactly.
__device__ __forceinline__ float block_dot(const uint32_t cw[8], const uint32_t xd[kXqWords]) {
  int A[3] = {0, 0, 0};
#pragma unroll
  for (int dg = 0; dg < 3; ++dg)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      A[dg] = __builtin_amdgcn_sdot4(static_cast<int>(cw[2 * g]), static_cast<int>(xd[(dg * 4 + g) * 2]), A[dg], false);
      A[dg] = __builtin_amdgcn_sdot4(static_cast<int>(cw[2 * g + 1]), static_cast<int>(xd[(dg * 4 + g) * 2 + 1]),
                                     A[dg], false);
    }
  return fmaf(static_cast<float>(A[2]), 65536.f, static_cast<float>(A[0] + A[1] * 256));
}
// The fold of one block: acc + s * step * dot + m * sum(x), with the block's scale s and minimum m.
__device__ __forceinline__ float block_fold(float dot, float sc, float mn, float step, float xsum, float acc) {
  return fmaf(sc * step, dot, fmaf(mn, xsum, acc));
}
template <typename BS>
__device__ __forceinline__ float block_dot_q8(const uint32_t cw[8], const uint32_t xd[kXqWords], float step,
                                              float xsum, const BS& sm, float acc) {
  return block_fold(block_dot(cw, xd), sm.scale(), sm.minv(), step, xsum, acc);
}

__device__ __forceinline__ void unpack_bytes(const uint4 c, uint32_t cw[8]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cw[2 * i] = w[i] & 0x0F0F0F0Fu;
    cw[2 * i + 1] = (w[i] >> 4) & 0x0F0F0F0Fu;
  }
}

// T > 1: the input digits of the rows routed to the expert are copied into LDS, gateup_stage_rows
// rows at a time, by direct global->LDS loads (global_load_lds_dwordx4: no registers held while in
// flight). LDS layout per chunk: digits [rows][H/32][24 words] as in global memory, then (step,
// block sum) [rows][H/32][2 floats]; each region is followed by 1 KB of slack for the clamped lanes
// of a partial wave-wide copy.
constexpr int kGuLdsSlackWords = 256;

// Rows per staged chunk for reduction length H: within 32 KB of LDS, at most 4.
__host__ __device__ inline int gateup_stage_rows(int H) {
  const int r = 32768 / ((H / 32) * (kXqWords + 2) * 4);
  return r < 1 ? 1 : (r > 4 ? 4 : r);
}

__host__ __device__ inline int gateup_stage_words(int H) {
  return gateup_stage_rows(H) * (H / 32) * (kXqWords + 2) + 2 * kGuLdsSlackWords;
}

// One wave-wide copy of 64 16-byte chunks: lane l's chunk lands at lds + 16 * l bytes.
__device__ __forceinline__ void copy_to_lds16(const void* src, uint32_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void*)src, (__attribute__((address_space(3))) void*)lds_wave_base,
                                   16, 0, 0);
}

// ------------------------------------------------------------------------------------------
// Matrix-core tile for experts with several routed rows (H = 2048: 64 blocks of 32 per row).
//
// The block's 16 rows of gate and of up are multiplied with up to 16 of the expert's rows at a
// time by v_mfma_i32_16x16x32_i8, one 32-weight block per instruction: A = the 16 rows' 4-bit
// codes as bytes (even elements of each 8-group, then odd ones: the order the input digits are
// stored in), B = one int8 digit plane of the 16 input rows, D = exact int32 block dot products.
// Three planes give the 24-bit dot product, folded per block as s * step * (65536 D2 + 256 D1 + D0)
// + m * sum(x), like the GEMV fold. Lane l of A/B holds row/column l % 16 and elements 8(l/16)..+7;
// D lane l holds rows 4(l/16)..+3 of column l % 16. The 4 waves split the 64 blocks (16 each) and
// add their partial sums in LDS. The B columns are the expert's rows staged in LDS, gateup_stage_rows
// at a time (the remaining columns repeat a staged row and are dropped); a pass costs the same for
// any number of rows up to that, against one GEMV pass per row, so it pays from a few rows on.
// ------------------------------------------------------------------------------------------
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaBlocksPerWave = 16;  // 32-blocks of the reduction per wave (H = 2048)

// LDS words of the tile beyond the staged rows: per wave (s, m) as floats [matrix][16 blocks]
// [16 rows], then the partial sums [wave][matrix][16 rows][16 columns].
constexpr int kMfmaSmWords = 2 * kMfmaBlocksPerWave * 16 * 2;
constexpr int kMfmaExtraWords = kWaves * kMfmaSmWords + kWaves * 2 * 256;

__device__ __forceinline__ uint64_t code_bytes64(uint32_t w) {
  const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
  return static_cast<uint64_t>(ev) | (static_cast<uint64_t>(od) << 32);
}

// 4x4 transpose of dwords across the four 16-lane groups: before, group g holds words 0..3 of
// block g; after, group g holds word g of blocks 0..3.
__device__ __forceinline__ void transpose_groups(uint4& v) {
  permlane32_swap(v.x, v.z);
  permlane32_swap(v.y, v.w);
  permlane16_swap(v.x, v.y);
  permlane16_swap(v.z, v.w);
}

__device__ __forceinline__ float fold_block(const i32x4& d0, const i32x4& d1, const i32x4& d2, int i, float s_step,
                                            float m, float xsum, float acc) {
  const float val = fmaf(static_cast<float>(d2[i]), 65536.f, static_cast<float>(d1[i] * 256 + d0[i]));
  return fmaf(s_step, val, fmaf(m, xsum, acc));
}

template <typename StageFn>
__device__ __forceinline__ void gateup_mfma_tile(const Args& a, const ExpertWork& wk, const ExpertPtrs& W,
                                                 int row0, const uint32_t* xs_dig, const float* xs_ss, int SR,
                                                 uint32_t* lds, StageFn stage) {
  const int I = a.I;
  const int nblk = kWaves * kMfmaBlocksPerWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int kb0 = wave * kMfmaBlocksPerWave;
  const size_t rg = min(row0 + r, I - 1);  // row of the expert's gate and up matrices
  const size_t rq = static_cast<size_t>(nblk) * 16, rsm = nblk;

  // Codes: for group j lane (r, q) loads block kb0 + 4j + q of row r; after the transpose lane
  // (r, q) holds word q of blocks kb0 + 4j + 0..3. Scale/min: blocks kb0 + 4q .. +3 of row r.
  uint4 cg[4], cu[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cg[j] = load_stream_u4(W.gq + rg * rq + 16 * (kb0 + 4 * j + q));
    cu[j] = load_stream_u4(W.uq + rg * rq + 16 * (kb0 + 4 * j + q));
  }
  const uint4 smg = load_stream_u4(W.gs + rg * rsm + kb0 + 4 * q);
  const uint4 smu = load_stream_u4(W.us + rg * rsm + kb0 + 4 * q);

  float* sm_lds = reinterpret_cast<float*>(lds) + wave * kMfmaSmWords;  // [matrix][block][row] (s, m)
  float* red = reinterpret_cast<float*>(lds) + kWaves * kMfmaSmWords;   // [wave][matrix][row][column]
  {
    const uint32_t wg[4] = {smg.x, smg.y, smg.z, smg.w}, wu[4] = {smu.x, smu.y, smu.z, smu.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int bl = 4 * q + c;
      *reinterpret_cast<f32x2*>(sm_lds + ((0 * kMfmaBlocksPerWave + bl) * 16 + r) * 2) =
          f32x2{half_bits_to_float(wg[c]), half_bits_to_float(wg[c] >> 16)};
      *reinterpret_cast<f32x2*>(sm_lds + ((1 * kMfmaBlocksPerWave + bl) * 16 + r) * 2) =
          f32x2{half_bits_to_float(wu[c]), half_bits_to_float(wu[c] >> 16)};
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    transpose_groups(cg[j]);
    transpose_groups(cu[j]);
  }
  __syncthreads();  // scale/min tables written, first chunk of rows staged

  for (int c0 = 0; c0 < wk.np; c0 += SR) {
    if (c0 > 0) {
      stage(c0);
      __syncthreads();  // (the compiler waits for the LDS copies before the barrier)
    }
    const int nr = min(SR, wk.np - c0);
    const int col = min(r, nr - 1);  // B column r: staged row r of the chunk
    const uint32_t* bsrc = xs_dig + (col * nblk + kb0) * kXqWords + 2 * q;
    const float* ssrc = xs_ss + (col * nblk + kb0) * 2;
    float accg[4] = {0.f, 0.f, 0.f, 0.f}, accu[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int bs = 0; bs < kMfmaBlocksPerWave; ++bs) {
      uint64_t dig[3];
#pragma unroll
      for (int d = 0; d < 3; ++d) dig[d] = *reinterpret_cast<const uint64_t*>(bsrc + bs * kXqWords + d * 8);
      const f32x2 ss = *reinterpret_cast<const f32x2*>(ssrc + 2 * bs);
      const uint4& wgq = cg[bs >> 2];
      const uint4& wuq = cu[bs >> 2];
      const uint32_t wgw = (bs & 3) == 0 ? wgq.x : (bs & 3) == 1 ? wgq.y : (bs & 3) == 2 ? wgq.z : wgq.w;
      const uint32_t wuw = (bs & 3) == 0 ? wuq.x : (bs & 3) == 1 ? wuq.y : (bs & 3) == 2 ? wuq.z : wuq.w;
      const float step = ss.x, xsum = ss.y;
      const i32x4 z = {0, 0, 0, 0};
      {
        const long ag = static_cast<long>(code_bytes64(wgw));
        const i32x4 g0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(ag, static_cast<long>(dig[0]), z, 0, 0, 0);
        const i32x4 g1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(ag, static_cast<long>(dig[1]), z, 0, 0, 0);
        const i32x4 g2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(ag, static_cast<long>(dig[2]), z, 0, 0, 0);
        const float* sp = sm_lds + ((0 * kMfmaBlocksPerWave + bs) * 16 + 4 * q) * 2;
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(sp), s1 = *reinterpret_cast<const f32x4*>(sp + 4);
        accg[0] = fold_block(g0, g1, g2, 0, s0.x * step, s0.y, xsum, accg[0]);
        accg[1] = fold_block(g0, g1, g2, 1, s0.z * step, s0.w, xsum, accg[1]);
        accg[2] = fold_block(g0, g1, g2, 2, s1.x * step, s1.y, xsum, accg[2]);
        accg[3] = fold_block(g0, g1, g2, 3, s1.z * step, s1.w, xsum, accg[3]);
      }
      {
        const long au = static_cast<long>(code_bytes64(wuw));
        const i32x4 u0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(au, static_cast<long>(dig[0]), z, 0, 0, 0);
        const i32x4 u1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(au, static_cast<long>(dig[1]), z, 0, 0, 0);
        const i32x4 u2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(au, static_cast<long>(dig[2]), z, 0, 0, 0);
        const float* sp = sm_lds + ((1 * kMfmaBlocksPerWave + bs) * 16 + 4 * q) * 2;
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(sp), s1 = *reinterpret_cast<const f32x4*>(sp + 4);
        accu[0] = fold_block(u0, u1, u2, 0, s0.x * step, s0.y, xsum, accu[0]);
        accu[1] = fold_block(u0, u1, u2, 1, s0.z * step, s0.w, xsum, accu[1]);
        accu[2] = fold_block(u0, u1, u2, 2, s1.x * step, s1.y, xsum, accu[2]);
        accu[3] = fold_block(u0, u1, u2, 3, s1.z * step, s1.w, xsum, accu[3]);
      }
    }
    // Partial sums of this wave's quarter of the reduction -> LDS; then one (row, column) per thread.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[((wave * 2 + 0) * 16 + 4 * q + i) * 16 + r] = accg[i];
      red[((wave * 2 + 1) * 16 + 4 * q + i) * 16 + r] = accu[i];
    }
    __syncthreads();
    {
      const int rr = tid >> 4, cc = tid & 15;
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        gs += red[((w * 2 + 0) * 16 + rr) * 16 + cc];
        us += red[((w * 2 + 1) * 16 + rr) * 16 + cc];
      }
      const int i = row0 + rr;
      if (cc < nr && i < I) a.hbuf[static_cast<size_t>(wk.p0 + c0 + cc) * I + i] = silu(gs) * us;
    }
    __syncthreads();  // the staged rows and the partial-sum area are reused by the next chunk
  }
}

constexpr int kGuOneRow = 0, kGuPairs = 1, kGuStaged = 2, kGuRowItems = 3;

// MODE: kGuOneRow (T == 1), kGuRowItems (verify rounds of one-row work items: the one-row unit
// with the many-row selection), kGuPairs (verify rounds: rows two at a time from L2), kGuStaged
// (wide rounds: rows staged in LDS, matrix-core tile for items with many rows).
// SEL > 0 (verify rounds): the block first computes the round's selection itself from the logits
// (select_block with SEL keys per lane), finds its work item in LDS, and the last block publishes the
// records and outputs that the down kernel and the caller read; no separate selection launch.
// SEL == 0: the work item comes from the records written by select_kernel.
constexpr int kFusedPairs = 256;  // (row, rank) pairs of a round with the selection fused in
// Fused blocks of the many-row forms are kFusedGroups groups of kWaves waves: the block's selection
// runs once for the whole CU (each row on a wave of its own), then each group works on its own
// units as a four-wave block would.
constexpr int kFusedGroups = 3;
constexpr int gateup_groups(int mode, int sel) {
  return sel > 0 && (mode == kGuRowItems || mode == kGuPairs) ? kFusedGroups : 1;
}

// One unit of gate/up work: work item `wk`, rows tile * ROWS_B .. of I.
template <int G, int NB, int RW, int MODE, int FMT>
__device__ __forceinline__ void gateup_unit(const Args& a, int layer, const ExpertWork& wk, int tile, uint32_t* xs) {
  constexpr int RPI = 64 / G;
  constexpr int ROWS_W = RW * RPI;
  constexpr int ROWS_B = kWaves * ROWS_W;
  const int I = a.I, H = a.H, T = a.T;
  constexpr bool STAGE = MODE == kGuStaged;
  const int nblk = H / 32;

  // the wave index as a uniform value: row addresses shared by the wave's lanes are then scalar math
  // (in a block of several groups, the thread's index within its group of kWaves waves)
  const int tid = threadIdx.x & (kThreads - 1), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane % G, rs = lane / G;
  const ExpertPtrs W = expert_ptrs<FMT>(a, wk.e);  // issued first: every weight address needs it
  const int row0 = tile * ROWS_B + wave * ROWS_W + rs;
  const size_t rq = static_cast<size_t>(H) / 2, rsm = sm_row_words<FMT>(H);
  const int SR = a.xstage_h;

  // Staging (STAGE): wave w issues the chunk copies w, w + 4, ...; a lane's 16-byte chunk c of the
  // chunk's rows goes to LDS word 4c. Copies are issued before the weight loads and need no registers.
  uint32_t* xs_dig = xs;
  uint32_t* xs_ss = xs + SR * nblk * kXqWords + kGuLdsSlackWords;
  auto stage = [&](int r0) {
    const int nr = min(SR, wk.np - r0);          // rows of this chunk
    const int per_row = nblk * (kXqWords / 4);  // 16-byte chunks of one row's digits
    const int total = nr * per_row;
    for (int ins = wave; ins * 64 < total; ins += kWaves) {
      const int c = min(ins * 64 + lane, total - 1);
      const int rr = c / per_row, j = c - rr * per_row;
      const int t = work_row(wk, r0 + rr, T);
      copy_to_lds16(a.xq + static_cast<size_t>(t) * nblk * kXqWords + 4 * j, xs_dig + ins * 256);
    }
    const int per_row2 = nblk / 2;  // 16-byte chunks of one row's (step, sum) pairs
    const int total2 = nr * per_row2;
    for (int ins = wave; ins * 64 < total2; ins += kWaves) {
      const int c = min(ins * 64 + lane, total2 - 1);
      const int rr = c / per_row2, j = c - rr * per_row2;
      const int t = work_row(wk, r0 + rr, T);
      copy_to_lds16(a.xss + static_cast<size_t>(t) * nblk + 2 * j, xs_ss + ins * 256);
    }
  };
  if constexpr (STAGE) stage(0);
  if constexpr (STAGE && FMT == kFmtQ4B32 && G == 64 && NB == 1 && RW == 4) {  // 16-row tiles over H = 2048
    if (a.mfma_rows > 0 && wk.np >= a.mfma_rows) {
      gateup_mfma_tile(a, wk, W, tile * ROWS_B, xs_dig, reinterpret_cast<const float*>(xs_ss), SR,
                       xs + gateup_stage_words(H), stage);
      return;
    }
  }

  // Digits of the item's rows for this lane's blocks (NB x 24 words plus (step, block sum) per row).
  // Without STAGE (verify rounds, at most two rows per item in the usual split) they come from
  // global memory (L2) two rows at a time, both loaded before either is used; with STAGE from LDS.
  // The first rows' loads are issued before the weight loads: they return sooner and are needed
  // first, and no wait the compiler places before the row loop (for converted scales) can then
  // hold them back behind the weights.
  constexpr int SLOTS = MODE == kGuPairs ? 2 : 1;
  uint32_t xd[SLOTS][NB][kXqWords];
  float xstep[SLOTS][NB], xsum[SLOTS][NB];
  auto load_row = [&](int slot, int rr) {
    const int t = work_row(wk, rr, T);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const size_t blk = static_cast<size_t>(t) * nblk + min(g + nb * G, nblk - 1);
      const MOE_GLOBAL u32x4* src = (const MOE_GLOBAL u32x4*)(a.xq + blk * kXqWords);
#pragma unroll
      for (int q = 0; q < kXqWords / 4; ++q) {
        const u32x4 v = src[q];
        xd[slot][nb][4 * q + 0] = v.x;
        xd[slot][nb][4 * q + 1] = v.y;
        xd[slot][nb][4 * q + 2] = v.z;
        xd[slot][nb][4 * q + 3] = v.w;
      }
      const f32x2 ss = ((const MOE_GLOBAL f32x2*)(a.xss))[blk];
      xstep[slot][nb] = ss.x;
      xsum[slot][nb] = ss.y;
    }
  };
  const int np = wk.np;
  if constexpr (MODE == kGuOneRow || MODE == kGuRowItems) {
    load_row(0, 0);
  } else if constexpr (MODE == kGuPairs) {
    load_row(0, 0);
    load_row(SLOTS - 1, min(1, np - 1));
  }

  // This unit's share of its expert's down rows (H split like I over the item's tiles), touched now
  // so the down kernel's block with the same index finds them in cache (see touch_lines). Issued
  // before the weight loads, so the wait for the weights covers them; issued in any case (without
  // prefetching they touch a line of the input digits, read anyway).
  const int pf_tiles = (I + ROWS_B - 1) / ROWS_B;
  const int pf_r0 = tile * H / pf_tiles;  // tile < I / 16 and H <= 8192: no overflow
  const int pf_r1 = (tile + 1) * H / pf_tiles;
  const bool pf_on = a.prefetch != 0 && pf_r1 > pf_r0;
  const size_t pf_q = static_cast<size_t>(I) / 2, pf_s = sm_row_words<FMT>(I) * 4;  // bytes per down row
  const size_t pf_d0 = pf_r0;
  const uint8_t* pf_idle = reinterpret_cast<const uint8_t*>(a.xq);  // a line read anyway (no weight address)
  const Touched<2> pfq = touch_lines<2>(pf_on ? W.dq + pf_d0 * pf_q : pf_idle,
                                        pf_on ? (pf_r1 - pf_r0) * pf_q : 64, tid, kThreads);
  const Touched<1> pfs = touch_lines<1>(pf_on ? reinterpret_cast<const uint8_t*>(W.ds) + pf_d0 * pf_s : pf_idle,
                                        pf_on ? (pf_r1 - pf_r0) * pf_s : 64, tid, kThreads);

  __builtin_amdgcn_sched_barrier(0);  // the loads above stay ahead of the weight loads
  uint4 cg[RW][NB], cu[RW][NB];
  BlockScale<FMT> sg[RW][NB], su[RW][NB];
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    const size_t r = min(row0 + w * RPI, I - 1);  // rows past I: not stored
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int bl = g + nb * G, b = min(bl, nblk - 1);
      cg[w][nb] = load_stream_u4(W.gq + r * rq + 16 * b);
      cu[w][nb] = load_stream_u4(W.uq + r * rq + 16 * b);
      sg[w][nb].load(W.gs + r * rsm, b);
      su[w][nb].load(W.us + r * rsm, b);
      sg[w][nb].mask(bl < nblk);
      su[w][nb].mask(bl < nblk);
    }
  }

  auto stage_row = [&](int slot, int rr) {  // STAGE: row rr of the current chunk, from LDS
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int blk = rr * nblk + min(g + nb * G, nblk - 1);
      const uint32_t* src = xs_dig + blk * kXqWords;
#pragma unroll
      for (int q = 0; q < kXqWords / 4; ++q) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + 4 * q);
        xd[slot][nb][4 * q + 0] = v.x;
        xd[slot][nb][4 * q + 1] = v.y;
        xd[slot][nb][4 * q + 2] = v.z;
        xd[slot][nb][4 * q + 3] = v.w;
      }
      const f32x2 ss = *reinterpret_cast<const f32x2*>(xs_ss + 2 * blk);
      xstep[slot][nb] = ss.x;
      xsum[slot][nb] = ss.y;
    }
  };
  // One row through gate and up, reduced and written (slot: which digit registers hold it).
  auto do_row = [&](int slot, int p) {
    float acc[2 * RW];
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      float ag = 0.f, au = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint4 c = cg[w][nb];
        opaque(c);  // unpack here, per row: not hoisted out of the row loop
        uint32_t cw[8];
        unpack_bytes(c, cw);
        ag = block_dot_q8(cw, xd[slot][nb], xstep[slot][nb], xsum[slot][nb], sg[w][nb], ag);
        c = cu[w][nb];
        opaque(c);
        unpack_bytes(c, cw);
        au = block_dot_q8(cw, xd[slot][nb], xstep[slot][nb], xsum[slot][nb], su[w][nb], au);
      }
      acc[w] = ag;       // gate partials: acc[0 .. RW-1]
      acc[RW + w] = au;  // up partials:   acc[RW .. 2RW-1]
    }
    MOE_GLOBAL float* hrow = (MOE_GLOBAL float*)(a.hbuf + static_cast<size_t>(wk.p0 + p) * I);  // global stores
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
  };

  if constexpr (MODE == kGuOneRow) {
    do_row(0, 0);
  } else if constexpr (MODE == kGuRowItems) {
    do_row(0, 0);
    for (int r = 1; r < np; ++r) {  // items of one row; more only with a wider rows_per_item
      load_row(0, r);
      do_row(0, r);
    }
  } else if constexpr (MODE == kGuPairs) {
    do_row(0, 0);  // the first pair, loaded before the weights (peeled off the loop so that the
    if (np > 1) do_row(SLOTS - 1, 1);  // compiler keeps those loads where they are)
    for (int r0 = 2; r0 < np; r0 += 2) {  // further pairs; the usual item is one pair
      load_row(0, r0);
      load_row(SLOTS - 1, min(r0 + 1, np - 1));
      do_row(0, r0);
      if (r0 + 1 < np) do_row(SLOTS - 1, r0 + 1);
    }
  } else {
    for (int r0 = 0; r0 < np; r0 += SR) {
      if (r0 > 0) {
        __syncthreads();  // the previous chunk has been read by every wave
        stage(r0);
      }
      __syncthreads();  // (the compiler waits for the LDS copies before the barrier)
      const int n = min(SR, np - r0);
      for (int rr = 0; rr < n; ++rr) {
        stage_row(0, rr);
        do_row(0, r0 + rr);
      }
    }
  }
  keep_live(pfq);
  keep_live(pfs);
}

// Rounds without the residual (and with the atomic combine) start the output rows at zero: the down
// kernel adds into them. Stores only, spread over the grid, issued by every block after its own
// work (nothing in this kernel reads the output, and the router has read the input by now), as
// global stores: a flat store would also count against the scalar-load counter, so the next
// wait for a kernel argument would wait for its write to complete.
template <int NT>  // the launched block size
__device__ __forceinline__ void zero_output(const Args& a, int layer) {
  const Ingress in = get_ingress(a);
  MOE_GLOBAL f32x4* o = (MOE_GLOBAL f32x4*)(layer_output(a, in, layer));
  const int n4 = a.T * a.H / 4;
  for (int i = blockIdx.x * NT + threadIdx.x; i < n4; i += gridDim.x * NT) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Blocks with the selection folded in (SEL > 0) compute it once and then take the units (item,
// tile) blockIdx.x, blockIdx.x + gridDim.x, ... (in blocks of GR four-wave groups, group g starts at
// blockIdx.x + g * gridDim.x and steps by GR * gridDim.x): the grid is sized for the chip, not for
// the largest possible item count, so no block repeats the selection only to find no work.
template <int G, int NB, int RW, int MODE, int SEL, int FMT>
__global__ __launch_bounds__(kThreads * gateup_groups(MODE, SEL)) void gateup_kernel(Args a, int layer) {
  constexpr int GR = gateup_groups(MODE, SEL), NT = kThreads * GR;  // launched with NT threads
  constexpr int ROWS_B = kWaves * RW * (64 / G);
  extern __shared__ uint32_t xs[];  // staged form: gateup_stage_words(H) (+ matrix-core tile) words
  const int tiles = (a.I + ROWS_B - 1) / ROWS_B;
  if constexpr (SEL > 0) {
    __shared__ SelectSharedT<kFusedPairs, NT / 64> ssel;
    // The last block publishes: it is the one most likely to have no (item, tile) unit of its own.
    select_block<SEL, NT, MODE == kGuOneRow>(a, layer, ssel, blockIdx.x == gridDim.x - 1);
    const int units = ssel.ni * tiles;
    const int grp = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kThreads);
    for (int w = blockIdx.x + grp * gridDim.x; w < units; w += gridDim.x * GR) {
      const int u = w / tiles;
      gateup_unit<G, NB, RW, MODE, FMT>(a, layer, work_from_lds(a, ssel, u), w - u * tiles, xs);
    }
  } else {
    const int u = blockIdx.x / tiles, tile = blockIdx.x - u * tiles;
    const ExpertWork wk = load_work(a, layer, u);
    if (u < wk.nu) gateup_unit<G, NB, RW, MODE, FMT>(a, layer, wk, tile, xs);
  }
  if (!a.residual && !a.exact) zero_output<NT>(a, layer);
}

}  // namespace moe
