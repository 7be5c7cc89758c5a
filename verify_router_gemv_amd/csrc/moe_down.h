// Kernel 4: down dequant-GEMV with the routing-weighted scatter-add.
#pragma once

#include "moe_gateup.h"

namespace moe {


// The item's SwiGLU rows as int8 digits in LDS, by the whole block: 8 threads per 32-block, 4
// elements each, in the layout and with the rounding of the layer input's digits (kXqWords words
// per block: three balanced base-256 digits of rint(h / step), step = max|h| / kXqMax), plus the
// block's (step, sum of h). `n` rows of length K, contiguous from `src`.
// The four values this thread quantises in the pass starting at block blk0 (blocks past the end:
// the last block again, still in the reductions).
__device__ __forceinline__ float4 stage_load(const float* src, int K, int n, int blk0) {
  const int total = n * (K / 32), sub = threadIdx.x & 7;
  const int bc = min(blk0 + static_cast<int>(threadIdx.x >> 3), total - 1);
  return load_f4(src + static_cast<size_t>(bc) * 32 + 4 * sub);
}

// first: the first pass's values, stage_load(src, K, n, 0), which the caller loads (early).
__device__ __forceinline__ void stage_digits(const float* src, int K, int n, uint32_t* dig, float2* ss,
                                             float4 first) {
  const int nblk = K / 32, total = n * nblk;
  const int tid = threadIdx.x, sub = tid & 7;
  float4 v = first;
  for (int blk0 = 0; blk0 < total; blk0 += kThreads / 8) {
    if (blk0 > 0) v = stage_load(src, K, n, blk0);
    const int blk = blk0 + (tid >> 3);
    float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    float sum = (v.x + v.y) + (v.z + v.w);
    mx = fmaxf(mx, dpp_f32<kDppXor1>(mx));
    sum += dpp_f32<kDppXor1>(sum);
    mx = fmaxf(mx, dpp_f32<kDppXor2>(mx));
    sum += dpp_f32<kDppXor2>(sum);
    mx = fmaxf(mx, dpp_f32<kDppHalfMirror>(mx));  // the 8 lanes of this block
    sum += dpp_f32<kDppHalfMirror>(sum);
    const float inv = mx > 0.f ? kXqMax / mx : 0.f;
    const float e[4] = {v.x, v.y, v.z, v.w};
    int d[3][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = static_cast<int>(rintf(e[i] * inv));
      q = max(-static_cast<int>(kXqMax), min(static_cast<int>(kXqMax), q));
      const int d0 = ((q + 128) & 255) - 128;
      const int q1 = (q - d0) >> 8;
      const int d1 = ((q1 + 128) & 255) - 128;
      d[0][i] = d0;
      d[1][i] = d1;
      d[2][i] = (q1 - d1) >> 8;
    }
    if (blk < total) {
      // element 4*sub + i: group sub / 2, even word for i = 0, 2 and odd for i = 1, 3, bytes
      // 2*(sub % 2) + i / 2 of the word
      uint16_t* base = reinterpret_cast<uint16_t*>(dig + static_cast<size_t>(blk) * kXqWords);
      const int g = sub >> 1, half = sub & 1;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const uint16_t ev = static_cast<uint16_t>((d[p][0] & 0xFF) | ((d[p][2] & 0xFF) << 8));
        const uint16_t od = static_cast<uint16_t>((d[p][1] & 0xFF) | ((d[p][3] & 0xFF) << 8));
        base[((p * 4 + g) * 2 + 0) * 2 + half] = ev;
        base[((p * 4 + g) * 2 + 1) * 2 + half] = od;
      }
      if (sub == 0) ss[blk] = make_float2(mx / kXqMax, sum);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Matrix-core tile of the down projection (I = 512: 16 blocks of 32 per row), wide rounds.
//
// Wave w of the block takes output rows row0 + 16w .. +15 over the whole reduction, so no partial
// sums meet in LDS: per 32-weight block, v_mfma_i32_16x16x32_i8 multiplies A = the 16 rows' codes as
// bytes with B = one digit plane of up to 16 staged SwiGLU rows (the chunk's rows; spare columns
// repeat a staged row and are dropped), three planes per block, folded per block like the GEMV:
// s * step * (65536 D2 + 256 D1 + D0) + m * sum(h). Lane layouts as in the gate/up tile: lane
// (r, q) = (l % 16, l / 16) holds row / column r, elements 8q..8q+7 of a block in A and B, and
// rows 4q..4q+3 of column r in D. The codes arrive as whole 16-byte blocks per lane and are
// transposed across the lane groups; the rows' (s, m) go through a per-wave table in LDS.
// ------------------------------------------------------------------------------------------
constexpr int kDownTileBlocks = 16;                             // I / 32 of the tile
constexpr int kDownTileSmWords = kDownTileBlocks * 16 * 2;      // per wave: [block][row] (s, m)
constexpr int kDownTileExtraWords = kWaves * kDownTileSmWords;

template <bool EXACT>
__device__ __forceinline__ void down_mfma_tile(const Args& a, int layer, const ExpertWork& wk, const ExpertPtrs& W,
                                               int row0, uint32_t* dig, float2* ss, int xst, float* sm_all,
                                               float4 h0) {
  const int H = a.H, I = a.I, T = a.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int hrow = row0 + wave * 16 + r;                       // this lane's code row
  const size_t rr = static_cast<size_t>(min(hrow, H - 1));
  uint4 cd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cd[j] = load_stream_u4(W.dq + rr * (I / 2) + 16 * (4 * j + q));
  const uint4 smw = load_stream_u4(W.ds + rr * (I / 32) + 4 * q);
  float* sm_lds = sm_all + wave * kDownTileSmWords;
  {
    const uint32_t wv[4] = {smw.x, smw.y, smw.z, smw.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<f32x2*>(sm_lds + ((4 * q + c) * 16 + r) * 2) =
          f32x2{half_bits_to_float(wv[c]), half_bits_to_float(wv[c] >> 16)};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) transpose_groups(cd[j]);

  const float* pw = a.pair_w + static_cast<size_t>(layer) * a.Pcap;
  const Ingress in = get_ingress(a);
  MOE_GLOBAL float* __restrict__ xn = gptr(layer_output(a, in, layer));
  for (int s0 = 0; s0 < wk.np; s0 += xst) {
    const int ns = min(xst, wk.np - s0);
    if (s0 > 0) __syncthreads();  // the previous chunk has been read by every wave
    const float* hsrc = a.hbuf + static_cast<size_t>(wk.p0 + s0) * I;
    stage_digits(hsrc, I, ns, dig, ss, s0 == 0 ? h0 : stage_load(hsrc, I, ns, 0));
    __syncthreads();  // (also: the (s, m) table written)
    const int col = min(r, ns - 1);  // B column r: staged row r of the chunk
    const uint32_t* bsrc = dig + static_cast<size_t>(col) * kDownTileBlocks * kXqWords + 2 * q;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int bs = 0; bs < kDownTileBlocks; ++bs) {
      uint64_t dg[3];
#pragma unroll
      for (int d = 0; d < 3; ++d) dg[d] = *reinterpret_cast<const uint64_t*>(bsrc + bs * kXqWords + d * 8);
      const float2 sx = ss[col * kDownTileBlocks + bs];
      const uint4& wq = cd[bs >> 2];
      const uint32_t ww = (bs & 3) == 0 ? wq.x : (bs & 3) == 1 ? wq.y : (bs & 3) == 2 ? wq.z : wq.w;
      const long av = static_cast<long>(code_bytes64(ww));
      const i32x4 z = {0, 0, 0, 0};
      const i32x4 d0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, static_cast<long>(dg[0]), z, 0, 0, 0);
      const i32x4 d1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, static_cast<long>(dg[1]), z, 0, 0, 0);
      const i32x4 d2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, static_cast<long>(dg[2]), z, 0, 0, 0);
      const float* sp = sm_lds + (bs * 16 + 4 * q) * 2;
      const f32x4 s0v = *reinterpret_cast<const f32x4*>(sp), s1v = *reinterpret_cast<const f32x4*>(sp + 4);
      acc[0] = fold_block(d0, d1, d2, 0, s0v.x * sx.x, s0v.y, sx.y, acc[0]);
      acc[1] = fold_block(d0, d1, d2, 1, s0v.z * sx.x, s0v.w, sx.y, acc[1]);
      acc[2] = fold_block(d0, d1, d2, 2, s1v.x * sx.x, s1v.y, sx.y, acc[2]);
      acc[3] = fold_block(d0, d1, d2, 3, s1v.z * sx.x, s1v.w, sx.y, acc[3]);
    }
    if (r < ns) {  // column r is pair slot s0 + r of the item
      const int slot = s0 + r;
      if constexpr (EXACT) {
        float* y = a.ybuf + static_cast<size_t>(wk.p0 + slot) * H;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hr = row0 + wave * 16 + 4 * q + i;
          if (hr < H) y[hr] = acc[i];
        }
      } else {
        const int t = work_row(wk, slot, T);
        const float wgt = load_const_f32(pw + wk.p0 + slot);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hr = row0 + wave * 16 + 4 * q + i;
          if (hr < H) atomic_add_global(xn + static_cast<size_t>(t) * H + hr, wgt * acc[i]);
        }
      }
    }
  }
}

// Down: W_d h for each pair of the work item, the same integer-digit dot product as gate/up: the
// item's h rows are quantised into LDS (a chunk of a.xstage_i rows at a time), then each lane takes
// its 32-blocks' digits row by row against its RW weight rows.
// EXACT: store W_d h of each pair in its slot of ybuf (the combine kernel adds them in rank order)
// instead of adding the weighted product into the output with an atomic.
// TILE (G = 16, NB = 1, RW = 4, Q4B32 only; wide rounds with the matrix-core tile enabled): items of at
// least a.mfma_rows rows take down_mfma_tile. A separate instantiation, so the registers the tile
// needs do not lower the occupancy of the plain form.
template <int G, int NB, int RW, bool EXACT, int FMT, bool TILE = false>
__global__ __launch_bounds__(kThreads) void down_kernel(Args a, int layer) {
  constexpr int RPI = 64 / G;
  constexpr int ROWS_W = RW * RPI;
  constexpr int ROWS_B = kWaves * ROWS_W;
  extern __shared__ uint32_t dlds[];  // [xstage_i][I/32][kXqWords] digits, then [xstage_i][I/32] (step, sum)
  const int I = a.I, H = a.H, T = a.T;
  const int nblk = I / 32;
  const int tiles = (H + ROWS_B - 1) / ROWS_B;
  const int u = blockIdx.x / tiles, tile = blockIdx.x - u * tiles;
  const ExpertWork wk = load_work(a, layer, u);
  if (u >= wk.nu) return;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int g = lane % G, rs = lane / G;
  const int xst = a.xstage_i;
  if constexpr (TILE) {  // 64 rows of H per block, I = 512
    static_assert(FMT == kFmtQ4B32 && G == 16 && NB == 1 && RW == 4, "the tile's shape");
    if (a.mfma_rows > 0 && wk.np >= a.mfma_rows) {
      const ExpertPtrs W = expert_ptrs<FMT>(a, wk.e);
      const float4 h0 = stage_load(a.hbuf + static_cast<size_t>(wk.p0) * I, I, min(xst, wk.np), 0);
      float* sm_all = reinterpret_cast<float*>(dlds + static_cast<size_t>(xst) * nblk * (kXqWords + 2));
      down_mfma_tile<EXACT>(a, layer, wk, W, tile * ROWS_B, dlds,
                            reinterpret_cast<float2*>(dlds + static_cast<size_t>(xst) * nblk * kXqWords), xst,
                            sm_all, h0);
      return;
    }
  }
  const float* pw = a.pair_w + static_cast<size_t>(layer) * a.Pcap;
  const Ingress in = get_ingress(a);
  MOE_GLOBAL float* __restrict__ xn = gptr(layer_output(a, in, layer));
  const int row0 = tile * ROWS_B + wave * ROWS_W + rs;
  const size_t rq = static_cast<size_t>(I) / 2, rsm = sm_row_words<FMT>(I);

  // The next layer's router row of the logits block with this block's index, touched (see
  // touch_lines) after the record (whose wait must not include it) and before the weights (whose
  // wait covers it); issued in any case (without prefetching: the first line of the item's SwiGLU rows).
  const float* rnext = a.router_next;
  const ExpertPtrs W = expert_ptrs<FMT>(a, wk.e);
  const bool pf_on = a.prefetch != 0 && rnext != nullptr && static_cast<int>(blockIdx.x) < a.E;
  const Touched<1> pfr = touch_lines<1>(pf_on ? static_cast<const void*>(rnext + static_cast<size_t>(blockIdx.x) * H)
                                              : static_cast<const void*>(a.hbuf + static_cast<size_t>(wk.p0) * I),
                                        pf_on ? static_cast<size_t>(H) * 4 : 64, threadIdx.x, kThreads);

  // The first chunk's SwiGLU values, loaded before the weights (they return sooner and are needed
  // first: the chunk is quantised into LDS before any weight is used). The scheduling barrier keeps
  // these loads (and the touch) ahead of the weight loads.
  const float4 h0 = stage_load(a.hbuf + static_cast<size_t>(wk.p0) * I, I, min(xst, wk.np), 0);
  __builtin_amdgcn_sched_barrier(0);

  // The scale words are masked where they are used (an idle block slot of a padded split), not
  // here: a mask here would make the wave wait for them before it stages the first chunk.
  uint4 cd[RW][NB];
  BlockScale<FMT> sd[RW][NB];
#pragma unroll
  for (int w = 0; w < RW; ++w) {
    const size_t r = min(row0 + w * RPI, H - 1);  // rows past H: not stored
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = min(g + nb * G, nblk - 1);
      cd[w][nb] = load_stream_u4(W.dq + r * rq + 16 * b);
      sd[w][nb].load(W.ds + r * rsm, b);
    }
  }

  uint32_t* dig = dlds;
  float2* ss = reinterpret_cast<float2*>(dlds + static_cast<size_t>(xst) * nblk * kXqWords);
  // The first chunk is staged ahead of the loop, from the values loaded before the weights: its
  // wait then covers those loads alone, and the staging and the barrier overlap the weight loads
  // (inside the loop the compiler would wait for every load at the loop head).
  stage_digits(a.hbuf + static_cast<size_t>(wk.p0) * I, I, min(xst, wk.np), dig, ss, h0);
  for (int s0 = 0; s0 < wk.np; s0 += xst) {
    const int ns = min(xst, wk.np - s0);
    if (s0 > 0) {
      __syncthreads();  // the previous chunk has been read by every wave
      const float* hsrc = a.hbuf + static_cast<size_t>(wk.p0 + s0) * I;
      stage_digits(hsrc, I, ns, dig, ss, stage_load(hsrc, I, ns, 0));
    }
    __syncthreads();
    for (int c = 0; c < ns; ++c) {
      const float wgt = load_const_f32(pw + wk.p0 + s0 + c);  // scalar: waits for no atomic
      uint32_t xd[NB][kXqWords];
      float xstep[NB], xsum[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int blk = c * nblk + min(g + nb * G, nblk - 1);
        const uint32_t* srcw = dig + static_cast<size_t>(blk) * kXqWords;
#pragma unroll
        for (int q = 0; q < kXqWords / 4; ++q) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(srcw + 4 * q);
          xd[nb][4 * q + 0] = v.x;
          xd[nb][4 * q + 1] = v.y;
          xd[nb][4 * q + 2] = v.z;
          xd[nb][4 * q + 3] = v.w;
        }
        const float2 t = ss[blk];
        xstep[nb] = t.x;
        xsum[nb] = t.y;
      }
      float acc[RW];
#pragma unroll
      for (int w = 0; w < RW; ++w) {
        float ay = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          uint4 cc = cd[w][nb];
          opaque(cc);  // unpack here, per row: not hoisted out of the row loop
          uint32_t cw[8];
          unpack_bytes(cc, cw);
          BlockScale<FMT> sc = sd[w][nb];
          sc.mask(g + nb * G < nblk);
          ay = block_dot_q8(cw, xd[nb], xstep[nb], xsum[nb], sc, ay);
        }
        acc[w] = group_sum<G>(ay);
      }
      if (g == 0) {
        const int slot = s0 + c;
        if constexpr (EXACT) {
          float* y = a.ybuf + static_cast<size_t>(wk.p0 + slot) * H;
#pragma unroll
          for (int w = 0; w < RW; ++w) {
            const int hr = row0 + w * RPI;
            if (hr < H) y[hr] = acc[w];
          }
        } else {
          const int t = work_row(wk, slot, T);
#pragma unroll
          for (int w = 0; w < RW; ++w) {
            const int hr = row0 + w * RPI;
            if (hr < H) atomic_add_global(xn + static_cast<size_t>(t) * H + hr, wgt * acc[w]);
          }
        }
      }
    }
  }
  keep_live(pfr);
}

// Exact mode: out[t][h] = (residual ? x[t][h] : 0) + sum over ranks j = 0..k-1, in that order, of
// p[t][j] * y[slot(t, j)][h] (ranks whose pair the tail skip left out add nothing). Grid (T, ceil(H / 1024)) x 256 threads, four columns per thread.
static __global__ __launch_bounds__(kThreads) void combine_kernel(Args a, int layer) {
  const Ingress in = get_ingress(a);
  const float* x = layer_input(a, in, layer);  // may be xn itself (the caller's hidden == out)
  float* xn = layer_output(a, in, layer);
  const int t = blockIdx.x, H = a.H, k = a.k;
  const int h = (blockIdx.y * kThreads + threadIdx.x) * 4;
  if (h >= H) return;
  const int32_t* slot_of = a.slot_of + static_cast<size_t>(layer) * a.Pcap + t * k;
  const float* pw = a.pair_w + static_cast<size_t>(layer) * a.Pcap;
  float4 acc = a.residual ? load_f4(x + static_cast<size_t>(t) * H + h) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    if (slot_of[j] < 0) continue;  // a pair the tail skip left out
    const int s = min(slot_of[j], a.Pcap - 1);
    const float w = pw[s];
    const float4 y = load_f4(a.ybuf + static_cast<size_t>(s) * H + h);
    acc.x = fmaf(w, y.x, acc.x);
    acc.y = fmaf(w, y.y, acc.y);
    acc.z = fmaf(w, y.z, acc.z);
    acc.w = fmaf(w, y.w, acc.w);
  }
  *reinterpret_cast<MOE_GLOBAL f32x4*>(gptr(xn) + static_cast<size_t>(t) * H + h) = f32x4{acc.x, acc.y, acc.z, acc.w};
}

}  // namespace moe
