// Router logits, selection and the per-expert work records (kernels 1 and 2).
#pragma once

#include "moe_common.h"

namespace moe {

// ------------------------------------------------------------------------------------------
// Kernel 1: router logits (+ output seeding)
// ------------------------------------------------------------------------------------------

// Grid: (E + ceil(T * H / 256), ceil(T / TC)) x 256 threads.
//  * Blocks x < E: expert x's logits for rows y * TC .. y * TC + TC - 1. The reduction over H is split
//    over the block's four waves (thread i takes float4 chunks i, i + 256, ... of the row), every load
//    of the thread (its router chunks and the TC rows' chunks) is issued before any arithmetic, each
//    wave sums its part of all TC rows at once in fp64 (by a tree that is the same for every row and
//    every TC) and wave 0 adds the four parts in wave order (a fixed order).
//  * Blocks x >= E (row chunk 0 only): the layer input as int8 digits per 32-block for the gate/up
//    kernel, two 32-blocks per wave; with the residual (and the atomic combine) they also seed the
//    layer's output rows with the input rows. These blocks read no router row, so the router waves
//    finish after one load round trip. (Without the residual the output rows are zeroed by the gate/up
//    kernel instead: nothing may write the output while the router reads the input, since a caller
//    may pass the same buffer as both.)
template <int NJ, int TC>  // NJ = ceil(H / 1024): float4 chunks of a row per thread
__global__ __launch_bounds__(kThreads) void logits_kernel(Args a, int layer) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E, H = a.H;
  // Only the first layer reads its input through the ingress pointers (in graph mode a load from
  // device memory that every later address would wait for); later layers' inputs are fixed.
  const float* __restrict__ x =
      layer == 0 ? get_ingress(a).hidden : a.xall + static_cast<size_t>((layer - 1) % a.xslots) * a.xstride;
  const moe_layer_weights& W = get_weights(a, layer);
  const float* __restrict__ router = W.router_w;
  const float* __restrict__ rbias = W.router_bias;
  asm volatile("" ::"s"(router), "s"(rbias));  // fetched with the first kernel arguments, not after the branch

  if (static_cast<int>(blockIdx.x) >= E) {
    if (blockIdx.y != 0) return;
    const int nq = T * (H / 32);  // 32-blocks of the layer input, two per wave
    const int qb = 2 * ((blockIdx.x - E) * kWaves + wave);
    if (qb >= nq) return;
    MOE_GLOBAL float* seed = (a.residual && !a.exact) ? gptr(layer_output(a, get_ingress(a), layer)) : nullptr;
    quantize_block_pair(x, a.xq, a.xss, qb, nq, seed);
    return;
  }
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * TC;
  const int n4 = H / 4;
  float4 w[NJ], xv[TC][NJ];
  const float4* wr = reinterpret_cast<const float4*>(router + static_cast<size_t>(e) * H);
#pragma unroll
  for (int j = 0; j < NJ; ++j) w[j] = load_stream_f4(wr + min(tid + kThreads * j, n4 - 1));
#pragma unroll
  for (int r = 0; r < TC; ++r) {
    const float4* xr = reinterpret_cast<const float4*>(x + static_cast<size_t>(min(t0 + r, T - 1)) * H);
#pragma unroll
    for (int j = 0; j < NJ; ++j) xv[r][j] = load_f4(xr + min(tid + kThreads * j, n4 - 1));
  }
  const double bias = rbias ? static_cast<double>(rbias[e]) : 0.0;

  double acc[TC];
#pragma unroll
  for (int r = 0; r < TC; ++r) {
    acc[r] = 0.0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (tid + kThreads * j >= n4) continue;  // past the end of the row (its load was clamped)
      acc[r] = fma(static_cast<double>(w[j].x), static_cast<double>(xv[r][j].x), acc[r]);
      acc[r] = fma(static_cast<double>(w[j].y), static_cast<double>(xv[r][j].y), acc[r]);
      acc[r] = fma(static_cast<double>(w[j].z), static_cast<double>(xv[r][j].z), acc[r]);
      acc[r] = fma(static_cast<double>(w[j].w), static_cast<double>(xv[r][j].w), acc[r]);
    }
  }
  __shared__ double part[kWaves][TC];
  {
    const double sum = wave_sums_f64<TC>(acc);  // row lane / (64 / TC)
    if ((lane & (64 / TC - 1)) == 0) part[wave][lane / (64 / TC)] = sum;
  }
  __syncthreads();
  if (tid < TC && t0 + tid < T) {
    double z = part[0][0];
#pragma unroll
    for (int r = 0; r < TC; ++r)
      if (r == tid) z = ((part[0][r] + part[1][r]) + part[2][r]) + part[3][r];
    a.logits[static_cast<size_t>(t0 + tid) * E + e] = z + bias;
  }
}

// ------------------------------------------------------------------------------------------
// Kernel 2: selection + worklist (one block)
// ------------------------------------------------------------------------------------------

// Selection state of one round in LDS, for up to PMAX (row, rank) pairs and NW waves.
template <int PMAX, int NW>
struct SelectSharedT {
  int sel[PMAX];                                       // [t][j] expert id
  float p[PMAX];                                       // [t][j] routing weight
  unsigned long long mask[MOE_ROUND_MAX_EXPERTS];      // rows choosing expert e
  int uidx[MOE_ROUND_MAX_EXPERTS];                     // e -> unique index
  int uniq[MOE_ROUND_MAX_EXPERTS];
  int offs[MOE_ROUND_MAX_EXPERTS + 1];
  int ioffs[MOE_ROUND_MAX_EXPERTS];                    // unique index -> first work item
  int pairs[PMAX];                                     // by pair slot: t | j << 8
  int item_u[PMAX];                                    // work item -> unique index
  unsigned long long ctot[MOE_ROUND_MAX_EXPERTS / 64];  // per 64-expert chunk: chosen, rows, items, skipped
  unsigned long long tmask[MOE_ROUND_MAX_EXPERTS];     // tail skip: rows whose pair with e is a tail pair
  int slot[PMAX];                                      // [t][j] the pair's worklist slot, -1 if skipped
  uint32_t res[MOE_ROUND_MAX_EXPERTS / 32];            // tail skip: the layer's residency bits
  int nu, ni;
  int np;     // pairs kept (all of them without the tail skip)
  int nskip;  // experts the tail skip left out
};
using SelectShared = SelectSharedT<MOE_ROUND_MAX_ROWS * MOE_ROUND_MAX_TOPK, kSelectWaves>;

// Sorts n keys in registers, largest first: the 5- and 19-comparator networks for 4 and 8 keys
// (both checked on every 0/1 input), odd-even transposition otherwise.
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&key)[N]) {
  auto cx = [&](int i, int j) {
    const uint64_t a = key[i], b = key[j];
    key[i] = a < b ? b : a;
    key[j] = a < b ? a : b;
  };
  if constexpr (N == 8) {
    cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
    cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
    cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
    cx(2, 4); cx(3, 5);
    cx(1, 4); cx(3, 6);
    cx(1, 2); cx(3, 4); cx(5, 6);
  } else if constexpr (N == 4) {
    cx(0, 1); cx(2, 3);
    cx(0, 2); cx(1, 3);
    cx(1, 2);
  } else {
#pragma unroll
    for (int pass = 0; pass < N; ++pass)
#pragma unroll
      for (int i = pass & 1; i + 1 < N; i += 2) cx(i, i + 1);
  }
}

// Top-k of one row on one wave (of NW waves in the block). Each lane sorts its NPL (logit, id) keys
// once and parks them in LDS, keeping its largest (the head) and the next one in registers. Each of
// the k rounds then takes the largest head over the wave: a wave max of the heads' high words (sign,
// exponent and 20 mantissa bits), and only when several lanes hold that high word (a ballot tells)
// a second one over their low words (the low bits carry the id, so the winner is unique). The
// winner lane's next key becomes its head and every lane re-reads its next key from LDS, a read
// whose latency the following round hides. Lane j keeps the j-th id. The exact fp64 logits of the
// k ids come from their owner lanes once, after the rounds, for the softmax over the k selected.
// With E even the row is read 16 bytes per lane (slot i of lane l holds expert 128 (i / 2) + 2 l +
// i % 2), else 8 bytes (expert l + 64 i). Lane j < k ends with rank j's id and routing weight.
template <int NPL, int NW>
__device__ __forceinline__ void topk_row(const double* zrow, int E, int k, int& id_out, float& p_out,
                                         bool need_p = true) {
  // Per wave: the lanes' sorted keys by rank (row r holds every lane's r-th largest), then two
  // rows of zeros, below every real key, for lanes that run out.
  __shared__ uint64_t lst[NW][NPL + 2][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr bool kPairs = NPL % 2 == 0;
  const bool paired = kPairs && (E & 1) == 0;
  double z[NPL];
  uint64_t key[NPL];
  if (paired) {
    const double2* z2 = reinterpret_cast<const double2*>(zrow);
    const int n2 = E >> 1;
#pragma unroll
    for (int i = 0; i < NPL / 2; ++i) {
      const double2 v = z2[min(lane + 64 * i, n2 - 1)];  // all loads issued together
      z[2 * i] = v.x;
      z[2 * i + 1] = v.y;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = 128 * (i >> 1) + 2 * lane + (i & 1);
      key[i] = logit_key(z[i], e) & (e < E ? ~0ull : 0ull);  // 0 is below every real key
    }
  } else {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      z[i] = zrow[min(e, E - 1)];
      key[i] = logit_key(z[i], e) & (e < E ? ~0ull : 0ull);
    }
  }
  sort_desc<NPL>(key);
  MOE_LDS uint64_t* mine = (MOE_LDS uint64_t*)&lst[wave][0][lane];  // rank r at mine[64 r]
#pragma unroll
  for (int i = 1; i < NPL; ++i) mine[64 * i] = key[i];
  mine[64 * NPL] = 0ull;
  mine[64 * (NPL + 1)] = 0ull;
  uint64_t head = key[0];
  uint64_t nxt = NPL > 1 ? key[NPL > 1 ? 1 : 0] : 0ull;
  int c = 1;  // rank of nxt in this lane's list
  int myid = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t hh = static_cast<uint32_t>(head >> 32), hl = static_cast<uint32_t>(head);
    const uint32_t mhi = wave_max_u32(hh);
    const uint64_t tie = __ballot(hh == mhi);
    int w;
    if (__popcll(tie) == 1) {
      w = __builtin_ctzll(tie);
    } else {
      const uint32_t mlo = wave_max_u32(hh == mhi ? hl : 0u);
      w = __builtin_ctzll(__ballot(hh == mhi && hl == mlo));
    }
    const int e = key_expert(__builtin_amdgcn_readlane(hl, w));
    if (lane == j) myid = e;
    const bool pop = lane == w;
    head = pop ? nxt : head;
    c += pop ? 1 : 0;  // at most NPL + 1: a lane whose head is 0 never wins again
    nxt = mine[64 * c];
  }
  id_out = myid;
  p_out = 0.f;
  if (!need_p) return;  // callers that use only the ids skip the softmax
  // Lane j < k: the logit of its id, from the register slot and lane that loaded it, through the
  // wave's list rows (free now; LDS operations of one wave complete in order).
  const int own = paired ? (myid & 127) >> 1 : myid & 63;
  const int slot = paired ? 2 * (myid >> 7) + (myid & 1) : myid >> 6;
#pragma unroll
  for (int i = 0; i < NPL; ++i) mine[64 * i] = __builtin_bit_cast(uint64_t, z[i]);
  const double myz = __builtin_bit_cast(double, ((MOE_LDS uint64_t*)&lst[wave][0][0])[64 * slot + own]);
  const double z0 = __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, myz), 0));
  const double ej = lane < k ? exp(myz - z0) : 0.0;  // rank 0 holds the largest selected logit
  const double sum = wave_sum_f64(ej);
  p_out = static_cast<float>(ej / sum);
}

// Top-k of row t into the selection state in LDS.
template <int NPL, int NW, typename SS>
__device__ __forceinline__ void select_row(const Args& a, SS& s, int t, bool need_p) {
  const int lane = threadIdx.x & 63;
  const int k = a.k;
  const int slot = t * k + lane;
  int id;
  float p;
  topk_row<NPL, NW>(a.logits + static_cast<size_t>(t) * a.E, a.E, k, id, p, need_p);
  if (lane < k) {
    s.sel[slot] = id;
    s.p[slot] = p;
  }
}

// Tail skip: is the pair (rank j, expert e) a tail pair, i.e. e is missed (its residency bit is
// clear) and j is at or past the skip rank? A missed expert is skipped when all its pairs are.
template <typename SS>
__device__ __forceinline__ bool tail_pair(const Args& a, const SS& s, int j, int e) {
  return j >= a.skip_j && !((s.res[e >> 5] >> (e & 31)) & 1u);
}

// The union of a round by the whole block (any number of pairs; s.mask zero, s.sel written; with
// `skip`, s.tmask zero and s.res written). Experts the tail skip leaves out get no pairs, slot -1.
template <int NT, typename SS>
__device__ __forceinline__ void union_block(const Args& a, SS& s, int npairs, bool skip, int& nu, int& ni) {
  constexpr int NWMIN = NT / 64;  // the caller's waves (sizes the per-wave arrays)
  constexpr int nt = NT, nw = NT / 64;  // the launched block size (not read from the dispatch)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E, k = a.k;
  for (int idx = tid; idx < npairs; idx += nt) {
    const int e = s.sel[idx], t = idx / k;
    const bool tail = skip && tail_pair(a, s, idx - t * k, e);
    atomicOr(tail ? &s.tmask[e] : &s.mask[e], 1ull << t);
  }
  __syncthreads();

  // The union and its prefix sums, with ballots instead of a shuffle scan. Chunk ch of 64
  // consecutive experts (ch = q * nw + wave) gives each expert lane its rank among the chunk's
  // chosen experts, and the sums below it of the row counts and of the work-item counts (an
  // expert's rows split into items of at most a.rg), bit plane by bit plane: mbcnt of the ballot of
  // each bit. Chunk totals meet once in LDS for the exclusive prefix over chunks.
  constexpr int NCH = MOE_ROUND_MAX_EXPERTS / 64;
  constexpr int CPW = (NCH + NWMIN - 1) / NWMIN;  // chunks per wave (at most)
  const int rg = a.rg;
  const int cbits = 32 - __clz(T);                  // bits of a row count (at most T)
  const int gbits = 32 - __clz((T + rg - 1) / rg);  // bits of an item count
  int cnt[CPW], ngs[CPW], uin[CPW], cin[CPW], gin[CPW];
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int ch = q * nw + wave, e = ch * 64 + lane;
    const bool valid = ch < NCH && e < E;
    const int ec = min(e, MOE_ROUND_MAX_EXPERTS - 1);
    uint64_t m = valid ? s.mask[ec] : 0ull;
    bool skipped = false;
    if (skip && valid) {  // an expert with a kept pair keeps its tail pairs too; one without is skipped
      const uint64_t tm = s.tmask[ec];
      if (m != 0ull) {
        m |= tm;
        s.mask[ec] = m;
      } else {
        skipped = tm != 0ull;
      }
    }
    const int c = __popcll(m);
    cnt[q] = c;
    ngs[q] = (c + rg - 1) / rg;
    const uint64_t chosen = __ballot(c > 0);
    uin[q] = mbcnt64(chosen);
    uint64_t tot = static_cast<uint64_t>(__popcll(chosen));
    int ci = 0, gi = 0;
    for (int b = 0; b < cbits; ++b) {
      const uint64_t mb = __ballot((c >> b) & 1);
      ci += mbcnt64(mb) << b;
      tot += static_cast<uint64_t>(__popcll(mb)) << (16 + b);
    }
    for (int b = 0; b < gbits; ++b) {
      const uint64_t mb = __ballot((ngs[q] >> b) & 1);
      gi += mbcnt64(mb) << b;
      tot += static_cast<uint64_t>(__popcll(mb)) << (32 + b);
    }
    tot += static_cast<uint64_t>(__popcll(__ballot(skipped))) << 48;
    cin[q] = ci;
    gin[q] = gi;
    if (lane == 0 && ch < NCH) s.ctot[ch] = tot;  // chosen | rows << 16 | items << 32 | skipped << 48
  }
  __syncthreads();
  uint64_t all = 0, pre[CPW];
#pragma unroll
  for (int q = 0; q < CPW; ++q) pre[q] = 0;
#pragma unroll
  for (int c2 = 0; c2 < NCH; ++c2) {
    const uint64_t v = s.ctot[c2];
    all += v;
#pragma unroll
    for (int q = 0; q < CPW; ++q)
      if (c2 < q * nw + wave) pre[q] += v;
  }
  nu = min(static_cast<int>(all & 0xFFFF), a.Ucap);
  ni = min(static_cast<int>((all >> 32) & 0xFFFF), a.Icap);
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int e = (q * nw + wave) * 64 + lane;
    if (cnt[q] > 0) {
      const int u = static_cast<int>(pre[q] & 0xFFFF) + uin[q];
      const int io = static_cast<int>((pre[q] >> 32) & 0xFFFF) + gin[q];
      s.uidx[e] = u;
      s.uniq[u] = e;
      s.offs[u] = static_cast<int>((pre[q] >> 16) & 0xFFFF) + cin[q];
      s.ioffs[u] = io;
      for (int g2 = 0; g2 < ngs[q]; ++g2) s.item_u[io + g2] = u;
    }
  }
  if (tid == 0) {
    const int kept = static_cast<int>((all >> 16) & 0xFFFF);
    s.nu = nu;
    s.ni = ni;
    s.np = kept;
    s.nskip = static_cast<int>((all >> 48) & 0xFFFF);
    s.offs[nu] = kept;
  }
  __syncthreads();
  for (int idx = tid; idx < npairs; idx += nt) {
    const int t = idx / k, j = idx - t * k;
    const int e = s.sel[idx];
    const uint64_t m = s.mask[e];
    if (!((m >> t) & 1ull)) {  // a pair of a skipped expert
      s.slot[idx] = -1;
      continue;
    }
    const int pos = s.offs[s.uidx[e]] + __popcll(m & ((1ull << t) - 1ull));
    s.pairs[pos] = t | (j << 8);
    s.slot[idx] = pos;
  }
  __syncthreads();
}

// The value of lane (lane ^ stride), stride a power of two below 64 (constant after unrolling), on
// VALU only: xor 4 and xor 8 are two DPP moves each (lane ^ 3 then the 8-lane mirror lane ^ 7;
// lane ^ 7 then the 16-lane mirror lane ^ 15), the upper strides the permlane swaps.
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v, int stride) {
  constexpr int kDppRev4 = 0x1B;  // quad_perm [3,2,1,0]: lane ^ 3
  switch (stride) {
    case 1: return dpp_u32<kDppXor1>(v);
    case 2: return dpp_u32<kDppXor2>(v);
    case 4: return dpp_u32<kDppHalfMirror>(dpp_u32<kDppRev4>(v));
    case 8: return dpp_u32<kDppMirror>(dpp_u32<kDppHalfMirror>(v));
    case 16: return swap_partner_u32<false>(v);
    default: return swap_partner_u32<true>(v);
  }
}
__device__ __forceinline__ uint64_t low_bits(int n) { return n >= 64 ? ~0ull : ((1ull << n) - 1ull); }

// floor(n / d) for 0 <= n < 128 and 1 <= d <= 64 through one fp32 reciprocal: n / d is at least
// 1 / (2 d) away from the next integer, far beyond the reciprocal's error.
__device__ __forceinline__ int small_div(int n, float rcp_d) {
  return static_cast<int>((static_cast<float>(n) + 0.5f) * rcp_d);
}

// The union of a round of at most 64 (row, rank) pairs by one wave (s.sel written; with `skip`,
// s.res written), the same worklist as union_block: lane i takes pair i = t k + j as the key
// expert | i, a bitonic network sorts the 64 keys across the lanes in registers (ascending, so by
// expert, then row, then rank), and runs of equal experts become the unique experts, their
// offsets and work items through ballots: the kept pairs at run positions 0, rg, 2 rg, ... start
// the work items. With the tail skip a run is kept when any of its pairs is not a tail pair.
template <typename SS>
__device__ __forceinline__ void union_wave(const Args& a, SS& s, int npairs, bool skip) {
  const int lane = threadIdx.x & 63;
  const int k = a.k, rg = a.rg;
  uint32_t key = 0xFFFFFFFFu;  // past the pairs: sorts last
  if (lane < npairs) key = (static_cast<uint32_t>(s.sel[lane]) << 6) | static_cast<uint32_t>(lane);
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
    // With at most 32 pairs, lanes 32-63 hold only the padding key once the 32-lane halves are
    // sorted (the lower half ascending), so the last merge would change nothing.
    if (size == 64 && npairs <= 32) break;
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint32_t other = lane_xor_u32(key, stride);
      const bool keep_min = ((lane & stride) == 0) == ((lane & size) == 0);
      key = keep_min ? min(key, other) : max(key, other);
    }
  }
  const bool valid = lane < npairs;
  const int e = static_cast<int>(key >> 6), pi = static_cast<int>(key & 63);
  const int t = small_div(pi, __builtin_amdgcn_rcpf(static_cast<float>(k))), j = pi - t * k;
  constexpr int kDppWaveShr1 = 0x138;  // lane i takes lane i - 1 (lane 0 keeps `old`)
  const uint32_t prev = __builtin_amdgcn_update_dpp(0xFFFFFFFFu, key, kDppWaveShr1, 0xF, 0xF, false);
  const bool head = valid && (lane == 0 || (prev >> 6) != (key >> 6));
  const uint64_t heads = __ballot(head);
  const int first = 63 - __builtin_clzll((heads & low_bits(lane + 1)) | 1ull);  // start of this lane's run
  bool kept = valid;
  if (skip) {
    const uint64_t above = heads & ~low_bits(lane + 1);
    const int next = above ? __builtin_ctzll(above) : npairs;  // end of this lane's run
    const bool nt = valid && !tail_pair(a, s, j, e);
    const uint64_t nts = __ballot(nt);
    kept = valid && (nts & low_bits(next) & ~low_bits(first)) != 0ull;
  }
  const uint64_t keptm = __ballot(kept);
  const bool khead = kept && head;
  const uint64_t kheads = __ballot(khead);
  const int below = mbcnt64(keptm);                      // slot among the kept pairs
  const int u = mbcnt64(kheads) + (khead ? 1 : 0) - 1;   // this lane's expert among the kept ones
  const int pos = lane - first;
  const bool starter = kept && pos == small_div(pos, __builtin_amdgcn_rcpf(static_cast<float>(rg))) * rg;
  const uint64_t starters = __ballot(starter);
  const int item = mbcnt64(starters);
  if (khead) {
    s.uniq[u] = e;
    s.offs[u] = below;
    s.ioffs[u] = item;
  }
  if (starter) s.item_u[item] = u;
  if (valid) {
    s.slot[pi] = kept ? below : -1;
    if (kept) s.pairs[below] = t | (j << 8);
  }
  if (lane == 0) {
    const int nu = static_cast<int>(__popcll(kheads)), kept_n = static_cast<int>(__popcll(keptm));
    s.nu = min(nu, a.Ucap);
    s.ni = min(static_cast<int>(__popcll(starters)), a.Icap);
    s.np = kept_n;
    s.nskip = static_cast<int>(__popcll(heads)) - nu;
    s.offs[min(nu, a.Ucap)] = kept_n;
  }
}

// The selection of one round by one block of NT threads: per-row top-k and softmax, the union of
// the rows' experts, the counting sort of the (row, rank) pairs by expert and the work items (an
// expert and at most a.rg of its rows). Results stay in `s`; with `publish` the block also writes
// the per-item records, the unique list, pair table and pair weights, and the caller's ids and
// routing weights. Deterministic: every block computing it gets the same result.
// PRESEL: the rows' top-k already ran (topk_rows_kernel); their ids and weights are read from
// a.tsel / a.tp instead of computed here.
template <int NPL, int NT, bool ONE_ROW = false, bool PRESEL = false, typename SS>
__device__ __forceinline__ void select_block(const Args& a, int layer, SS& s, bool publish) {
  constexpr int nt = NT, nw = NT / 64;  // the launched block size (not read from the dispatch)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E, k = a.k, npairs = T * k;

  // Tail skip: the layer's residency words, loaded before the top-k (which hides their latency) and
  // put into LDS after it.
  const bool skip = a.resident != nullptr && a.skip_j < k;
  const int nres = (E + 31) >> 5;
  uint32_t resw = 0u;
  if (skip && tid < nres) resw = a.resident[tid];

  int nu, ni;
  if constexpr (ONE_ROW) {
    // Rounds of one row (callers that only run at T == 1): the union is its k ids, one row each,
    // so one wave ranks them (ascending expert id) and writes the worklist directly. With the tail
    // skip an expert is skipped exactly when its one pair is a tail pair.
    if (wave == 0) {
      select_row<NPL, NT / 64>(a, s, 0, publish);
      const int j = min(lane, k - 1);
      const int id = s.sel[j];
      bool keep = lane < k;
      if (skip) {
        const uint32_t word = static_cast<uint32_t>(__shfl(static_cast<int>(resw), id >> 5, 64));
        keep = keep && (j < a.skip_j || ((word >> (id & 31)) & 1u));
      }
      if (lane < k && !keep) s.slot[lane] = -1;
      // The kept (expert, rank) pairs sorted by expert across lanes 0-15 (a bitonic network of
      // 16; the ids of one row are distinct): lane u then holds the u-th unique expert.
      uint32_t key = keep ? (static_cast<uint32_t>(id) << 4) | static_cast<uint32_t>(j) : 0xFFFFFFFFu;
#pragma unroll
      for (int size = 2; size <= 16; size <<= 1) {
        if (size == 16 && k <= 8) break;  // lanes 8-15 hold only the padding key: already in place
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          const uint32_t other = lane_xor_u32(key, stride);
          const bool keep_min = ((lane & stride) == 0) == ((lane & size) == 0);
          key = keep_min ? min(key, other) : max(key, other);
        }
      }
      const int nk = static_cast<int>(__popcll(__ballot(keep)));
      if (lane < nk) {
        const int u = lane, e = static_cast<int>(key >> 4), jr = static_cast<int>(key & 15);
        s.slot[jr] = u;
        s.uniq[u] = e;
        s.offs[u] = u;
        s.ioffs[u] = u;
        s.item_u[u] = u;
        s.pairs[u] = jr << 8;  // row 0, rank jr
      }
      if (lane == 0) {
        s.nu = min(nk, a.Ucap);
        s.ni = min(nk, a.Icap);
        s.np = nk;
        s.nskip = k - nk;
        s.offs[nk] = nk;
      }
    }
    __syncthreads();
    nu = s.nu;
    ni = s.ni;
  } else {
    const bool small = npairs <= 64;  // the one-wave union (union_wave), else the block's
    if (!small)
      for (int e = tid; e < E; e += nt) {
        s.mask[e] = 0ull;
        if (skip) s.tmask[e] = 0ull;
      }
    if constexpr (PRESEL) {
      for (int idx = tid; idx < npairs; idx += nt) {
        s.sel[idx] = min(max(a.tsel[idx], 0), E - 1);
        s.p[idx] = a.tp[idx];
      }
    } else {
      for (int t = wave; t < T; t += nw) select_row<NPL, NT / 64>(a, s, t, publish);
    }
    if (skip && tid < nres) s.res[tid] = resw;
    __syncthreads();
    if (small) {
      if (wave == 0) union_wave(a, s, npairs, skip);
      __syncthreads();
      nu = s.nu;
      ni = s.ni;
    } else {
      union_block<NT>(a, s, npairs, skip, nu, ni);
    }
  }
  if (!publish) return;

  // Publish: per-item records, the unique list and pair table, the caller's ids / routing weights.
  const Ingress in = get_ingress(a);
  int32_t* rec = a.rec + static_cast<size_t>(layer) * a.Icap * kRecWords;
  int32_t* uniq = a.uniq + static_cast<size_t>(layer) * a.Ucap;
  int32_t* offs = a.offs + static_cast<size_t>(layer) * (a.Ucap + 1);
  int32_t* pairs = a.pairs + static_cast<size_t>(layer) * a.Pcap;
  float* pw = a.pair_w + static_cast<size_t>(layer) * a.Pcap;
  // One thread per item writes its record: the four header words and the row words an item of at
  // most a.rg rows can use (readers never look at rows past np, so the rest are not written).
  const int nrw = (a.rg + 3) / 4;
  for (int it = tid; it < ni; it += nt) {
    const int uu = s.item_u[it];
    const int p0 = s.offs[uu] + (it - s.ioffs[uu]) * a.rg;
    const int np = min(a.rg, s.offs[uu + 1] - p0);
    int32_t* r = rec + static_cast<size_t>(it) * kRecWords;
    r[0] = s.uniq[uu];
    r[1] = p0;
    r[2] = np;
    r[3] = ni;
    for (int wd = 0; wd < nrw; ++wd) {
      int v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (4 * wd + b < np) v |= (s.pairs[p0 + 4 * wd + b] & 0xFF) << (8 * b);
      r[kRecRowWord + wd] = v;
    }
  }
  // Record 0 carries the item count every GEMV block reads; a round whose pairs the tail skip left
  // out entirely has no item to write it, so it is written here.
  if (tid == 0 && ni == 0) rec[3] = 0;
  for (int i = tid; i < nu; i += nt) uniq[i] = s.uniq[i];
  for (int i = tid; i <= nu; i += nt) offs[i] = s.offs[i];
  int32_t* slot_of = a.slot_of + static_cast<size_t>(layer) * a.Pcap;
  const int kept = s.np;
  for (int i = tid; i < kept; i += nt) {  // the worklist's pair slots
    const int pr = s.pairs[i];
    pairs[i] = pr;
    pw[i] = s.p[(pr & 0xFF) * k + (pr >> 8)];
  }
  for (int i = tid; i < npairs; i += nt) {  // by (row, rank): i = t*k + j
    slot_of[i] = s.slot[i];
    const size_t o = static_cast<size_t>(layer) * npairs + i;  // [L][T][k]
    if (in.ids) gptr(in.ids)[o] = s.sel[i];
    if (in.route_w) gptr(in.route_w)[o] = s.p[i];
  }
  if (tid == 0) {
    a.n_unique[layer] = nu;
    if (a.n_skipped) a.n_skipped[layer] = s.nskip;
  }
}

template <int NPL, bool PRESEL = false>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(Args a, int layer) {
  __shared__ SelectShared s;
  select_block<NPL, kSelectThreads, false, PRESEL>(a, layer, s, true);
}

// Wide rounds: the rows' top-k on many CUs, one wave per row (the one-block selection's top-k is
// bound by that block's one CU from about 16 rows on), into a.tsel / a.tp for the select kernel.
// Grid: ceil(T / 4) x 256 threads.
template <int NPL>
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(Args a, int layer) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= a.T) return;  // whole waves leave together
  const int k = a.k;
  int id;
  float p;
  topk_row<NPL, kWaves>(a.logits + static_cast<size_t>(t) * a.E, a.E, k, id, p);
  if (lane < k) {
    a.tsel[t * k + lane] = id;
    a.tp[t * k + lane] = p;
  }
}

// Every GEMV block reads its work item's record and record 0 (whose item count is always valid)
// in one round trip; values are clamped so nothing read back can index out of bounds. An item is
// one expert and at most a.rg of the rows routed to it (pair slots p0 .. p0 + np - 1).
struct ExpertWork {
  int e, p0, np, nu;  // nu: number of items of the layer
  int rows[MOE_ROUND_MAX_ROWS / 4];  // packed row ids, 4 per word (from a record)
  const MOE_LDS int* lrows;  // or, with the selection in LDS: the item's pair entries (t | j << 8) there
};

__device__ __forceinline__ ExpertWork load_work(const Args& a, int layer, int u) {
  const int32_t* rec = a.rec + static_cast<size_t>(layer) * a.Icap * kRecWords;
  const int32_t* r = rec + static_cast<size_t>(min(u, a.Icap - 1)) * kRecWords;
  ExpertWork w;
  const int nu = rec[3];
  w.e = r[0];
  w.p0 = r[1];
  w.np = r[2];
#pragma unroll
  for (int i = 0; i < MOE_ROUND_MAX_ROWS / 4; ++i) w.rows[i] = r[kRecRowWord + i];
  const int npairs = a.T * a.k;
  w.lrows = nullptr;
  w.nu = min(max(nu, 0), a.Icap);
  w.e = min(max(w.e, 0), a.E - 1);
  w.p0 = min(max(w.p0, 0), npairs);
  w.np = min(max(w.np, 0), npairs - w.p0);
  return w;
}

// The work item `it` of a selection held in LDS (see select_block). Only the item's expert and pair
// range are read here, so the weight loads can be issued before the item's row ids are fetched;
// work_row reads those from the pair list in LDS when they are used.
template <typename SS>
__device__ __forceinline__ ExpertWork work_from_lds(const Args& a, const SS& s, int it) {
  ExpertWork w;
  it = min(it, max(s.ni - 1, 0));
  const int uu = s.item_u[it];
  w.nu = s.ni;
  w.e = s.uniq[uu];
  w.p0 = s.offs[uu] + (it - s.ioffs[uu]) * a.rg;
  w.np = min(a.rg, s.offs[uu + 1] - w.p0);
  // an LDS pointer, not a generic one: a generic load would also count against the vector-memory
  // counter and so wait for every weight load issued before it
  w.lrows = (const MOE_LDS int*)(s.pairs + w.p0);
  return w;
}

__device__ __forceinline__ int work_row(const ExpertWork& w, int r, int T) {
  if (w.lrows) return min(w.lrows[r] & 0xFF, T - 1);
  // r is wave-uniform; select the packed word without dynamic register indexing
  int word = 0;
#pragma unroll
  for (int i = 0; i < MOE_ROUND_MAX_ROWS / 4; ++i)
    if (i == (r >> 2)) word = w.rows[i];
  return min((word >> (8 * (r & 3))) & 0xFF, T - 1);
}

}  // namespace moe
