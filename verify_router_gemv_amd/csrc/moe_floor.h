// Measurement kernels: the byte floor of a round and a plain streaming read.
//
// The byte floor replays only the weight reads of a round: per layer one launch reads the router
// matrix, one the gate and up codes and scale/min words of the layer's unique experts, one their down
// codes and scale/min words, at the addresses the round read, with nothing else (no routing, no
// arithmetic beyond folding the loaded words together). It is the time a round with that many
// dependent launches cannot beat while it moves those bytes (the infero README, "Where the time goes":
// a decode-floor program that replays exactly a step's matrix-vector reads). The streaming read is
// the same kernel over one contiguous buffer in one launch: the same-session control for the chip's
// read rate at that size ("How AlphaInfer makes local decoding fast", section 7, rule 2: always run
// a same-session control).
#pragma once

#include "moe_common.h"

namespace moe {

constexpr int kFloorLoads = 8;                              // 16-byte loads per thread per chunk
constexpr int kFloorChunk = kThreads * kFloorLoads * 16;    // 32 KB per block and chunk
constexpr int kFloorMaxBlocks = 4096;

// One byte range per listed expert: [base + e * stride, base + e * stride + bytes). Bytes and
// stride are multiples of 16 and base is 16-byte aligned.
struct FloorRange {
  const uint8_t* base;
  int64_t stride;
  int64_t bytes;
};

struct FloorArgs {
  FloorRange r[4];
  int nr;
  int chunks_per_expert;      // sum over ranges of ceil(bytes / kFloorChunk)
  const int32_t* uniq;        // device list of the experts to read, or null: expert 0 only
  const int32_t* n_unique;    // device count of that list (null with uniq null)
  int ucap;                   // entries the list can hold (clamp)
  int emax;                   // largest expert id (clamp)
  uint32_t magic;             // a word the folded loads are compared with, so they stay live
  uint32_t* sink;             // [kFloorMaxBlocks]: written only when the fold equals magic
};

__global__ __launch_bounds__(kThreads) void floor_read_kernel(FloorArgs a) {
  const int tid = threadIdx.x;
  const int nu = a.uniq ? min(max(*a.n_unique, 0), a.ucap) : 1;
  const int units = nu * a.chunks_per_expert;
  uint32_t fold = 0;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int ui = u / a.chunks_per_expert;
    int c = u - ui * a.chunks_per_expert;
    const int e = a.uniq ? min(max(a.uniq[ui], 0), a.emax) : 0;
    int ri = 0;
    int64_t nch = (a.r[0].bytes + kFloorChunk - 1) / kFloorChunk;
    while (ri + 1 < a.nr && c >= nch) {  // the range holding chunk c (at most four)
      c -= static_cast<int>(nch);
      ++ri;
      nch = (a.r[ri].bytes + kFloorChunk - 1) / kFloorChunk;
    }
    const FloorRange rg = a.r[ri];
    const uint8_t* base = rg.base + static_cast<int64_t>(e) * rg.stride;
    uint4 v[kFloorLoads];
#pragma unroll
    for (int i = 0; i < kFloorLoads; ++i) {
      const int64_t off = static_cast<int64_t>(c) * kFloorChunk + static_cast<int64_t>(i * kThreads + tid) * 16;
      v[i] = load_stream_u4(base + min(off, rg.bytes - 16));  // past the range: its last 16 bytes again
    }
#pragma unroll
    for (int i = 0; i < kFloorLoads; ++i) fold ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  if (fold == a.magic) a.sink[blockIdx.x & (kFloorMaxBlocks - 1)] = fold;
}

}  // namespace moe
