// All kernels of the round and the launch-shape pickers.
#pragma once

#include "moe_down.h"
#include "moe_gateup.h"
#include "moe_route.h"

namespace moe {

// ------------------------------------------------------------------------------------------
// Kernel selection
// ------------------------------------------------------------------------------------------

using KernelFn = void (*)(Args, int);

constexpr int rows_per_lane_group(int NB) { return NB == 1 ? 4 : (NB == 2 ? 2 : 1); }

template <int G, int NB, int FMT>
struct GemvPick {
  static constexpr int RW = rows_per_lane_group(NB);
  // sel: keys per lane of the fused selection (4: E <= 256, 8: E <= 512), 0: read the records of
  // the selection kernel (always for the staged form).
  static KernelFn gateup(int mode, int sel) {
    if (mode == kGuStaged) return gateup_kernel<G, NB, RW, kGuStaged, 0, FMT>;
    if (mode == kGuOneRow)
      return sel == 4   ? gateup_kernel<G, NB, RW, kGuOneRow, 4, FMT>
             : sel == 8 ? gateup_kernel<G, NB, RW, kGuOneRow, 8, FMT>
                        : gateup_kernel<G, NB, RW, kGuOneRow, 0, FMT>;
    if (mode == kGuRowItems)
      return sel == 4   ? gateup_kernel<G, NB, RW, kGuRowItems, 4, FMT>
             : sel == 8 ? gateup_kernel<G, NB, RW, kGuRowItems, 8, FMT>
                        : gateup_kernel<G, NB, RW, kGuRowItems, 0, FMT>;
    return sel == 4   ? gateup_kernel<G, NB, RW, kGuPairs, 4, FMT>
           : sel == 8 ? gateup_kernel<G, NB, RW, kGuPairs, 8, FMT>
                      : gateup_kernel<G, NB, RW, kGuPairs, 0, FMT>;
  }
  // down: mode 1 the matrix-core tile (where the shape has one), mode 2 half-height blocks (two
  // rows per lane group where there are four, for rounds whose full-height grid is small), mode 3
  // double-height blocks (eight rows per lane group there, for one-row items on large grids).
  static KernelFn down(bool exact, int mode) {
    if constexpr (G == 16 && NB == 1 && RW == 4 && FMT == kFmtQ4B32)
      if (mode == 1) return exact ? down_kernel<G, NB, RW, true, FMT, true> : down_kernel<G, NB, RW, false, FMT, true>;
    if constexpr (RW == 4) {
      if (mode == 2) return exact ? down_kernel<G, NB, 2, true, FMT> : down_kernel<G, NB, 2, false, FMT>;
      if (mode == 3) return exact ? down_kernel<G, NB, 8, true, FMT> : down_kernel<G, NB, 8, false, FMT>;
    }
    return exact ? down_kernel<G, NB, RW, true, FMT> : down_kernel<G, NB, RW, false, FMT>;
  }
  static constexpr int rows_per_block() { return kWaves * RW * (64 / G); }
  static constexpr int rows_per_half_block() { return kWaves * (RW == 4 ? 2 : RW) * (64 / G); }
  static constexpr int rows_per_double_block() { return kWaves * (RW == 4 ? 8 : RW) * (64 / G); }
};

// up: the gate/up kernel of form `mode` (kGuOneRow, kGuRowItems, kGuPairs, kGuStaged) with `sel` keys per lane
// of a folded selection (0: none); otherwise the down kernel, exact mode if sel != 0, with the
// matrix-core tile if mode == 1 (where the shape has one), half-height blocks if mode == 2,
// double-height blocks if mode == 3.
template <int G, int NB, int FMT>
inline bool pick_form(int mode, bool up, int sel, KernelFn* fn, int* rows) {
  *fn = up ? GemvPick<G, NB, FMT>::gateup(mode, sel) : GemvPick<G, NB, FMT>::down(sel != 0, mode);
  *rows = up          ? GemvPick<G, NB, FMT>::rows_per_block()
          : mode == 2 ? GemvPick<G, NB, FMT>::rows_per_half_block()
          : mode == 3 ? GemvPick<G, NB, FMT>::rows_per_double_block()
                      : GemvPick<G, NB, FMT>::rows_per_block();
  return true;
}

template <int G, int FMT>
inline bool pick_nb(int NB, int mode, bool up, int sel, KernelFn* fn, int* rows) {
  switch (NB) {
    case 1: return pick_form<G, 1, FMT>(mode, up, sel, fn, rows);
    case 2: return pick_form<G, 2, FMT>(mode, up, sel, fn, rows);
    case 3: return pick_form<G, 3, FMT>(mode, up, sel, fn, rows);
    case 4: return pick_form<G, 4, FMT>(mode, up, sel, fn, rows);
  }
  return false;
}

// Each (lane split G, weight format) pair is instantiated in its own translation unit
// (moe_gemv_g<G>.hip for the per-32 format, moe_gemv_g<G>_s256.hip for super-blocks) so the library
// builds in parallel.
#define MOE_DECLARE_PICK(NAME) bool NAME(int NB, int mode, bool up, int sel, KernelFn* fn, int* rows);
MOE_DECLARE_PICK(pick_gemv_g4)
MOE_DECLARE_PICK(pick_gemv_g8)
MOE_DECLARE_PICK(pick_gemv_g16)
MOE_DECLARE_PICK(pick_gemv_g32)
MOE_DECLARE_PICK(pick_gemv_g64)
MOE_DECLARE_PICK(pick_gemv_g4_s256)
MOE_DECLARE_PICK(pick_gemv_g8_s256)
MOE_DECLARE_PICK(pick_gemv_g16_s256)
MOE_DECLARE_PICK(pick_gemv_g32_s256)
MOE_DECLARE_PICK(pick_gemv_g64_s256)
#undef MOE_DECLARE_PICK

inline bool pick_gemv(int G, int NB, int mode, bool up, int sel, int fmt, KernelFn* fn, int* rows) {
  if (fmt == kFmtQ4S256) {
    switch (G) {
      case 4: return pick_gemv_g4_s256(NB, mode, up, sel, fn, rows);
      case 8: return pick_gemv_g8_s256(NB, mode, up, sel, fn, rows);
      case 16: return pick_gemv_g16_s256(NB, mode, up, sel, fn, rows);
      case 32: return pick_gemv_g32_s256(NB, mode, up, sel, fn, rows);
      case 64: return pick_gemv_g64_s256(NB, mode, up, sel, fn, rows);
    }
    return false;
  }
  switch (G) {
    case 4: return pick_gemv_g4(NB, mode, up, sel, fn, rows);
    case 8: return pick_gemv_g8(NB, mode, up, sel, fn, rows);
    case 16: return pick_gemv_g16(NB, mode, up, sel, fn, rows);
    case 32: return pick_gemv_g32(NB, mode, up, sel, fn, rows);
    case 64: return pick_gemv_g64(NB, mode, up, sel, fn, rows);
  }
  return false;
}

// Rows per logits block: the round's rows up to 8 (rounded up to 1, 2, 4 or 8), so a block reads
// its router row once for all of them; wider rounds use ceil(T / 8) row chunks.
inline int logits_rows(int T) { return T <= 1 ? 1 : (T <= 2 ? 2 : (T <= 4 ? 4 : 8)); }

template <int TC>
inline KernelFn pick_logits_tc(int H) {
  switch ((H + 1023) / 1024) {
#define MOE_NJ(N) \
  case N: return logits_kernel<N, TC>;
    MOE_NJ(1) MOE_NJ(2) MOE_NJ(3) MOE_NJ(4) MOE_NJ(5) MOE_NJ(6) MOE_NJ(7) MOE_NJ(8)
#undef MOE_NJ
  }
  return nullptr;
}

inline KernelFn pick_logits(int H, int T) {
  switch (logits_rows(T)) {
    case 1: return pick_logits_tc<1>(H);
    case 2: return pick_logits_tc<2>(H);
    case 4: return pick_logits_tc<4>(H);
  }
  return pick_logits_tc<8>(H);
}

// Grid of the logits kernel: E router blocks plus the blocks that write the input's digits.
inline dim3 logits_grid(int E, int H, int T) {
  const int tc = logits_rows(T);
  return dim3(E + (T * H + 255) / 256, (T + tc - 1) / tc);
}

// Keys per lane of the fused selection in the gate/up kernel (E <= 512).
inline int fused_select_keys(int E) { return E <= 256 ? 4 : 8; }

// presel: the round's top-k runs in topk_rows_kernel (pick_topk_rows) before the select kernel.
inline KernelFn pick_select(int E, bool presel) {
  if (E <= 64) return presel ? select_kernel<1, true> : select_kernel<1>;
  if (E <= 128) return presel ? select_kernel<2, true> : select_kernel<2>;
  if (E <= 256) return presel ? select_kernel<4, true> : select_kernel<4>;
  return presel ? select_kernel<8, true> : select_kernel<8>;
}
inline KernelFn pick_topk_rows(int E) {
  if (E <= 64) return topk_rows_kernel<1>;
  if (E <= 128) return topk_rows_kernel<2>;
  if (E <= 256) return topk_rows_kernel<4>;
  return topk_rows_kernel<8>;
}
// Rounds of at least this many rows run the top-k as its own many-block kernel.
constexpr int kSplitTopkRows = 32;

// Rounds of at most this many rows fold the selection into the gate/up kernel: every block
// recomputes it (one block per CU in the many-row forms, each row on a wave of its own), which
// saves a launch, its gap and a dependent load; timed faster than the one-block selection kernel
// up to 15 rows, the most the fused selection state holds (15 rows of 16 ranks).
constexpr int kFusedMaxRows = 15;
// Gate/up blocks of a round with the selection folded in (each loops over its share of the units).
constexpr int kFusedBlocks = 768;
// Down grids of at most this many full-height blocks use half-height blocks; grids of one-row items
// past kDownDoubleMinBlocks (more than the CUs hold at once) use double-height blocks (see make_plan).
constexpr int kDownHalfMaxBlocks = 768;
constexpr int kDownDoubleMinBlocks = 1280;


}  // namespace moe
