// GEMV kernels (gate/up and down) for rows split over 64 lanes; see moe_kernels.h.
#include "moe_kernels.h"

namespace moe {
bool pick_gemv_g64(int NB, int mode, bool up, int sel, KernelFn* fn, int* rows) {
  return pick_nb<64, kFmtQ4B32>(NB, mode, up, sel, fn, rows);
}
}  // namespace moe
