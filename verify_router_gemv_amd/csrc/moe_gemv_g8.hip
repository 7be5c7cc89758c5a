// GEMV kernels (gate/up and down) for rows split over 8 lanes; see moe_kernels.h.
#include "moe_kernels.h"

namespace moe {
bool pick_gemv_g8(int NB, int mode, bool up, int sel, KernelFn* fn, int* rows) {
  return pick_nb<8, kFmtQ4B32>(NB, mode, up, sel, fn, rows);
}
}  // namespace moe
