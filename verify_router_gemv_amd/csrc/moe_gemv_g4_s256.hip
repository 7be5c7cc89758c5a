// GEMV kernels (gate/up and down) for rows split over 4 lanes, 4.5-bit super-block weights;
// see moe_kernels.h.
#include "moe_kernels.h"

namespace moe {
bool pick_gemv_g4_s256(int NB, int mode, bool up, int sel, KernelFn* fn, int* rows) {
  return pick_nb<4, kFmtQ4S256>(NB, mode, up, sel, fn, rows);
}
}  // namespace moe
