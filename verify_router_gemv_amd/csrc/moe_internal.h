// Internal declarations shared by the host translation units of the library (not part of the ABI).
#pragma once
#include <stdint.h>

#include "moe_round.h"

namespace moe {

// Split a reduction length K into G lanes per matrix row and NB 32-weight blocks per lane
// (K/32 = G * NB, G = largest power of two <= 64 dividing K/32, G >= 4, NB <= 4).
bool split_blocks(int K, int* G, int* NB);

moe_status validate_config(const moe_round_config* c);
moe_status validate_layers(const moe_round_config* c, const moe_layer_weights* layers);
moe_status validate_run(const moe_round_config* c, const float* hidden, int32_t T, int32_t k,
                        const float* out, const int32_t* ids, const float* rw);

}  // namespace moe
