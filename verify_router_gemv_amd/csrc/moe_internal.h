// Internal declarations shared by the host translation units of the library (not part of the ABI).
#pragma once
#include <stdint.h>

#include "moe_round.h"

namespace moe {

// Split a reduction length K (a multiple of 32, K/32 <= 256) into G lanes per matrix row and NB
// 32-weight blocks per lane, G in {4..64} a power of two, NB <= 4, G * NB >= K/32: the exact split
// when one exists, else the one with the fewest idle block slots (the kernels mask those).
bool split_blocks(int K, int* G, int* NB);

moe_status validate_config(const moe_round_config* c);
moe_status validate_layers(const moe_round_config* c, const moe_layer_weights* layers);
moe_status validate_run(const moe_round_config* c, const float* hidden, int32_t T, int32_t k,
                        const float* out, const int32_t* ids, const float* rw);

}  // namespace moe
