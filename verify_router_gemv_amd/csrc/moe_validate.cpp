// Host-only validation of a moe_round configuration and of the shapes the kernels support.
// Kept free of HIP so that it runs (and is tested) on a machine without a GPU.
#include "moe_internal.h"

namespace moe {

bool split_blocks(int K, int* G, int* NB) {
  if (K <= 0 || K % 32 != 0) return false;
  const int bpr = K / 32;
  if (bpr > 256) return false;
  // An exact split (no idle lane) when there is one: G the largest power of two <= 64 dividing
  // K/32, with G >= 4 and NB <= 4.
  int g = 1;
  while (g < 64 && (bpr % (g * 2)) == 0) g *= 2;
  if (g >= 4 && bpr / g <= 4) {
    *G = g;
    *NB = bpr / g;
    return true;
  }
  // Otherwise the split with the fewest idle block slots (G * NB - K/32, ties to the smaller G):
  // the kernels clamp the idle slots' loads into the row and zero their scale and minimum.
  int best_g = 0, best_nb = 0, best_waste = 1 << 30;
  for (int gg = 4; gg <= 64; gg *= 2) {
    const int nb = (bpr + gg - 1) / gg;
    if (nb > 4) continue;
    const int waste = gg * nb - bpr;
    if (waste < best_waste) {
      best_g = gg;
      best_nb = nb;
      best_waste = waste;
    }
  }
  if (!best_g) return false;
  *G = best_g;
  *NB = best_nb;
  return true;
}

moe_status validate_config(const moe_round_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->abi_version != MOE_ROUND_ABI_VERSION) return MOE_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->inter <= 0 || c->n_experts <= 0 || c->top_k_max <= 0 ||
      c->n_layers <= 0 || c->max_rows <= 0)
    return MOE_ERR_INVALID_ARG;
  if (c->residual != 0 && c->residual != 1) return MOE_ERR_INVALID_ARG;
  if (c->use_graph != 0 && c->use_graph != 1) return MOE_ERR_INVALID_ARG;
  if (!c->residual && c->n_layers != 1) return MOE_ERR_INVALID_ARG;
  if (c->fused_max_rows < -1 || c->fused_max_rows > 15) return MOE_ERR_INVALID_ARG;
  if (c->rows_per_item < 0 || c->rows_per_item > MOE_ROUND_MAX_ROWS) return MOE_ERR_INVALID_ARG;
  if (c->mfma_min_rows < -1 || c->mfma_min_rows > MOE_ROUND_MAX_ROWS) return MOE_ERR_INVALID_ARG;
  if (c->exact != 0 && c->exact != 1) return MOE_ERR_INVALID_ARG;
  if (c->weight_format != MOE_WEIGHT_Q4B32 && c->weight_format != MOE_WEIGHT_Q4S256) return MOE_ERR_INVALID_ARG;
  if (c->prefetch != 0 && c->prefetch != 1) return MOE_ERR_INVALID_ARG;
  if (c->record_layers != 0 && c->record_layers != 1) return MOE_ERR_INVALID_ARG;
  if (c->expert_table != 0 && c->expert_table != 1) return MOE_ERR_INVALID_ARG;
  if (c->tail_skip_rank < 0 || c->tail_skip_rank > MOE_ROUND_MAX_TOPK + 1) return MOE_ERR_INVALID_ARG;
  if (c->top_k_max > c->n_experts) return MOE_ERR_INVALID_ARG;
  if (c->max_rows > MOE_ROUND_MAX_PREFILL_ROWS) return MOE_ERR_UNSUPPORTED;
  if (c->n_experts > MOE_ROUND_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (c->top_k_max > MOE_ROUND_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (c->hidden % 256 != 0 || c->hidden > 8192) return MOE_ERR_UNSUPPORTED;
  int g, nb;
  if (!split_blocks(c->hidden, &g, &nb)) return MOE_ERR_UNSUPPORTED;
  if (!split_blocks(c->inter, &g, &nb)) return MOE_ERR_UNSUPPORTED;
  if (c->n_layers > 4096) return MOE_ERR_UNSUPPORTED;
  if (c->weight_format == MOE_WEIGHT_Q4S256 && c->inter % 256 != 0) return MOE_ERR_UNSUPPORTED;
  // Prefill GEMMs step through the reduction four 32-blocks at a time and tile I by 64 rows.
  if (c->max_rows > MOE_ROUND_MAX_ROWS && c->inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
  // The expert table and the tail skip are decode/verify features (the prefill GEMMs address the
  // contiguous expert arrays and sort every pair).
  if (c->max_rows > MOE_ROUND_MAX_ROWS && (c->expert_table || c->tail_skip_rank)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status validate_layers(const moe_round_config* c, const moe_layer_weights* layers) {
  if (!layers) return MOE_ERR_INVALID_ARG;
  for (int l = 0; l < c->n_layers; ++l) {
    const moe_layer_weights& w = layers[l];
    if (!w.router_w || !aligned16(w.router_w)) return MOE_ERR_INVALID_ARG;
    if (w.router_bias && (reinterpret_cast<uintptr_t>(w.router_bias) & 3u)) return MOE_ERR_INVALID_ARG;
    if (c->expert_table) {  // the experts come from the bound table: these must be unset
      if (w.gate_q || w.gate_sm || w.up_q || w.up_sm || w.down_q || w.down_sm) return MOE_ERR_INVALID_ARG;
      continue;
    }
    if (!w.gate_q || !w.gate_sm || !w.up_q || !w.up_sm || !w.down_q || !w.down_sm)
      return MOE_ERR_INVALID_ARG;
    if (!aligned16(w.gate_q) || !aligned16(w.up_q) || !aligned16(w.down_q) || !aligned16(w.gate_sm) ||
        !aligned16(w.up_sm) || !aligned16(w.down_sm))
      return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

moe_status validate_run(const moe_round_config* c, const float* hidden, int32_t T, int32_t k,
                        const float* out, const int32_t* ids, const float* rw) {
  if (T < 0 || T > c->max_rows) return MOE_ERR_INVALID_ARG;
  if (k < 1 || k > c->top_k_max) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;  // an empty round: no buffer is touched
  if (!hidden || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(hidden) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  if ((ids && (reinterpret_cast<uintptr_t>(ids) & 3u)) || (rw && (reinterpret_cast<uintptr_t>(rw) & 3u)))
    return MOE_ERR_INVALID_ARG;
  // hidden may be out itself (the round then overwrites its input), but not a shifted view of it.
  const uintptr_t bytes = static_cast<uintptr_t>(T) * c->hidden * sizeof(float);
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(hidden), a1 = reinterpret_cast<uintptr_t>(out);
  if (a0 != a1 && a0 < a1 + bytes && a1 < a0 + bytes) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace moe

extern "C" moe_status moe_round_validate_config(const moe_round_config* cfg) {
  return moe::validate_config(cfg);
}

extern "C" const char* moe_round_strerror(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "shape outside the supported set";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_OOM: return "out of device memory";
    case MOE_ERR_STATE: return "call out of order";
    default: return "unknown status";
  }
}
