// Host-side logic of the Gemma attention library: configuration checks, layer
// resolution and launch plans.  Plain C++ (no HIP types), so it builds and is
// tested with an ordinary host compiler.
#pragma once

#include <cstddef>
#include <cstdint>

#include "gemma_attn.h"

namespace ga {

// Whole-config validation shared by every entry point.
int validate_config(const gemma_attn_config* cfg);

// Layer resolution (the integer logic of the path, bit-exact).
int resolve_layer(const gemma_attn_config* cfg, int32_t layer_idx, gemma_attn_layer* out);

// Prologue: D must be a power of two in [8, 512] (one row = D/8 lanes of a wave).
bool prologue_dim_supported(int32_t d);

// Prefill / decode instantiations.
bool attn_dim_supported(int32_t d);
bool attn_group_supported(int32_t g);

// Split-KV decode plan: keys of one (sequence, KV head) are cut into n_split
// chunks of `chunk` keys (a power of two, >= 256), counted from the first key
// the sequence reads.  `span_max` is the longest key range one sequence can
// read: min(W + q_len - 1, max_ctx) on local layers (q_len query tokens at the
// end of the context), max_ctx on global layers.
struct DecodePlan {
  int32_t chunk;
  int32_t n_split;
  int32_t span_max;
};
DecodePlan decode_plan(const gemma_attn_layer& L, int32_t num_heads, int32_t batch, int32_t max_ctx, int32_t q_len);

// Workspace layout: o partials fp32 [B, q_len, Hq, n_split, D], then m and l
// fp32 [B, q_len, Hq, n_split] each; every region starts on a 256-byte boundary.
struct DecodeWorkspace {
  size_t o_off, m_off, l_off, total;
};
DecodeWorkspace decode_workspace(const gemma_attn_layer& L, int32_t num_heads, int32_t batch, int32_t q_len,
                                 const DecodePlan& p);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace ga
