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

// The parts of the device that the launch plans depend on.  MI355X in its
// single-partition mode has 256 CUs in 8 XCDs and 160 KB of LDS per CU; a
// partitioned device reports fewer CUs and XCDs.
struct DeviceShape {
  int32_t cus;          // compute units
  int32_t lds_per_cu;   // bytes of LDS per compute unit
  int32_t xcds;         // XCDs (separate L2 domains) the dispatcher deals workgroups over
};
constexpr DeviceShape kMI355X{256, 160 * 1024, 8};

// Split-KV decode plan.  The keys every sequence reads are laid end to end
// (on the device, from ctx_len) and each (KV head, 16-column block) row of
// the grid gets n_wg workgroups that take equal consecutive ranges of that
// line.  n_wg targets one round of workgroups on the device's CUs (workgroups
// per CU from the split kernel's LDS ring), within [line/16384, line/256] for the
// longest possible line (B x span_max keys).  When every span is short and
// the sequences alone fill the round, workgroup w takes sequence w instead.  `span_max` is
// the longest key range one sequence can read: min(W + q_len - 1, max_ctx) on
// local layers (q_len query tokens at the end of the context), max_ctx on
// global layers.  `int8`: the plan of an int8-cache call, which always takes
// the split kernel (never the bf16 tile kernel).
struct DecodePlan {
  int32_t n_wg;
  int32_t span_max;
  bool per_seq;   // workgroup w takes sequence w whole (n_wg = B); see decode_plan
  bool tile;      // bf16 keys-as-values caches at head width 512 with >= 48 query columns per KV head:
                  // the 32-key tile kernel, 64 columns per workgroup, two workgroups per CU
};
DecodePlan decode_plan(const gemma_attn_layer& L, int32_t num_heads, int32_t batch, int32_t max_ctx, int32_t q_len,
                       const DeviceShape& dev = kMI355X, bool int8 = false);

// Decode shapes the kernels' grids and the workspace layout can hold:
// batch <= 65535, KV heads x 16-column blocks <= 65535, Hq x q_len < 2^31.
// Checked before any plan or size is computed (GA_ERR_UNSUPPORTED / size 0).
bool decode_shape_supported(const gemma_attn_layer& L, int32_t num_heads, int32_t batch, int32_t q_len);

// Workspace layout, every region on a 256-byte boundary: int64 prefix sums of
// the spans [B + 1]; int32 first readable keys [B]; then fp32 partials for
// n_wg + B slots (a workgroup's range touching sequence b stores at slot
// w + b): o [slots, q_len, Hq, D], m and l [slots, q_len, Hq].
struct DecodeWorkspace {
  size_t prefix_off, lo_off, o_off, m_off, l_off, total;
};
DecodeWorkspace decode_workspace(const gemma_attn_layer& L, int32_t num_heads, int32_t batch, int32_t q_len,
                                 const DecodePlan& p);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace ga
