// Host-side logic: validation, layer resolution, decode split plan.
// Sources: the argument tables of the Gemma, Gemma 2, Gemma 3 and Gemma 4 model
// pages, and the Gemma 3 / Gemma 2 descriptions of the local/global interleave.
#include "host_logic.h"

#include <cmath>
#include <cstring>

namespace ga {

namespace {
bool finite(double x) { return std::isfinite(x); }
}  // namespace

int validate_config(const gemma_attn_config* c) {
  if (!c) return GA_ERR_INVALID_ARG;
  if (c->num_heads <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0) return GA_ERR_INVALID_ARG;
  if (c->num_global_kv_heads < 0 || c->global_head_dim < 0) return GA_ERR_INVALID_ARG;
  if (c->reserved != 0) return GA_ERR_INVALID_ARG;
  if (c->k_eq_v != 0 && c->k_eq_v != 1) return GA_ERR_INVALID_ARG;
  if (c->norm_weight_offset != 0 && c->norm_weight_offset != 1) return GA_ERR_INVALID_ARG;
  if (!finite(c->rope_theta) || !(c->rope_theta > 0.0)) return GA_ERR_INVALID_ARG;
  if (!finite(c->rope_local_theta)) return GA_ERR_INVALID_ARG;
  if (!(c->partial_rotary_factor >= 0.0 && c->partial_rotary_factor <= 1.0)) return GA_ERR_INVALID_ARG;
  if (!finite(c->attn_logit_softcapping) || !finite(c->query_pre_attn_scalar)) return GA_ERR_INVALID_ARG;
  if (!finite(c->norm_eps) || !(c->norm_eps > 0.0)) return GA_ERR_INVALID_ARG;
  if (!finite(c->rope_scaling_factor)) return GA_ERR_INVALID_ARG;
  if (c->num_heads % c->num_kv_heads != 0) return GA_ERR_INVALID_ARG;
  const int32_t hg = c->num_global_kv_heads > 0 ? c->num_global_kv_heads : c->num_kv_heads;
  if (c->num_heads % hg != 0) return GA_ERR_INVALID_ARG;
  return GA_OK;
}

int resolve_layer(const gemma_attn_config* c, int32_t layer_idx, gemma_attn_layer* out) {
  if (!out) return GA_ERR_INVALID_ARG;
  const int rc = validate_config(c);
  if (rc != GA_OK) return rc;
  if (layer_idx < 0) return GA_ERR_INVALID_ARG;
  gemma_attn_layer L;
  std::memset(&L, 0, sizeof(L));
  const int32_t n = c->sliding_window_pattern;
  // One global layer every n layers, local layers first in each period.
  // (64-bit: layer_idx + 1 overflows int32 at the largest index)
  const bool is_global = c->sliding_window <= 0 || (n >= 1 && (static_cast<int64_t>(layer_idx) + 1) % n == 0);
  L.is_global = is_global ? 1 : 0;
  if (is_global) {
    L.window = 0;
    L.theta = c->rope_theta;
    L.num_kv_heads = c->num_global_kv_heads > 0 ? c->num_global_kv_heads : c->num_kv_heads;
    L.head_dim = c->global_head_dim > 0 ? c->global_head_dim : c->head_dim;
    L.k_eq_v = c->k_eq_v;
  } else {
    L.window = c->sliding_window;
    L.theta = c->rope_local_theta > 0.0 ? c->rope_local_theta : c->rope_theta;
    L.num_kv_heads = c->num_kv_heads;
    L.head_dim = c->head_dim;
    L.k_eq_v = 0;
  }
  L.group = c->num_heads / L.num_kv_heads;
  // r = 2*floor(f*D/2), evaluated as (f*D)/2 in double.
  L.rotary_dim = 2 * static_cast<int32_t>(std::floor(c->partial_rotary_factor * L.head_dim / 2.0));
  const double qpas = c->query_pre_attn_scalar > 0.0 ? c->query_pre_attn_scalar : static_cast<double>(L.head_dim);
  L.scale = std::pow(qpas, -0.5);
  L.softcap = c->attn_logit_softcapping > 0.0 ? c->attn_logit_softcapping : 0.0;
  // Long-context rope scaling, read as linear position division on the global layers.
  L.pos_div = (is_global && c->rope_scaling_factor > 0.0) ? c->rope_scaling_factor : 1.0;
  *out = L;
  return GA_OK;
}

bool prologue_dim_supported(int32_t d) {
  return d >= 8 && d <= 512 && (d & (d - 1)) == 0;
}

bool attn_dim_supported(int32_t d) { return d == 64 || d == 256 || d == 512; }

bool attn_group_supported(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

DecodePlan decode_plan(const gemma_attn_layer& L, int32_t num_heads, int32_t batch, int32_t max_ctx, int32_t q_len,
                       const DeviceShape& dev, bool int8) {
  (void)num_heads;
  DecodePlan p;
  const long long cus = dev.cus > 0 ? dev.cus : kMI355X.cus;
  const long long lds_cu = dev.lds_per_cu > 0 ? dev.lds_per_cu : kMI355X.lds_per_cu;
  const long long ql = q_len > 0 ? q_len : 1;
  const long long wspan = static_cast<long long>(L.window) + ql - 1;
  p.span_max = L.window > 0 ? static_cast<int32_t>(wspan < max_ctx ? wspan : max_ctx) : max_ctx;
  if (p.span_max < 1) p.span_max = 1;
  const long long col_blocks = (static_cast<long long>(L.group) * ql + 15) / 16;
  // Many query columns per KV head at head width 512 with keys as values (a
  // multi-token step on an MQA global layer): the tile kernel, which takes 64
  // columns per workgroup through 32x32 products, two workgroups per CU.
  // (Not for int8 caches: they always take the split kernel.)
  p.tile = !int8 && L.k_eq_v && L.head_dim == 512 && col_blocks >= 3;
  long long rows = static_cast<long long>(L.num_kv_heads) * col_blocks;
  long long per_cu;
  if (p.tile) {
    rows = static_cast<long long>(L.num_kv_heads) * ((static_cast<long long>(L.group) * ql + 63) / 64);
    per_cu = 2;
  } else {
    // One round of workgroups on the device: the split kernel's workgroups
    // per CU follow from its LDS (two waves per workgroup, two waves per
    // SIMD): two slots of 16 bf16 rows (or 32 int8 rows, the same bytes) per
    // team, plus, for bf16 caches with keys as values at width 512, a third
    // slot's worth that the launch reserves so that three workgroups share a
    // CU.
    const long long team = L.head_dim > 256 ? 2 : 1;
    const long long slots = (!int8 && L.k_eq_v && L.head_dim == 512) ? 3 : 2;
    const long long lds = (2 / team) * slots * 16LL * L.head_dim * 2 * (L.k_eq_v ? 1 : 2);
    per_cu = lds_cu / lds;
    if (per_cu > 4) per_cu = 4;
    if (per_cu < 1) per_cu = 1;
  }
  long long n = (cus * per_cu) / rows;
  const long long line_max = static_cast<long long>(batch > 0 ? batch : 1) * p.span_max;
  const long long at_least = (line_max + 16383) / 16384;   // at most 16K keys per workgroup
  const long long at_most = (line_max + 255) / 256;        // at least 256 keys per workgroup
  if (n < at_least) n = at_least;
  if (n > at_most) n = at_most;
  if (n > 65535) n = 65535;   // bounds the partial slots of the workspace
  if (n < 1) n = 1;
  p.n_wg = static_cast<int32_t>(n);
  // Short spans (local windows) with enough sequences to fill the round: one
  // workgroup per sequence.  Every span is then at most 8K keys, so no
  // workgroup runs long, and none straddles two sequences.
  const long long round = cus * per_cu;
  p.per_seq = batch > 0 && batch >= (round + rows - 1) / rows && p.span_max <= 8192;
  if (p.per_seq) p.n_wg = batch;
  return p;
}

bool decode_shape_supported(const gemma_attn_layer& L, int32_t num_heads, int32_t batch, int32_t q_len) {
  if (batch > 65535 || q_len < 1 || L.num_kv_heads < 1) return false;
  const long long col_blocks = (static_cast<long long>(L.group) * q_len + 15) / 16;
  if (col_blocks * L.num_kv_heads > 65535) return false;
  return static_cast<long long>(num_heads) * q_len <= 0x7fffffff;
}

DecodeWorkspace decode_workspace(const gemma_attn_layer& L, int32_t num_heads, int32_t batch, int32_t q_len,
                                 const DecodePlan& p) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t b = static_cast<size_t>(batch > 0 ? batch : 0);
  const size_t rows = (static_cast<size_t>(p.n_wg) + b) * static_cast<size_t>(q_len) * static_cast<size_t>(num_heads);
  DecodeWorkspace w;
  w.prefix_off = 0;
  w.lo_off = up((b + 1) * sizeof(int64_t));
  w.o_off = w.lo_off + up(b * sizeof(int32_t) + 4);
  w.m_off = w.o_off + up(rows * static_cast<size_t>(L.head_dim) * sizeof(float));
  w.l_off = w.m_off + up(rows * sizeof(float));
  w.total = w.l_off + up(rows * sizeof(float));
  return w;
}

}  // namespace ga
