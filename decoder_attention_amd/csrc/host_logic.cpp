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
  const bool is_global = c->sliding_window <= 0 || (n >= 1 && (layer_idx + 1) % n == 0);
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

DecodePlan decode_plan(const gemma_attn_layer& L, int32_t num_heads, int32_t batch, int32_t max_ctx, int32_t q_len) {
  (void)num_heads;
  DecodePlan p;
  const long long ql = q_len > 0 ? q_len : 1;
  const long long wspan = static_cast<long long>(L.window) + ql - 1;
  p.span_max = L.window > 0 ? static_cast<int32_t>(wspan < max_ctx ? wspan : max_ctx) : max_ctx;
  if (p.span_max < 1) p.span_max = 1;
  // Aim for >= 2048 workgroups over (split, KV head x 16-column block,
  // sequence) so that 256 CUs stay busy on ragged lengths; chunks are powers
  // of two in [256, 4096] keys.
  const long long col_blocks = (static_cast<long long>(L.group) * ql + 15) / 16;
  const long long units = static_cast<long long>(batch > 0 ? batch : 1) * L.num_kv_heads * col_blocks;
  long long want = (2048 + units - 1) / units;
  if (want < 1) want = 1;
  long long chunk = 256;
  while (chunk < 4096 && chunk * want < p.span_max) chunk *= 2;
  // With enough units to fill the chip, longer chunks amortise each
  // workgroup's start-up (first copy latency, merge, partial write-back).
  if (units >= 256 && chunk < 1024) chunk = 1024;
  p.chunk = static_cast<int32_t>(chunk);
  // Splits are relative to the first key a sequence reads, so span/chunk
  // chunks (rounded up) cover every sequence.
  long long ns = (p.span_max + chunk - 1) / chunk;
  if (ns < 1) ns = 1;
  p.n_split = static_cast<int32_t>(ns);
  return p;
}

DecodeWorkspace decode_workspace(const gemma_attn_layer& L, int32_t num_heads, int32_t batch, int32_t q_len,
                                 const DecodePlan& p) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t rows = static_cast<size_t>(batch) * num_heads * static_cast<size_t>(q_len) * p.n_split;
  DecodeWorkspace w;
  w.o_off = 0;
  w.m_off = up(rows * L.head_dim * sizeof(float));
  w.l_off = w.m_off + up(rows * sizeof(float));
  w.total = w.l_off + up(rows * sizeof(float));
  return w;
}

}  // namespace ga
