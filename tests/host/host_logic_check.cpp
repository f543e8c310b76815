// Drives the library's host logic (layer resolution, config validation,
// decode plan and workspace layout) over configurations read from stdin, one
// per line, and prints what it computes.  Built with g++ and the address and
// undefined-behaviour sanitizers by tests/test_host_sanitize.py, which feeds
// it edge values (extreme integers, NaN and infinite doubles, null pointers)
// and checks every printed value against the oracle's layer resolution.
//
// Input line:  layer num_heads num_kv_heads num_global_kv_heads head_dim
//              global_head_dim sliding_window sliding_window_pattern k_eq_v
//              norm_weight_offset reserved rope_theta rope_local_theta
//              partial_rotary_factor attn_logit_softcapping
//              query_pre_attn_scalar norm_eps rope_scaling_factor
//              batch max_ctx q_len cus lds_per_cu
// Output line: rc [is_global window num_kv_heads head_dim group rotary_dim
//              k_eq_v theta scale softcap pos_div n_wg span_max per_seq tile
//              workspace_total]
#include <cinttypes>
#include <cstdio>
#include <cstring>

#include "host_logic.h"

int main() {
  char line[2048];
  // a null config and a null output are refused
  gemma_attn_layer L;
  if (ga::resolve_layer(nullptr, 0, &L) != GA_ERR_INVALID_ARG) return 2;
  while (std::fgets(line, sizeof line, stdin)) {
    gemma_attn_config c;
    std::memset(&c, 0, sizeof c);
    long long layer = 0, batch = 0, max_ctx = 0, q_len = 0, cus = 0, lds = 0;
    int n = std::sscanf(line,
                        "%lld %" SCNd32 " %" SCNd32 " %" SCNd32 " %" SCNd32 " %" SCNd32 " %" SCNd32 " %" SCNd32
                        " %" SCNd32 " %" SCNd32 " %" SCNd32 " %lf %lf %lf %lf %lf %lf %lf %lld %lld %lld %lld %lld",
                        &layer, &c.num_heads, &c.num_kv_heads, &c.num_global_kv_heads, &c.head_dim,
                        &c.global_head_dim, &c.sliding_window, &c.sliding_window_pattern, &c.k_eq_v,
                        &c.norm_weight_offset, &c.reserved, &c.rope_theta, &c.rope_local_theta,
                        &c.partial_rotary_factor, &c.attn_logit_softcapping, &c.query_pre_attn_scalar, &c.norm_eps,
                        &c.rope_scaling_factor, &batch, &max_ctx, &q_len, &cus, &lds);
    if (n != 23) return 3;
    if (ga::resolve_layer(&c, static_cast<int32_t>(layer), nullptr) != GA_ERR_INVALID_ARG) return 4;
    const int rc = ga::resolve_layer(&c, static_cast<int32_t>(layer), &L);
    if (rc != GA_OK) {
      std::printf("%d\n", rc);
      continue;
    }
    if (batch < 0 || max_ctx < 1 || q_len < 1 || q_len > max_ctx || batch > 0x7fffffff ||
        !ga::decode_shape_supported(L, c.num_heads, static_cast<int32_t>(batch), static_cast<int32_t>(q_len))) {
      std::printf("%d %d %d %d %d %d %d %d %.17g %.17g %.17g %.17g -1 -1 -1 -1 0 -1 -1 -1 0\n", rc, L.is_global, L.window,
                  L.num_kv_heads, L.head_dim, L.group, L.rotary_dim, L.k_eq_v, L.theta, L.scale, L.softcap,
                  L.pos_div);
      continue;
    }
    ga::DeviceShape dev{static_cast<int32_t>(cus), static_cast<int32_t>(lds), 8};
    const ga::DecodePlan p = ga::decode_plan(L, c.num_heads, static_cast<int32_t>(batch),
                                             static_cast<int32_t>(max_ctx), static_cast<int32_t>(q_len), dev);
    const ga::DecodeWorkspace w = ga::decode_workspace(L, c.num_heads, static_cast<int32_t>(batch),
                                                       static_cast<int32_t>(q_len), p);
    // the int8 cache's plan (its own ring depth; never the bf16 tile kernel)
    const ga::DecodePlan p8 = ga::decode_plan(L, c.num_heads, static_cast<int32_t>(batch),
                                              static_cast<int32_t>(max_ctx), static_cast<int32_t>(q_len), dev, true);
    const ga::DecodeWorkspace w8 = ga::decode_workspace(L, c.num_heads, static_cast<int32_t>(batch),
                                                        static_cast<int32_t>(q_len), p8);
    std::printf("%d %d %d %d %d %d %d %d %.17g %.17g %.17g %.17g %d %d %d %d %zu %d %d %d %zu\n", rc, L.is_global,
                L.window, L.num_kv_heads, L.head_dim, L.group, L.rotary_dim, L.k_eq_v, L.theta, L.scale, L.softcap,
                L.pos_div, p.n_wg, p.span_max, p.per_seq ? 1 : 0, p.tile ? 1 : 0, w.total, p8.n_wg, p8.per_seq ? 1 : 0,
                p8.tile ? 1 : 0, w8.total);
  }
  return 0;
}
