// Launch interfaces of the Gemma attention kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

struct PrologueArgs {
  int32_t batch, seq, hq, hkv, dim, rotary_dim;
  const void* q_in;
  const void* k_in;
  void* q_out;
  void* k_out;
  const float* q_norm_w;
  const float* k_norm_w;
  const int32_t* pos0;
  double theta;
  float eps, offset;
  // Cache mode (ctx_len != null): token s of sequence b sits at position
  // ctx_len[b] - seq + s; k_out and v_out are caches [B, max_ctx, Hkv, D] and
  // the processed keys (and raw values, when v_in is set) land at that row.
  const int32_t* ctx_len;
  int32_t max_ctx;
  const void* v_in;
  void* v_out;
};
hipError_t launch_qk_prologue(const PrologueArgs& a, hipStream_t stream);

struct PrefillArgs {
  int32_t batch, seq, hq, hkv, dim, group, window, k_eq_v;
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  double scale, softcap;
};
// Returns hipErrorInvalidValue for an unsupported (dim, group) pair.
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

struct DecodeArgs {
  int32_t batch, max_ctx, hq, hkv, dim, group, window, k_eq_v;
  int32_t chunk, n_split, q_len;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* ctx_len;
  void* out;
  float* lse;
  float* ws_o;
  float* ws_m;
  float* ws_l;
  double scale, softcap;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace ga
