// Launch interfaces of the Gemma attention kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

namespace ga {

// Host side of the shared rotary arithmetic (rotary_rev_freq in ga_device.h):
// w1 = theta^(-2/r) and c0 = 1 / (2 pi pos_div), formed once per launch by the
// prologue's and the attention kernel's launchers alike.
inline double rotary_w1(double theta, int32_t rotary_dim) { return std::pow(theta, -2.0 / rotary_dim); }
inline double rotary_c0(double pos_div) {
  return 1.0 / (2.0 * 3.14159265358979323846 * (pos_div > 0.0 ? pos_div : 1.0));
}

// Launch a kernel that takes one parameter struct and return the launch's own
// status (hipLaunchKernel reports it directly, so no stale error from an
// earlier, unrelated call is picked up).  `lds_reserve` bytes of dynamic LDS
// that the kernel does not use limit how many of its workgroups share a CU.
template <class P>
inline hipError_t launch_kernel(void (*fn)(P), dim3 grid, dim3 block, hipStream_t stream, P p,
                                uint32_t lds_reserve = 0) {
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, args, lds_reserve, stream);
}

// Launchers return hipErrorNotSupported for a shape with no kernel
// instantiation or a grid beyond the launch limits; the C ABI reports that as
// GA_ERR_UNSUPPORTED and every other failure as GA_ERR_HIP.

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
  double pos_div;             // rotary positions are divided by this (rope scaling)
  float eps, offset;
  // Cache mode (max_ctx > 0): token s of sequence b sits at position
  // ctx_len[b] - seq + s (pos0[b] + s when ctx_len is null); k_out and v_out
  // are caches [B, max_ctx, Hkv, D] and the processed keys (and raw values,
  // when v_in is set) land at that row.  With k_scales set the caches are int8
  // instead: codes k_codes / v_codes [B, max_ctx, Hkv, D] and fp32 scales
  // k_scales / v_scales [B, Hkv, max_ctx].
  const int32_t* ctx_len;
  int32_t max_ctx;
  const void* v_in;
  void* v_out;
  void* k_codes;
  float* k_scales;
  void* v_codes;
  float* v_scales;
};
hipError_t launch_qk_prologue(const PrologueArgs& a, hipStream_t stream);

struct PrefillArgs {
  int32_t batch, seq, hq, hkv, dim, group, window, k_eq_v;
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* seq_start;   // padded batch (device [B], may be null): kept rows [start, end)
  const int32_t* seq_end;
  double scale, softcap;
  int32_t xcds;               // L2 domains (XCDs) the dispatcher deals workgroups over, round-robin
  // Fused query rotary (q_rope = 1): q holds the queries before rotary; the
  // kernel turns them by the layer's full-width rotary at positions
  // pos0[b] + s (pos0 device [B] or null), divided by rope_pos_div.
  int32_t q_rope;
  const int32_t* pos0;
  double rope_theta, rope_pos_div;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

struct DecodeArgs {
  int32_t batch, max_ctx, hq, hkv, dim, group, window, k_eq_v;
  int32_t n_wg, q_len;        // workgroups per (KV head, column block); query tokens per sequence
  int32_t per_seq;            // 1: workgroup w takes sequence w whole (n_wg = batch)
  int32_t tile;               // 1: the 32-key tile kernel (bf16, keys as values, head width 512)
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* ctx_len;
  const int32_t* kv_start;    // device [B] or null: first cache row each sequence may read
  void* out;
  float* lse;
  float* ws_o;
  float* ws_m;
  float* ws_l;
  int64_t* ws_prefix;         // [B + 1] prefix sums of the readable spans (written by the plan kernel)
  int32_t* ws_lo;             // [B] first readable key of each sequence
  // int8 caches (k_scales set): k_cache / v_cache hold int8 codes and these
  // the fp32 scales, [B, Hkv, max_ctx].
  const float* k_scales;
  const float* v_scales;
  double scale, softcap;
  int32_t xcds;               // L2 domains (XCDs) the dispatcher deals workgroups over, round-robin
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace ga
