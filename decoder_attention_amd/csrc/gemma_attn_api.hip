// C ABI entry points (include/gemma_attn.h): host-side checks, then launches.
// Every argument check runs before anything is enqueued, so an argument error
// means nothing was enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>

#include "gemma_attn.h"
#include "ga_kernels.h"
#include "host_logic.h"

namespace {

bool dev_ok(const void* p) { return p != nullptr && ga::aligned16(p); }

// hipErrorNotSupported is what the launchers return for a shape with no
// instantiation or a grid beyond the launch limits; any other failure is the
// runtime's.
int hip_rc(hipError_t e) {
  if (e == hipSuccess) return GA_OK;
  if (e == hipErrorNotSupported) return GA_ERR_UNSUPPORTED;
  return GA_ERR_HIP;
}

// CU count, LDS per CU and XCD count of the current device, queried once per
// device and cached (the values never change while the process runs).  Without
// a usable device the whole-MI355X shape stands in, so sizes computed on a
// host with no GPU match the single-partition part.
ga::DeviceShape current_device_shape() {
  constexpr int kMaxDev = 64;
  static std::atomic<int32_t> cus[kMaxDev], lds[kMaxDev], xcds[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return ga::kMI355X;
  ga::DeviceShape d{cus[dev].load(std::memory_order_acquire), lds[dev].load(std::memory_order_relaxed),
                    xcds[dev].load(std::memory_order_relaxed)};
  if (d.cus > 0) return d;
  int c = 0, l = 0, x = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) return ga::kMI355X;
  if (hipDeviceGetAttribute(&l, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess || l < 1)
    l = ga::kMI355X.lds_per_cu;
  if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x < 1) x = 1;
  lds[dev].store(l, std::memory_order_relaxed);
  xcds[dev].store(x, std::memory_order_relaxed);
  cus[dev].store(c, std::memory_order_release);
  return ga::DeviceShape{c, l, x};
}

// Scratch of the allocation-free decode entry point: one array per device,
// held from the library's first use of a device until the process ends.  In
// host code `scratch` only names the symbol; its device address (a different
// one on every GPU) comes from hipGetSymbolAddress, once per device, with
// that device current, and only that address is passed to kernels.
constexpr size_t kScratchBytes = size_t{80} << 20;   // 80 MiB
__device__ __align__(256) unsigned char scratch[kScratchBytes];

void* device_scratch() {
  constexpr int kMaxDev = 64;
  static std::atomic<void*> addr[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  addr[dev].store(p, std::memory_order_release);   // racing first calls store the same address
  return p;
}

int prefill_common(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t seq, const void* q,
                   const void* k, const void* v, void* out, float* lse, const int32_t* seq_start,
                   const int32_t* seq_end, void* stream, bool q_rope = false, const int32_t* pos0 = nullptr) {
  gemma_attn_layer L;
  const int rc = ga::resolve_layer(cfg, layer_idx, &L);
  if (rc != GA_OK) return rc;
  if (batch < 0 || seq < 0) return GA_ERR_INVALID_ARG;
  if (!ga::attn_dim_supported(L.head_dim) || !ga::attn_group_supported(L.group)) return GA_ERR_UNSUPPORTED;
  if (q_rope && (L.head_dim != 256 || L.k_eq_v || L.rotary_dim != L.head_dim)) return GA_ERR_UNSUPPORTED;
  if (batch > 65535 || L.num_kv_heads > 65535) return GA_ERR_UNSUPPORTED;
  if (batch == 0 || seq == 0) return GA_OK;
  if (!dev_ok(q) || !dev_ok(k) || !dev_ok(out)) return GA_ERR_INVALID_ARG;
  if (!L.k_eq_v && !dev_ok(v)) return GA_ERR_INVALID_ARG;
  if (lse && !ga::aligned16(lse)) return GA_ERR_INVALID_ARG;
  ga::PrefillArgs a{};
  a.batch = batch;
  a.seq = seq;
  a.hq = cfg->num_heads;
  a.hkv = L.num_kv_heads;
  a.dim = L.head_dim;
  a.group = L.group;
  a.window = L.window;
  a.k_eq_v = L.k_eq_v;
  a.q = q;
  a.k = k;
  a.v = L.k_eq_v ? k : v;
  a.out = out;
  a.lse = lse;
  a.seq_start = seq_start;
  a.seq_end = seq_end;
  a.scale = L.scale;
  a.softcap = L.softcap;
  a.xcds = current_device_shape().xcds;
  a.q_rope = q_rope ? 1 : 0;
  a.pos0 = pos0;
  a.rope_theta = L.theta;
  a.rope_pos_div = L.pos_div;
  return hip_rc(ga::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

// Shared by the bf16 and int8 decode entry points (k_scales set: int8 caches).
int decode_common(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len, int32_t max_ctx,
                  const void* q, const void* k_cache, const float* k_scales, const void* v_cache,
                  const float* v_scales, const int32_t* ctx_len, const int32_t* kv_start, void* out, float* lse,
                  void* workspace, size_t workspace_bytes, void* stream, bool use_scratch = false) {
  gemma_attn_layer L;
  const int rc = ga::resolve_layer(cfg, layer_idx, &L);
  if (rc != GA_OK) return rc;
  if (batch < 0 || max_ctx < 1 || q_len < 1 || q_len > max_ctx) return GA_ERR_INVALID_ARG;
  if (!ga::attn_dim_supported(L.head_dim) || !ga::attn_group_supported(L.group)) return GA_ERR_UNSUPPORTED;
  if (!ga::decode_shape_supported(L, cfg->num_heads, batch, q_len)) return GA_ERR_UNSUPPORTED;
  if (batch == 0) return GA_OK;
  if (!dev_ok(q) || !dev_ok(k_cache) || !dev_ok(out) || ctx_len == nullptr) return GA_ERR_INVALID_ARG;
  if (!L.k_eq_v && !dev_ok(v_cache)) return GA_ERR_INVALID_ARG;
  if (k_scales && (!dev_ok(k_scales) || (!L.k_eq_v && !dev_ok(v_scales)))) return GA_ERR_INVALID_ARG;
  if (lse && !ga::aligned16(lse)) return GA_ERR_INVALID_ARG;
  const ga::DeviceShape dev = current_device_shape();
  const ga::DecodePlan plan = ga::decode_plan(L, cfg->num_heads, batch, max_ctx, q_len, dev, k_scales != nullptr);
  const ga::DecodeWorkspace ws = ga::decode_workspace(L, cfg->num_heads, batch, q_len, plan);
  if (use_scratch) {   // the allocation-free entry point: the library's own scratch array
    if (ws.total > kScratchBytes) return GA_ERR_SCRATCH_LIMIT;
    workspace = device_scratch();
    if (workspace == nullptr) return GA_ERR_HIP;
    workspace_bytes = kScratchBytes;
  }
  if (workspace == nullptr || !ga::aligned16(workspace) || workspace_bytes < ws.total) return GA_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(workspace);
  ga::DecodeArgs a{};
  a.batch = batch;
  a.max_ctx = max_ctx;
  a.hq = cfg->num_heads;
  a.hkv = L.num_kv_heads;
  a.dim = L.head_dim;
  a.group = L.group;
  a.window = L.window;
  a.k_eq_v = L.k_eq_v;
  a.n_wg = plan.n_wg;
  a.per_seq = plan.per_seq ? 1 : 0;
  a.tile = (plan.tile && k_scales == nullptr) ? 1 : 0;
  a.q_len = q_len;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = L.k_eq_v ? k_cache : v_cache;
  a.k_scales = k_scales;
  a.v_scales = L.k_eq_v ? k_scales : v_scales;
  a.ctx_len = ctx_len;
  a.kv_start = kv_start;
  a.out = out;
  a.lse = lse;
  a.ws_o = reinterpret_cast<float*>(wsb + ws.o_off);
  a.ws_m = reinterpret_cast<float*>(wsb + ws.m_off);
  a.ws_l = reinterpret_cast<float*>(wsb + ws.l_off);
  a.ws_prefix = reinterpret_cast<int64_t*>(wsb + ws.prefix_off);
  a.ws_lo = reinterpret_cast<int32_t*>(wsb + ws.lo_off);
  a.scale = L.scale;
  a.softcap = L.softcap;
  a.xcds = dev.xcds;
  return hip_rc(ga::launch_decode(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int gemma_attn_resolve_layer(const gemma_attn_config* cfg, int32_t layer_idx, gemma_attn_layer* out) {
  return ga::resolve_layer(cfg, layer_idx, out);
}

const char* gemma_attn_strerror(int code) {
  switch (code) {
    case GA_OK: return "ok";
    case GA_ERR_INVALID_ARG: return "invalid argument";
    case GA_ERR_UNSUPPORTED: return "unsupported head width or group size";
    case GA_ERR_WORKSPACE: return "decode workspace missing or too small";
    case GA_ERR_HIP: return "HIP launch failed";
    case GA_ERR_SCRATCH_LIMIT: return "shape needs more decode workspace than the library's 80 MiB scratch holds";
    default: return "unknown error";
  }
}

int gemma_qk_prologue(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t seq,
                      const void* q_in, const void* k_in, void* q_out, void* k_out,
                      const float* q_norm_w, const float* k_norm_w, const int32_t* pos0, void* stream) {
  gemma_attn_layer L;
  const int rc = ga::resolve_layer(cfg, layer_idx, &L);
  if (rc != GA_OK) return rc;
  if (batch < 0 || seq < 0) return GA_ERR_INVALID_ARG;
  if (static_cast<long long>(batch) * seq > INT_MAX) return GA_ERR_UNSUPPORTED;
  if (!ga::prologue_dim_supported(L.head_dim)) return GA_ERR_UNSUPPORTED;
  if (batch == 0 || seq == 0) return GA_OK;
  if (!q_in && !k_in) return GA_ERR_INVALID_ARG;
  if (q_in && (!dev_ok(q_in) || !dev_ok(q_out))) return GA_ERR_INVALID_ARG;
  if (k_in && !dev_ok(k_out)) return GA_ERR_INVALID_ARG;
  if (k_in && !ga::aligned16(k_in)) return GA_ERR_INVALID_ARG;
  if ((q_norm_w && !ga::aligned16(q_norm_w)) || (k_norm_w && !ga::aligned16(k_norm_w))) return GA_ERR_INVALID_ARG;
  ga::PrologueArgs a{};
  a.batch = batch;
  a.seq = seq;
  a.hq = q_in ? cfg->num_heads : 0;      // keys only: no query rows
  a.hkv = L.num_kv_heads;
  a.dim = L.head_dim;
  a.rotary_dim = L.rotary_dim;
  a.q_in = q_in;
  a.k_in = k_in;
  a.q_out = q_in ? q_out : nullptr;
  a.k_out = k_in ? k_out : nullptr;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.pos0 = pos0;
  a.theta = L.theta;
  a.pos_div = L.pos_div;
  a.eps = static_cast<float>(cfg->norm_eps);
  a.offset = static_cast<float>(cfg->norm_weight_offset);
  a.ctx_len = nullptr;
  a.max_ctx = 0;
  a.v_in = nullptr;
  a.v_out = nullptr;
  return hip_rc(ga::launch_qk_prologue(a, static_cast<hipStream_t>(stream)));
}

int gemma_attn_prefill(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t seq,
                       const void* q, const void* k, const void* v, void* out, float* lse, void* stream) {
  return prefill_common(cfg, layer_idx, batch, seq, q, k, v, out, lse, nullptr, nullptr, stream);
}

int gemma_attn_prefill_qrope(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t seq,
                             const void* q_raw, const void* k, const void* v, const int32_t* pos0, void* out,
                             float* lse, void* stream) {
  return prefill_common(cfg, layer_idx, batch, seq, q_raw, k, v, out, lse, nullptr, nullptr, stream, true, pos0);
}

int gemma_attn_prefill_ragged(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t seq,
                              const void* q, const void* k, const void* v, void* out, float* lse,
                              const int32_t* seq_start, const int32_t* seq_end, void* stream) {
  return prefill_common(cfg, layer_idx, batch, seq, q, k, v, out, lse, seq_start, seq_end, stream);
}

size_t gemma_attn_decode_multi_workspace_size(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch,
                                              int32_t q_len, int32_t max_ctx) {
  gemma_attn_layer L;
  if (ga::resolve_layer(cfg, layer_idx, &L) != GA_OK) return 0;
  if (batch < 0 || max_ctx < 1 || q_len < 1 || q_len > max_ctx) return 0;
  if (!ga::decode_shape_supported(L, cfg->num_heads, batch, q_len)) return 0;
  // Either cache type: the larger of the bf16 and int8 plans' workspaces.
  const ga::DeviceShape dev = current_device_shape();
  const size_t a = ga::decode_workspace(L, cfg->num_heads, batch, q_len,
                                        ga::decode_plan(L, cfg->num_heads, batch, max_ctx, q_len, dev, false)).total;
  const size_t b = ga::decode_workspace(L, cfg->num_heads, batch, q_len,
                                        ga::decode_plan(L, cfg->num_heads, batch, max_ctx, q_len, dev, true)).total;
  return a > b ? a : b;
}

size_t gemma_attn_decode_workspace_size(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch,
                                        int32_t max_ctx) {
  return gemma_attn_decode_multi_workspace_size(cfg, layer_idx, batch, 1, max_ctx);
}

int gemma_attn_decode_multi(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len,
                            int32_t max_ctx, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* ctx_len, const int32_t* kv_start, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_common(cfg, layer_idx, batch, q_len, max_ctx, q, k_cache, nullptr, v_cache, nullptr, ctx_len, kv_start,
                       out, lse, workspace, workspace_bytes, stream);
}

int gemma_attn_decode_multi_noalloc(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len,
                                    int32_t max_ctx, const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* ctx_len, const int32_t* kv_start, void* out, float* lse,
                                    void* stream) {
  return decode_common(cfg, layer_idx, batch, q_len, max_ctx, q, k_cache, nullptr, v_cache, nullptr, ctx_len, kv_start,
                       out, lse, nullptr, 0, stream, /*use_scratch=*/true);
}

int gemma_attn_decode_int8(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len,
                           int32_t max_ctx, const void* q, const void* k_codes, const float* k_scales,
                           const void* v_codes, const float* v_scales, const int32_t* ctx_len,
                           const int32_t* kv_start, void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (k_scales == nullptr) return GA_ERR_INVALID_ARG;
  return decode_common(cfg, layer_idx, batch, q_len, max_ctx, q, k_codes, k_scales, v_codes, v_scales, ctx_len,
                       kv_start, out, lse, workspace, workspace_bytes, stream);
}

int gemma_attn_decode(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t max_ctx,
                      const void* q, const void* k_cache, const void* v_cache, const int32_t* ctx_len,
                      void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return gemma_attn_decode_multi(cfg, layer_idx, batch, 1, max_ctx, q, k_cache, v_cache, ctx_len, nullptr, out, lse,
                                 workspace, workspace_bytes, stream);
}

int gemma_qk_prologue_cache(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len,
                            int32_t max_ctx, const void* q_in, const void* k_in, const void* v_in, void* q_out,
                            void* k_cache, void* v_cache, const float* q_norm_w, const float* k_norm_w,
                            const int32_t* ctx_len, void* stream) {
  gemma_attn_layer L;
  const int rc = ga::resolve_layer(cfg, layer_idx, &L);
  if (rc != GA_OK) return rc;
  if (batch < 0 || q_len < 0 || max_ctx < 1 || q_len > max_ctx) return GA_ERR_INVALID_ARG;
  if (static_cast<long long>(batch) * q_len > INT_MAX) return GA_ERR_UNSUPPORTED;
  if (!ga::prologue_dim_supported(L.head_dim)) return GA_ERR_UNSUPPORTED;
  if (batch == 0 || q_len == 0) return GA_OK;
  if (!dev_ok(q_in) || !dev_ok(q_out) || !dev_ok(k_in) || !dev_ok(k_cache) || ctx_len == nullptr)
    return GA_ERR_INVALID_ARG;
  if (!L.k_eq_v && (!dev_ok(v_in) || !dev_ok(v_cache))) return GA_ERR_INVALID_ARG;
  if ((q_norm_w && !ga::aligned16(q_norm_w)) || (k_norm_w && !ga::aligned16(k_norm_w))) return GA_ERR_INVALID_ARG;
  ga::PrologueArgs a{};
  a.batch = batch;
  a.seq = q_len;
  a.hq = cfg->num_heads;
  a.hkv = L.num_kv_heads;
  a.dim = L.head_dim;
  a.rotary_dim = L.rotary_dim;
  a.q_in = q_in;
  a.k_in = k_in;
  a.q_out = q_out;
  a.k_out = k_cache;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.pos0 = nullptr;
  a.theta = L.theta;
  a.pos_div = L.pos_div;
  a.eps = static_cast<float>(cfg->norm_eps);
  a.offset = static_cast<float>(cfg->norm_weight_offset);
  a.ctx_len = ctx_len;
  a.max_ctx = max_ctx;
  a.v_in = L.k_eq_v ? nullptr : v_in;
  a.v_out = L.k_eq_v ? nullptr : v_cache;
  return hip_rc(ga::launch_qk_prologue(a, static_cast<hipStream_t>(stream)));
}

int gemma_qk_prologue_cache_int8(const gemma_attn_config* cfg, int32_t layer_idx, int32_t batch, int32_t q_len,
                                 int32_t max_ctx, const void* q_in, const void* k_in, const void* v_in, void* q_out,
                                 void* k_codes, float* k_scales, void* v_codes, float* v_scales,
                                 const float* q_norm_w, const float* k_norm_w, const int32_t* ctx_len, void* stream) {
  gemma_attn_layer L;
  const int rc = ga::resolve_layer(cfg, layer_idx, &L);
  if (rc != GA_OK) return rc;
  if (batch < 0 || q_len < 0 || max_ctx < 1 || q_len > max_ctx) return GA_ERR_INVALID_ARG;
  if (static_cast<long long>(batch) * q_len > INT_MAX) return GA_ERR_UNSUPPORTED;
  if (!ga::prologue_dim_supported(L.head_dim)) return GA_ERR_UNSUPPORTED;
  if (batch == 0 || q_len == 0) return GA_OK;
  if (!dev_ok(q_in) || !dev_ok(q_out) || !dev_ok(k_in) || !dev_ok(k_codes) || !dev_ok(k_scales) || ctx_len == nullptr)
    return GA_ERR_INVALID_ARG;
  if (!L.k_eq_v && (!dev_ok(v_in) || !dev_ok(v_codes) || !dev_ok(v_scales))) return GA_ERR_INVALID_ARG;
  if ((q_norm_w && !ga::aligned16(q_norm_w)) || (k_norm_w && !ga::aligned16(k_norm_w))) return GA_ERR_INVALID_ARG;
  ga::PrologueArgs a{};
  a.batch = batch;
  a.seq = q_len;
  a.hq = cfg->num_heads;
  a.hkv = L.num_kv_heads;
  a.dim = L.head_dim;
  a.rotary_dim = L.rotary_dim;
  a.q_in = q_in;
  a.k_in = k_in;
  a.q_out = q_out;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.theta = L.theta;
  a.pos_div = L.pos_div;
  a.eps = static_cast<float>(cfg->norm_eps);
  a.offset = static_cast<float>(cfg->norm_weight_offset);
  a.ctx_len = ctx_len;
  a.max_ctx = max_ctx;
  a.v_in = L.k_eq_v ? nullptr : v_in;
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.v_codes = L.k_eq_v ? nullptr : v_codes;
  a.v_scales = L.k_eq_v ? nullptr : v_scales;
  return hip_rc(ga::launch_qk_prologue(a, static_cast<hipStream_t>(stream)));
}

int gemma_kv_quantize_int8(int32_t batch, int32_t seq, int32_t num_kv_heads, int32_t head_dim, int32_t max_ctx,
                           const void* x, const int32_t* pos0, void* codes, float* scales, void* stream) {
  if (batch < 0 || seq < 0 || num_kv_heads < 1 || head_dim < 1 || max_ctx < 1) return GA_ERR_INVALID_ARG;
  if (static_cast<long long>(batch) * seq > INT_MAX) return GA_ERR_UNSUPPORTED;
  if (!ga::prologue_dim_supported(head_dim)) return GA_ERR_UNSUPPORTED;
  if (batch == 0 || seq == 0) return GA_OK;
  if (!dev_ok(x) || !dev_ok(codes) || !dev_ok(scales)) return GA_ERR_INVALID_ARG;
  if (pos0 && !ga::aligned16(pos0)) return GA_ERR_INVALID_ARG;
  // The prologue kernel with no query heads, no norm and no rotation: each key
  // row passes through unchanged and is quantized into its cache row.
  ga::PrologueArgs a{};
  a.batch = batch;
  a.seq = seq;
  a.hq = 0;
  a.hkv = num_kv_heads;
  a.dim = head_dim;
  a.rotary_dim = 0;
  a.k_in = x;
  a.pos0 = pos0;
  a.theta = 1.0;
  a.pos_div = 1.0;
  a.max_ctx = max_ctx;
  a.k_codes = codes;
  a.k_scales = scales;
  return hip_rc(ga::launch_qk_prologue(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
