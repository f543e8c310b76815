// Split-KV decode attention over a contiguous KV cache (gfx950).
//
// One query token per sequence (the decode step of generate()).  The keys a
// sequence reads -- [ctx - W, ctx) on local layers, [0, ctx) on global layers
// -- are cut into chunks; one workgroup handles one (chunk, KV head, sequence)
// and produces an unnormalised partial (m, l, o) for the g query heads of the
// group; a second kernel merges the partials of each (sequence, head) in a
// fixed order (log-sum-exp combine).
//
// Inside a workgroup each of the 4 waves streams 32-key tiles of the chunk
// (tiles interleaved across waves):
//   * K rows are loaded from HBM straight into the A-operand layout of
//     v_mfma_f32_16x16x32_bf16 (16-byte loads, lane = key row);
//   * S^T[16 keys x 16 cols] = K . Q^T with the g heads as columns (padded to
//     16), so each lane owns one head and the softmax reductions are over the
//     four lanes that share it;
//   * the value rows (the same registers with keys-as-values) are written to
//     the wave's own LDS tile and read back transposed (ds_read_b64_tr_b16) as
//     the A operand of O^T += V^T . P^T.
// Cache rows outside the sequence's range are never loaded.
//
// Sources: generate() decoding over cached keys and values (Gemma 4 page, API;
// the atlas summary on KV caches bounded by the window on local layers), the
// window, soft cap, scaling and keys-as-values as for prefill.
#include "ga_device.h"
#include "ga_kernels.h"

namespace ga {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKeys = 32;   // keys per wave tile
constexpr int kPad = 8;

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* ctx_len;
  uint16_t* out;
  float* lse;
  float* ws_o;
  float* ws_m;
  float* ws_l;
  int32_t max_ctx, hq, hkv, window, chunk, n_split;
  float scale_log2, cap_in2, cap_log2;
};

__device__ __forceinline__ void seq_range(const DecodeParams& p, int32_t b, int32_t& lo, int32_t& ctx) {
  int32_t c = p.ctx_len[b];
  c = c < 0 ? 0 : (c > p.max_ctx ? p.max_ctx : c);
  const int32_t span = p.window > 0 ? min(c, p.window) : c;
  ctx = c;
  lo = c - span;
}

template <int D, int G, bool KEQV, bool CAP>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
  constexpr int kDS = D / 32;        // k-steps of QK^T (16x16x32)
  constexpr int kDB = D / 16;        // 16-row blocks of O^T
  constexpr int kLd = D + kPad;
  constexpr int kTileElems = kKeys * kLd;
  static_assert(G <= 16, "at most 16 query heads per KV head");

  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int32_t split = blockIdx.x;
  const int32_t kvh = blockIdx.y;
  const int32_t b = blockIdx.z;
  int32_t lo, ctx;
  seq_range(p, b, lo, ctx);
  const int32_t s_lo = lo + split * p.chunk;
  if (s_lo >= ctx) return;   // this split is empty for the sequence (uniform)
  const int32_t s_hi = min(ctx, s_lo + p.chunk);

  const int32_t tid = threadIdx.x;
  const int32_t wave = tid >> 6;
  const int32_t lane = tid & 63;
  const int32_t col = lane & 15;     // query head within the group (valid if < G)
  const int32_t grp = lane >> 4;     // 16-lane group
  uint16_t* tile = smem + wave * kTileElems;

  // Q^T operand: lane holds d = ds*32 + grp*8 + [0, 8) of head `col`.
  bf16x8 qf[kDS];
  {
    const int32_t hcol = col < G ? col : 0;
    const uint16_t* qrow = p.q + (static_cast<int64_t>(b) * p.hq + kvh * G + hcol) * D + grp * 8;
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) {
      qf[ds] = col < G ? *reinterpret_cast<const bf16x8*>(qrow + ds * 32) : bf16x8{};
    }
  }

  f32x4 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x4{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int64_t row_stride = static_cast<int64_t>(p.hkv) * D;
  const uint16_t* kbase = p.kc + (static_cast<int64_t>(b) * p.max_ctx * p.hkv + kvh) * D;
  const uint16_t* vbase = KEQV ? kbase : p.vc + (static_cast<int64_t>(b) * p.max_ctx * p.hkv + kvh) * D;

  for (int32_t kt = s_lo + wave * kKeys; kt < s_hi; kt += kWaves * kKeys) {
    // K rows in A layout (lane: key kt + 16*kk + col, d = ds*32 + grp*8).
    bf16x8 ka[2][kDS];
    bf16x8 va[KEQV ? 1 : 2][KEQV ? 1 : kDS];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int32_t key = kt + 16 * kk + col;
      const bool ok = key < s_hi;
      const uint16_t* kr = kbase + static_cast<int64_t>(key) * row_stride + grp * 8;
      const uint16_t* vr = vbase + static_cast<int64_t>(key) * row_stride + grp * 8;
#pragma unroll
      for (int ds = 0; ds < kDS; ++ds) {
        ka[kk][ds] = ok ? *reinterpret_cast<const bf16x8*>(kr + ds * 32) : bf16x8{};
        if (!KEQV) va[kk][ds] = ok ? *reinterpret_cast<const bf16x8*>(vr + ds * 32) : bf16x8{};
      }
    }
    // Value rows into this wave's LDS tile, row-major [key][d].
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int ds = 0; ds < kDS; ++ds) {
        const bf16x8 vv = KEQV ? ka[kk][ds] : va[KEQV ? 0 : kk][KEQV ? 0 : ds];
        *reinterpret_cast<bf16x8*>(&tile[(16 * kk + col) * kLd + ds * 32 + grp * 8]) = vv;
      }
    }
    // S^T for the two 16-key halves.
    f32x4 sacc[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      sacc[kk] = f32x4{};
#pragma unroll
      for (int ds = 0; ds < kDS; ++ds) {
        sacc[kk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk][ds], qf[ds], sacc[kk], 0, 0, 0);
      }
    }
    // Lane holds keys kt + 16*kk + grp*4 + r for head `col`.
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float t;
        if (CAP) {
          const float e = __builtin_amdgcn_exp2f(sacc[kk][r] * p.cap_in2);
          t = fmaf(-2.f * p.cap_log2, __builtin_amdgcn_rcpf(e + 1.f), p.cap_log2);
        } else {
          t = sacc[kk][r] * p.scale_log2;
        }
        const int32_t key = kt + 16 * kk + grp * 4 + r;
        t = key < s_hi ? t : -INFINITY;
        x[kk * 4 + r] = t;
        mx = fmaxf(mx, t);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    uint32_t pk[4];
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pk[r] = pack_bf16x2(__builtin_amdgcn_exp2f(x[2 * r] - m_use), __builtin_amdgcn_exp2f(x[2 * r + 1] - m_use));
      ls += lo_bf16(pk[r]) + hi_bf16(pk[r]);
    }
    l_run = fmaf(l_run, alpha, ls);
#pragma unroll
    for (int db = 0; db < kDB; ++db) o[db] *= alpha;
    // P^T operand: slots 0-3 = keys grp*4 + [0,4), slots 4-7 = keys 16 + grp*4 + [0,4).
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
    const int32_t i16 = lane & 15;
    const int32_t r0 = grp * 4 + (i16 >> 2);
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const int32_t cc = db * 16 + 4 * (i16 & 3);
      const i16x4 a0 = lds_read_tr16(&tile[r0 * kLd + cc]);
      const i16x4 a1 = lds_read_tr16(&tile[(r0 + 16) * kLd + cc]);
      const bf16x8 aop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, pb, o[db], 0, 0, 0);
    }
  }

  // ---- merge the 4 waves' partials of this chunk ----
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __shared__ float m_w[kWaves][16];
  __shared__ float l_w[kWaves][16];
  __syncthreads();   // every wave is done with its tile; LDS reused below
  if (grp == 0) {
    m_w[wave][col] = m_run;
    l_w[wave][col] = l_run;
  }
  __syncthreads();
  float m_all = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) m_all = fmaxf(m_all, m_w[w][col]);
  const float m_ref = m_all == -INFINITY ? 0.f : m_all;
  const float f = __builtin_amdgcn_exp2f(m_run - m_ref);
  float* obuf = reinterpret_cast<float*>(smem);   // [16 cols][D] fp32
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* dst = obuf + col * D + db * 16 + grp * 4 + r;
          const float v = o[db][r] * f;
          *dst = (w == 0) ? v : *dst + v;
        }
      }
    }
    __syncthreads();
  }
  const int64_t part = (static_cast<int64_t>(b) * p.hq + kvh * G) * p.n_split + split;
  for (int i = tid; i < G * D; i += kThreads) {
    const int32_t cc = i / D;
    const int32_t d = i % D;
    p.ws_o[(part + static_cast<int64_t>(cc) * p.n_split) * D + d] = obuf[cc * D + d];
  }
  if (tid < G) {
    float l_sum = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float mw = m_w[w][tid];
      l_sum += l_w[w][tid] * __builtin_amdgcn_exp2f(mw - (m_all == -INFINITY ? 0.f : m_all));
    }
    p.ws_m[part + static_cast<int64_t>(tid) * p.n_split] = m_all;
    p.ws_l[part + static_cast<int64_t>(tid) * p.n_split] = l_sum;
  }
}

// Merge the split partials of one (sequence, query head) in split order.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeParams p) {
  constexpr int kPer = D / 64 > 0 ? D / 64 : 1;   // elements per lane
  const int32_t head = blockIdx.x;
  const int32_t b = blockIdx.y;
  const int32_t lane = threadIdx.x;
  int32_t lo, ctx;
  seq_range(p, b, lo, ctx);
  const int32_t n_valid = ctx > lo ? (ctx - lo + p.chunk - 1) / p.chunk : 0;
  const int64_t part = (static_cast<int64_t>(b) * p.hq + head) * p.n_split;
  float m_all = -INFINITY;
  for (int s = 0; s < n_valid; ++s) m_all = fmaxf(m_all, p.ws_m[part + s]);
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float l_all = 0.f;
  const int32_t d0 = lane * kPer;
  for (int s = 0; s < n_valid; ++s) {
    const float ms = p.ws_m[part + s];
    const float f = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - m_all);
    l_all = fmaf(p.ws_l[part + s], f, l_all);
    if (d0 < D) {
      const float* src = p.ws_o + (part + s) * D + d0;
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] = fmaf(src[e], f, acc[e]);
    }
  }
  const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
  if (d0 < D) {
    uint16_t* dst = p.out + (static_cast<int64_t>(b) * p.hq + head) * D + d0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) dst[e] = f32_to_bf16(acc[e] * inv);
  }
  if (p.lse && lane == 0) {
    p.lse[static_cast<int64_t>(b) * p.hq + head] = l_all > 0.f ? (m_all + __log2f(l_all)) * kLn2 : -INFINITY;
  }
}

template <int D, int G, bool KEQV, bool CAP>
hipError_t launch_t(const DecodeArgs& a, const DecodeParams& prm, hipStream_t stream) {
  constexpr int kLd = D + kPad;
  size_t lds = static_cast<size_t>(kWaves) * kKeys * kLd * sizeof(uint16_t);
  const size_t merge = static_cast<size_t>(16) * D * sizeof(float);
  if (merge > lds) lds = merge;
  auto kfn = decode_split_kernel<D, G, KEQV, CAP>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<uint32_t>(a.n_split), static_cast<uint32_t>(a.hkv), static_cast<uint32_t>(a.batch));
  hipLaunchKernelGGL(kfn, grid, dim3(kThreads), lds, stream, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(static_cast<uint32_t>(a.hq), static_cast<uint32_t>(a.batch)),
                     dim3(64), 0, stream, prm);
  return hipGetLastError();
}

template <int D, int G>
hipError_t dispatch_flags(const DecodeArgs& a, const DecodeParams& prm, hipStream_t s) {
  const bool cap = a.softcap > 0.0;
  if (a.k_eq_v) return cap ? launch_t<D, G, true, true>(a, prm, s) : launch_t<D, G, true, false>(a, prm, s);
  return cap ? launch_t<D, G, false, true>(a, prm, s) : launch_t<D, G, false, false>(a, prm, s);
}

template <int D>
hipError_t dispatch_group(const DecodeArgs& a, const DecodeParams& prm, hipStream_t s) {
  switch (a.group) {
    case 1: return dispatch_flags<D, 1>(a, prm, s);
    case 2: return dispatch_flags<D, 2>(a, prm, s);
    case 4: return dispatch_flags<D, 4>(a, prm, s);
    case 8: return dispatch_flags<D, 8>(a, prm, s);
    case 16: return dispatch_flags<D, 16>(a, prm, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  DecodeParams prm;
  prm.q = static_cast<const uint16_t*>(a.q);
  prm.kc = static_cast<const uint16_t*>(a.k_cache);
  prm.vc = static_cast<const uint16_t*>(a.v_cache);
  prm.ctx_len = a.ctx_len;
  prm.out = static_cast<uint16_t*>(a.out);
  prm.lse = a.lse;
  prm.ws_o = a.ws_o;
  prm.ws_m = a.ws_m;
  prm.ws_l = a.ws_l;
  prm.max_ctx = a.max_ctx;
  prm.hq = a.hq;
  prm.hkv = a.hkv;
  prm.window = a.window;
  prm.chunk = a.chunk;
  prm.n_split = a.n_split;
  const double log2e = 1.4426950408889634;
  prm.scale_log2 = static_cast<float>(a.scale * log2e);
  prm.cap_in2 = a.softcap > 0.0 ? static_cast<float>(2.0 * a.scale * log2e / a.softcap) : 0.f;
  prm.cap_log2 = static_cast<float>(a.softcap * log2e);
  switch (a.dim) {
    case 64: return dispatch_group<64>(a, prm, stream);
    case 256: return dispatch_group<256>(a, prm, stream);
    case 512: return dispatch_group<512>(a, prm, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ga
