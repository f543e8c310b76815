// Fused QK-norm + dual-base partial rotary prologue (gfx950).
//
// Two modes: rows in, rows out (positions pos0[b] + s); or cache mode, where
// the seq new tokens of each sequence sit at positions ctx_len[b] - seq + s
// (or pos0[b] + s without ctx_len) and their processed keys (and raw values)
// are written straight into the contiguous caches at those rows -- the cache
// append of a decode or chunked-prefill step.  An int8 cache stores each
// (token, head) vector of the bf16-rounded result as codes
// round-half-even(x / s) with s = max|x| / 127 (fp32 division), plus s.
//
// One workgroup per group of kTok consecutive tokens (flattened over batch and
// sequence).  The rotary frequencies w_i = theta^(-2i/r) are formed once per
// workgroup in fp64, then each token's cos/sin(p * w_i) table (angle reduced
// modulo 2*pi in fp64, fp32 sincos) goes to LDS; the row loads are issued
// before the tables are built so their latency overlaps it.  Each head row of
// width D is handled by D/8 lanes holding 8 contiguous bf16 (one 16-byte
// load); the RMS reduction is a butterfly inside those lanes.  The rotate-half
// partner of element d (d +- r/2) sits r/16 lanes away at the same slot, so
// when r/16 is a power of two it is one lane shuffle (lane ^ r/16); other
// rotary widths go through an LDS copy of the normalised row.
//
// Sources: RMSNorm QK-norm (google-gemma-4 atlas summary; weight used as w on
// Gemma 4, "Plain-weight RMSNorm", and as 1 + w on earlier Gemma), partial
// rotary ("Zero-pad partial rope", Gemma 4 page) and dual bases (Gemma 3 page,
// "Dual RoPE bases").
#include "ga_device.h"
#include "ga_kernels.h"

namespace ga {

namespace {

constexpr int kThreads = 256;
constexpr int kTok = 4;                 // tokens per workgroup
constexpr double kTwoPi = 6.283185307179586476925286766559;

struct ProParams {
  const uint16_t* q_in;
  const uint16_t* k_in;
  uint16_t* q_out;
  uint16_t* k_out;
  const float* qw;
  const float* kw;
  const int32_t* pos0;
  const int32_t* ctx_len;     // cache mode: positions ctx_len[b] - seq + s
  const uint16_t* v_in;       // cache mode: raw values copied into v_out
  uint16_t* v_out;
  int8_t* k_codes;            // int8 cache mode (k_scales set): codes [B,max_ctx,Hkv,D]
  float* k_scales;            //   and scales [B,Hkv,max_ctx] replace k_out / v_out
  int8_t* v_codes;
  float* v_scales;
  int64_t tokens;
  int32_t seq, hq, hkv, dim, rotary_dim, max_ctx;   // max_ctx > 0: cache mode
  double theta;
  double pos_div;
  float eps, offset;
};

// Position of token s of sequence b.
__device__ __forceinline__ int64_t token_pos(const ProParams& p, int32_t b, int32_t s) {
  if (p.ctx_len) {
    int32_t c = p.ctx_len[b];
    c = c < 0 ? 0 : (c > p.max_ctx ? p.max_ctx : c);
    return static_cast<int64_t>(c) - p.seq + s;
  }
  return static_cast<int64_t>(p.pos0 ? p.pos0[b] : 0) + s;
}

// SHFL: the partner is lane ^ (r/16) (r/16 a power of two, r <= D); else LDS.
template <bool SHFL>
__global__ __launch_bounds__(kThreads) void qk_prologue_kernel(ProParams p) {
  __shared__ double omega[256];
  __shared__ float2 cs_tab[kTok][256];
  __shared__ float rowbuf[SHFL ? 1 : kThreads * 8];

  const int32_t tid = threadIdx.x;
  const int32_t half = p.rotary_dim >> 1;
  const int32_t dim = p.dim;
  const int32_t tpr = dim >> 3;                 // lanes per row (power of two <= 64)
  const int32_t rows_per_pass = kThreads / tpr;
  const int32_t heads = p.hq + (p.k_in ? p.hkv : 0) + (p.v_in ? p.hkv : 0);
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const int32_t rows = kTok * heads;
  const int32_t sub = tid / tpr;
  const int32_t lane = tid % tpr;
  const int32_t d0 = lane * 8;

  // Row r of this workgroup: token tok0 + r / heads, head r % heads: the q
  // heads, then the k heads, then (cache mode) the v heads, which are copied
  // unchanged.  In cache mode k and v rows go to cache row pos of their token
  // and are skipped when that row is outside the cache; in int8 cache mode
  // they go to the code row (cdst) and the scale slot (sdst) instead of dst.
  struct RowDst {
    uint16_t* dst;
    int8_t* cdst;
    float* sdst;
  };
  auto row_ptrs = [&](int32_t row, const uint16_t*& src, RowDst& out, const float*& w, bool& copy) -> bool {
    const int32_t tt = row / heads;
    const int32_t hh = row % heads;
    const int64_t token = tok0 + tt;
    copy = false;
    out = RowDst{nullptr, nullptr, nullptr};
    if (row >= rows || token >= p.tokens) return false;
    if (hh < p.hq) {
      const int64_t off = (token * p.hq + hh) * dim + d0;
      src = p.q_in + off;
      out.dst = p.q_out + off;
      w = p.qw;
      return true;
    }
    const int32_t kh = (hh - p.hq) % p.hkv;
    const bool is_v = hh >= p.hq + p.hkv;
    src = (is_v ? p.v_in : p.k_in) + (token * p.hkv + kh) * dim + d0;
    w = is_v ? nullptr : p.kw;
    copy = is_v;
    if (p.max_ctx > 0) {
      const int32_t b = static_cast<int32_t>(token / p.seq);
      const int64_t pos = token_pos(p, b, static_cast<int32_t>(token % p.seq));
      if (pos < 0 || pos >= p.max_ctx) return false;
      const int64_t crow = (static_cast<int64_t>(b) * p.max_ctx + pos) * p.hkv + kh;
      if (p.k_scales) {
        out.cdst = (is_v ? p.v_codes : p.k_codes) + crow * dim + d0;
        out.sdst = (is_v ? p.v_scales : p.k_scales) + (static_cast<int64_t>(b) * p.hkv + kh) * p.max_ctx + pos;
      } else {
        out.dst = (is_v ? p.v_out : p.k_out) + crow * dim + d0;
      }
    } else {
      out.dst = p.k_out + (token * p.hkv + kh) * dim + d0;
    }
    return true;
  };

  // Issue the first pass's row load before building the tables.
  u32x4 raw = u32x4{0u, 0u, 0u, 0u};
  {
    const uint16_t* src;
    RowDst od;
    const float* w;
    bool cp;
    if (row_ptrs(sub, src, od, w, cp)) raw = *reinterpret_cast<const u32x4*>(src);
  }

  // (p / pos_div) * w_i, formed as p * (w_i / pos_div).
  for (int32_t i = tid; i < half; i += kThreads) omega[i] = pow(p.theta, -2.0 * i / p.rotary_dim) / p.pos_div;
  __syncthreads();
  for (int32_t e = tid; e < kTok * half; e += kThreads) {
    const int32_t tt = e / half;
    const int32_t i = e % half;
    const int64_t token = tok0 + tt;
    float sn = 0.f, cn = 1.f;
    if (token < p.tokens) {
      const int32_t b = static_cast<int32_t>(token / p.seq);
      const int32_t s = static_cast<int32_t>(token % p.seq);
      const int64_t pos = token_pos(p, b, s);
      double ang = fmod(static_cast<double>(pos) * omega[i], kTwoPi);
      if (ang < 0) ang += kTwoPi;
      sincosf(static_cast<float>(ang), &sn, &cn);
    }
    cs_tab[tt][i] = make_float2(cn, sn);
  }
  __syncthreads();

  const int32_t pmask = p.rotary_dim >> 4;   // partner lane distance (SHFL)
  for (int32_t row0 = 0; row0 < rows; row0 += rows_per_pass) {
    const int32_t row = row0 + sub;
    const uint16_t* src = nullptr;
    RowDst od;
    const float* w = nullptr;
    bool copy = false;
    const bool active = row_ptrs(row, src, od, w, copy);
    // prefetch the next pass's row
    u32x4 next = u32x4{0u, 0u, 0u, 0u};
    if (row0 + rows_per_pass < rows) {
      const uint16_t* s2;
      RowDst d2;
      const float* w2;
      bool c2;
      if (row_ptrs(row + rows_per_pass, s2, d2, w2, c2)) next = *reinterpret_cast<const u32x4*>(s2);
    }
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = lo_bf16(raw[e]);
      x[2 * e + 1] = hi_bf16(raw[e]);
    }
    // RMSNorm (only when this side has a weight).
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    for (int m = tpr >> 1; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (active && w) {
      const float inv = 1.0f / sqrtf(ss / static_cast<float>(dim) + p.eps);
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + d0);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + d0 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = x[e] * inv * (w0[e] + p.offset);
        x[e + 4] = x[e + 4] * inv * (w1[e] + p.offset);
      }
    }
    float partner[8];
    if constexpr (SHFL) {
#pragma unroll
      for (int e = 0; e < 8; ++e) partner[e] = __shfl_xor(x[e], pmask, 64);
    } else {
      float* rb = rowbuf + sub * dim;
#pragma unroll
      for (int e = 0; e < 8; ++e) rb[d0 + e] = x[e];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int32_t d = d0 + e;
        partner[e] = d < half ? rb[d + half] : (d < p.rotary_dim ? rb[d - half] : 0.f);
      }
      __syncthreads();
    }
    // Rows past the end take the last token's table (their results are dropped).
    const int32_t tt = min(row / heads, kTok - 1);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int32_t d = d0 + e;
      if (copy) {
        y[e] = x[e];
      } else if (d < half) {
        const float2 c = cs_tab[tt][d];
        y[e] = x[e] * c.x - partner[e] * c.y;
      } else if (d < p.rotary_dim) {
        const float2 c = cs_tab[tt][d - half];
        y[e] = x[e] * c.x + partner[e] * c.y;
      } else {
        y[e] = x[e];
      }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
    if (p.k_scales) {
      // int8 cache mode: every lane joins the row's max reduction.
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(o[e])), fabsf(hi_bf16(o[e]))));
      for (int m = tpr >> 1; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
      if (active && od.cdst) {
        const float sc = amax / 127.0f;
        uint32_t cw[2] = {0u, 0u};
        if (sc > 0.f) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = (e & 1) ? hi_bf16(o[e >> 1]) : lo_bf16(o[e >> 1]);
            const int32_t c = static_cast<int32_t>(__builtin_rintf(v / sc));
            cw[e >> 2] |= (static_cast<uint32_t>(c) & 0xffu) << (8 * (e & 3));
          }
        }
        *reinterpret_cast<u32x2*>(od.cdst) = u32x2{cw[0], cw[1]};
        if (lane == 0) *od.sdst = sc;
      } else if (active) {
        *reinterpret_cast<u32x4*>(od.dst) = o;
      }
    } else if (active) {
      *reinterpret_cast<u32x4*>(od.dst) = o;
    }
    raw = next;
  }
}

}  // namespace

hipError_t launch_qk_prologue(const PrologueArgs& a, hipStream_t stream) {
  const int64_t tokens = static_cast<int64_t>(a.batch) * a.seq;
  if (tokens == 0) return hipSuccess;
  ProParams p;
  p.q_in = static_cast<const uint16_t*>(a.q_in);
  p.k_in = static_cast<const uint16_t*>(a.k_in);
  p.q_out = static_cast<uint16_t*>(a.q_out);
  p.k_out = static_cast<uint16_t*>(a.k_out);
  p.qw = a.q_norm_w;
  p.kw = a.k_norm_w;
  p.pos0 = a.pos0;
  p.ctx_len = a.ctx_len;
  p.v_in = static_cast<const uint16_t*>(a.v_in);
  p.v_out = static_cast<uint16_t*>(a.v_out);
  p.k_codes = static_cast<int8_t*>(a.k_codes);
  p.k_scales = a.k_scales;
  p.v_codes = static_cast<int8_t*>(a.v_codes);
  p.v_scales = a.v_scales;
  p.max_ctx = a.max_ctx;
  p.tokens = tokens;
  p.seq = a.seq;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.dim = a.dim;
  p.rotary_dim = a.rotary_dim;
  p.theta = a.theta;
  p.pos_div = a.pos_div > 0.0 ? a.pos_div : 1.0;
  p.eps = a.eps;
  p.offset = a.offset;
  const int64_t blocks = (tokens + kTok - 1) / kTok;
  const int32_t r16 = a.rotary_dim >> 4;
  const bool shfl = a.rotary_dim % 16 == 0 && r16 > 0 && (r16 & (r16 - 1)) == 0 && a.rotary_dim <= a.dim;
  if (shfl || a.rotary_dim == 0) {
    hipLaunchKernelGGL(qk_prologue_kernel<true>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(qk_prologue_kernel<false>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace ga
