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
// The kernel streams rows (2 bytes read and 2 written per element), so it is
// laid out to keep HBM busy while spending few VALU instructions per row (a
// wave64 VALU instruction holds its SIMD for four cycles, and at 16-byte rows
// per lane that budget is small):
//  - persistent workgroups walk fixed-size items of consecutive (token, head)
//    rows; the next item's 16-byte row loads are issued before the current
//    item is worked on, so they stay in flight under its table build and row
//    math;
//  - the rotary frequencies theta^(-2i/r) / (2 pi pos_div), in revolutions
//    per position (fp64, rotary_rev_freq), and the norm weights are formed
//    once per workgroup; per item, each token's cos/sin (the fractional part
//    of p times the frequency in fp64, then the hardware fp32 cosine and sine,
//    rotary_cos_sin) goes to an LDS table laid out per element, with the
//    rotate-half sign folded in, so every element is one multiply and one FMA
//    (rotary_turn);
//  - each head row of width D is handled by D/8 lanes holding 8 contiguous
//    bf16; the RMS (and int8 absmax) reductions run inside those lanes with
//    DPP and lane swaps, and only on rows that have a norm weight.
// The rotate-half partner of element d (d +- r/2) sits r/16 lanes away at the
// same slot, so when r/16 is a power of two it is one lane shuffle (lane ^
// r/16); other rotary widths go through an LDS copy of the normalised row.
//
// Sources: RMSNorm QK-norm (google-gemma-4 atlas summary; weight used as w on
// Gemma 4, "Plain-weight RMSNorm", and as 1 + w on earlier Gemma), partial
// rotary ("Zero-pad partial rope", Gemma 4 page) and dual bases (Gemma 3 page,
// "Dual RoPE bases").
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "ga_device.h"
#include "ga_kernels.h"

namespace ga {

namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 7;               // 16-byte row loads per lane per item
// Tokens whose cos/sin tables (D entries of 8 bytes each) an item may touch:
// 32 KB of LDS up to D = 256, 28 KB at D = 512, at most 64 tokens.
constexpr int32_t tab_tokens(int32_t dim) {
  return dim <= 256 ? (4096 / dim < 64 ? 4096 / dim : 64) : 3584 / dim;
}

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
  int32_t tokens, rows_per_item;
  int32_t seq, hq, hkv, rotary_dim, max_ctx;   // max_ctx > 0: cache mode
  double rot_w1;    // theta^(-2/r)
  double rot_c0;    // 1 / (2 pi pos_div)
  float eps, offset;
};

// Reduction of v over the TPR consecutive lanes of a row, every lane getting
// the result: quad swaps, half-row and row mirrors (DPP), then the 16- and
// 32-lane swaps.  Each step combines a value with one from the other half of
// its group, so every lane forms the same operands and ends bitwise equal.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int TPR, typename Op>
__device__ __forceinline__ float row_reduce(float v, Op op) {
  if constexpr (TPR >= 2) v = op(v, dpp_mov<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (TPR >= 4) v = op(v, dpp_mov<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (TPR >= 8) v = op(v, dpp_mov<0x141>(v));   // row_half_mirror
  if constexpr (TPR >= 16) v = op(v, dpp_mov<0x140>(v));  // row_mirror
  if constexpr (TPR >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if constexpr (TPR >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return v;
}

// SHFL: the partner is lane ^ (r/16) (r/16 a power of two, r <= D); else LDS.
//
// Persistent: rows are numbered token-major over the whole launch (row
// t * heads + h is head h of token t: the q heads, then the k heads, then in
// cache mode the v heads, copied unchanged), and item j is rows
// [j * rpi, (j + 1) * rpi).  Workgroup w takes items w, w + G, w + 2G, ...
// (G = grid size) and issues the next item's row loads before it builds the
// current item's tables and processes its rows, so HBM always has the block's
// next rows in flight.
//
// Per token the cos/sin table has one entry per element d of the head row:
// (cos, -sin) of w_d for d < r/2, (cos, +sin) of w_{d-r/2} for r/2 <= d < r,
// so element d's result is x_d cos + partner_d * entry.y in both halves.
template <int TPR, bool SHFL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(SHFL ? 4 : 3))) void qk_prologue_kernel(
    ProParams p) {
  constexpr int32_t tpr = TPR;                  // lanes per row
  constexpr int32_t dim = TPR * 8;
  constexpr int32_t rpp = kThreads / TPR;       // rows per pass
  constexpr int32_t kTabTok = tab_tokens(dim);
  __shared__ double omega[256];
  __shared__ __attribute__((aligned(16))) float2 cs_tab[kTabTok * dim];
  __shared__ __attribute__((aligned(16))) float wtab[2][dim];   // q and k weights + offset
  __shared__ int64_t tok_pos[2][kTabTok];      // double-buffered: one item ahead
  __shared__ int32_t tok_b[2][kTabTok];
  __shared__ float rowbuf[SHFL ? 1 : kThreads * 8];
  lds_poison(omega, cs_tab, wtab, tok_pos, tok_b, rowbuf);

  const int32_t tid = threadIdx.x;
  const int32_t half = p.rotary_dim >> 1;
  const int32_t heads = p.hq + (p.k_in ? p.hkv : 0) + (p.v_in ? p.hkv : 0);
  const int32_t rpi = p.rows_per_item;
  const int64_t n_rows = static_cast<int64_t>(p.tokens) * heads;
  const int64_t n_items = (n_rows + rpi - 1) / rpi;
  const int32_t sub = tid / tpr;
  const int32_t lane = tid % tpr;
  const int32_t d0 = lane * 8;
  // Local row r (counted from the item's first token) is head r % heads of
  // token r / heads; the quotient is taken in fp32 as (r + 1/2) / heads: the
  // exact value is at least 1/(2 heads) from an integer and the two roundings
  // move it by under r * 2^-23 / heads, so the truncation is exact for r < 2^22.
  const float inv_heads = 1.0f / static_cast<float>(heads);
  auto split = [&](int32_t row, int32_t& tt, int32_t& hh) __attribute__((always_inline)) {
    tt = static_cast<int32_t>((static_cast<float>(row) + 0.5f) * inv_heads);
    hh = row - tt * heads;
  };
  // Element offset of head hh of token tok in its row-layout array.
  auto row_off = [&](int32_t tok, int32_t hh) __attribute__((always_inline)) -> int64_t {
    const int32_t hx = hh < p.hq ? p.hq : p.hkv;
    const int32_t hk = hh - p.hq;
    const int32_t hi = hh < p.hq ? hh : (hk < p.hkv ? hk : hk - p.hkv);
    return (static_cast<int64_t>(tok) * hx + hi) * dim + d0;
  };
  // First token of item j and the item's first row counted from that token.
  auto item_start = [&](int64_t j, int32_t& tok_first, int32_t& r0) __attribute__((always_inline)) {
    const int64_t row0 = j * rpi;
    tok_first = static_cast<int32_t>(row0 / heads);
    r0 = static_cast<int32_t>(row0 - static_cast<int64_t>(tok_first) * heads);
  };
  auto load_item = [&](int64_t j, u32x4 (&buf)[kLoads]) __attribute__((always_inline)) {
    int32_t tok_first = 0, r0 = 0, lim = 0;
    if (j < n_items) {
      item_start(j, tok_first, r0);
      lim = static_cast<int32_t>(min<int64_t>(rpi, n_rows - j * rpi));
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      buf[i] = u32x4{0u, 0u, 0u, 0u};
      const int32_t r = i * rpp + sub;
      if (r < lim) {
        int32_t tt, hh;
        split(r + r0, tt, hh);
        const uint16_t* base = hh < p.hq ? p.q_in : (hh < p.hq + p.hkv ? p.k_in : p.v_in);
        buf[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + row_off(tok_first + tt, hh)));
      }
    }
  };

  // Sequence and position of token tid of item j: fetch_tok issues the
  // position-array load early (so waiting for it does not wait for the row
  // loads issued after it), commit_tok stores the result into buffer buf.
  struct TokInfo {
    int32_t t, b, s, raw;
  };
  auto fetch_tok = [&](int64_t j) __attribute__((always_inline)) -> TokInfo {
    TokInfo ti{-1, 0, 0, 0};
    if (j >= n_items) return ti;
    int32_t tok_first, r0;
    item_start(j, tok_first, r0);
    const int32_t lim = static_cast<int32_t>(min<int64_t>(rpi, n_rows - j * rpi));
    const int32_t ntok = (r0 + lim - 1) / heads + 1;        // <= kTabTok <= kThreads
    if (tid < ntok) {
      const int32_t token = tok_first + tid;
      ti.t = tid;
      ti.b = token / p.seq;
      ti.s = token - ti.b * p.seq;
      if (p.ctx_len) ti.raw = p.ctx_len[ti.b];
      else if (p.pos0) ti.raw = p.pos0[ti.b];
    }
    return ti;
  };
  auto commit_tok = [&](const TokInfo& ti, int buf) __attribute__((always_inline)) {
    if (ti.t < 0) return;
    int64_t pos;
    if (p.ctx_len) {
      const int32_t c = ti.raw < 0 ? 0 : (ti.raw > p.max_ctx ? p.max_ctx : ti.raw);
      pos = static_cast<int64_t>(c) - p.seq + ti.s;
    } else {
      pos = static_cast<int64_t>(ti.raw) + ti.s;
    }
    tok_b[buf][ti.t] = ti.b;
    tok_pos[buf][ti.t] = pos;
  };

  int64_t j = blockIdx.x;
  u32x4 cur[kLoads];
  TokInfo nt_cur = fetch_tok(j);
  load_item(j, cur);
  // Once per workgroup: the frequencies in revolutions per position;
  // the norm weights; the pass-through entries.
  for (int32_t i = tid; i < half; i += kThreads) omega[i] = rotary_rev_freq(i, p.rot_w1, p.rot_c0);
  for (int32_t d = tid; d < dim; d += kThreads) {
    wtab[0][d] = p.qw ? p.qw[d] + p.offset : 1.0f;
    wtab[1][d] = p.kw ? p.kw[d] + p.offset : 1.0f;
  }
  for (int32_t e = tid; e < kTabTok * dim; e += kThreads)
    if (e % dim >= p.rotary_dim) cs_tab[e] = make_float2(1.0f, 0.0f);
  const bool q_norm = p.qw != nullptr, k_norm = p.kw != nullptr;

  const int32_t pmask = p.rotary_dim >> 4;   // partner lane distance (SHFL)
  const bool any_keep = p.rotary_dim < dim || p.v_in != nullptr;
  // One item: tables, then its rows from cur (token positions in buffer it).
  auto step = [&](int64_t j, int it, const u32x4 (&cur)[kLoads]) __attribute__((always_inline)) {
    int32_t tok_first, r0;
    item_start(j, tok_first, r0);
    const int32_t lim = static_cast<int32_t>(min<int64_t>(rpi, n_rows - j * rpi));
    const int32_t ntok = (r0 + lim - 1) / heads + 1;

    // The cos/sin tables of this item (the barrier first lets every wave
    // finish reading the previous item's tables and makes this item's token
    // positions visible).
    __syncthreads();
    for (int32_t e = tid; e < ntok * half; e += kThreads) {
      const int32_t tt = e / half;
      const int32_t i = e - tt * half;
      const float2 cs = rotary_cos_sin(static_cast<double>(tok_pos[it][tt]), omega[i]);
      cs_tab[tt * dim + i] = make_float2(cs.x, -cs.y);
      cs_tab[tt * dim + half + i] = make_float2(cs.x, cs.y);
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int32_t r = i * rpp + sub;
      const bool in_range = r < lim;
      int32_t tt, hh;
      split(in_range ? r + r0 : 0, tt, hh);
      const int32_t token = tok_first + tt;
      const bool is_q = hh < p.hq;
      const bool is_v = hh >= p.hq + p.hkv;
      // Destination; k and v rows outside the cache are skipped.
      uint16_t* dst = nullptr;
      int8_t* cdst = nullptr;
      float* sdst = nullptr;
      bool active = in_range;
      if (is_q) {
        dst = p.q_out + row_off(token, hh);
      } else if (p.max_ctx > 0) {
        const int32_t kh = is_v ? hh - p.hq - p.hkv : hh - p.hq;
        const int64_t pos = tok_pos[it][tt];
        const int32_t b = tok_b[it][tt];
        if (pos < 0 || pos >= p.max_ctx) active = false;
        const int64_t crow = (static_cast<int64_t>(b) * p.max_ctx + pos) * p.hkv + kh;
        if (p.k_scales) {
          cdst = (is_v ? p.v_codes : p.k_codes) + crow * dim + d0;
          sdst = (is_v ? p.v_scales : p.k_scales) + (static_cast<int64_t>(b) * p.hkv + kh) * p.max_ctx + pos;
        } else {
          dst = (is_v ? p.v_out : p.k_out) + crow * dim + d0;
        }
      } else {
        dst = p.k_out + row_off(token, hh);
      }

      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = lo_bf16(cur[i][e]);
        x[2 * e + 1] = hi_bf16(cur[i][e]);
      }
      // RMSNorm where this side has a weight: x * rsqrt(mean x^2 + eps) * (w +
      // offset).  All lanes of a row take the same branch, and the reduction
      // stays inside the row.
      const bool norm = is_q ? q_norm : (!is_v && k_norm);
      if (norm) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
        ss = row_reduce<TPR>(ss, [](float a, float b) { return a + b; });
        const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / static_cast<float>(dim)) + p.eps);
        const float* wrow = wtab[is_q ? 0 : 1] + d0;
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(wrow);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(wrow + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = x[e] * inv * w0[e];
          x[e + 4] = x[e + 4] * inv * w1[e];
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
      const f32x4* cs = reinterpret_cast<const f32x4*>(cs_tab + tt * dim + d0);
      float y[8];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const f32x4 c2 = cs[e2];                 // entries d0 + 2 e2 and d0 + 2 e2 + 1
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = 2 * e2 + h;
          const float rot = rotary_turn(x[e], partner[e], c2[2 * h], c2[2 * h + 1]);
          y[e] = any_keep && (is_v || d0 + e >= p.rotary_dim) ? x[e] : rot;   // v rows, pass-through part
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
        amax = row_reduce<TPR>(amax, [](float a, float b) { return fmaxf(a, b); });
        if (active && cdst) {
          const float sc = amax / 127.0f;
          uint32_t cw[2] = {0u, 0u};
          if (sc > 0.f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = (e & 1) ? hi_bf16(o[e >> 1]) : lo_bf16(o[e >> 1]);
              const int32_t q = static_cast<int32_t>(__builtin_rintf(v / sc));
              cw[e >> 2] |= (static_cast<uint32_t>(q) & 0xffu) << (8 * (e & 3));
            }
          }
          *reinterpret_cast<u32x2*>(cdst) = u32x2{cw[0], cw[1]};
          if (lane == 0) *sdst = sc;
        } else if (active) {
          *reinterpret_cast<u32x4*>(dst) = o;
        }
      } else if (active) {
        *reinterpret_cast<u32x4*>(dst) = o;
      }
    }
  };

  // Two named buffers in turn.  Each item starts by waiting for all of its
  // loads (issued during the previous item), then issues the next item's, so
  // those stay in flight while this item's tables are built and its rows
  // processed.  Token positions go to buffer it; the other buffer may still
  // be read by waves processing the previous item, and this one was last
  // read two items ago, before the previous item's first barrier.
  constexpr int kWaitVm0 = 0x0F70;          // s_waitcnt vmcnt(0), other counters untouched
  u32x4 alt[kLoads];
  TokInfo nt_alt;
  for (int it = 0;;) {
    if (j >= n_items) break;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    commit_tok(nt_cur, it);
    nt_alt = fetch_tok(j + gridDim.x);
    load_item(j + gridDim.x, alt);
    step(j, it, cur);
    j += gridDim.x;
    it ^= 1;
    if (j >= n_items) break;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    commit_tok(nt_alt, it);
    nt_cur = fetch_tok(j + gridDim.x);
    load_item(j + gridDim.x, cur);
    step(j, it, alt);
    j += gridDim.x;
    it ^= 1;
  }
}

// Resident workgroups per CU of one instantiation on the current device
// (cached per device; the value is the same whichever thread computes it).
template <int TPR, bool SHFL>
int resident_grid() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, qk_prologue_kernel<TPR, SHFL>, kThreads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 || cus < 1)
    return 0;
  v = per_cu * cus;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
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
  p.tokens = static_cast<int32_t>(tokens);
  p.seq = a.seq;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.rotary_dim = a.rotary_dim;
  p.rot_w1 = a.rotary_dim > 0 ? rotary_w1(a.theta, a.rotary_dim) : 0.0;
  p.rot_c0 = rotary_c0(a.pos_div);
  p.eps = a.eps;
  p.offset = a.offset;
  // Rows per item: kLoads passes of the block, fewer when the tokens an item
  // can touch would not fit the LDS tables.
  const int32_t heads = a.hq + (a.k_in ? a.hkv : 0) + (a.v_in ? a.hkv : 0);
  if (heads < 1) return hipErrorNotSupported;
  const int32_t rpp = kThreads / (a.dim >> 3);
  const int32_t tab_tok = tab_tokens(a.dim);     // >= 7
  // An item of n rows touches at most (n - 1) / heads + 2 tokens.
  const int32_t rpi = std::max(1, std::min(kLoads * rpp, (tab_tok - 2) * heads + 1));
  p.rows_per_item = rpi;
  const int64_t items = (tokens * heads + rpi - 1) / rpi;
  const int32_t r16 = a.rotary_dim >> 4;
  const bool shfl = a.rotary_dim % 16 == 0 && r16 > 0 && (r16 & (r16 - 1)) == 0 && a.rotary_dim <= a.dim;
  const bool use_shfl = shfl || a.rotary_dim == 0;
  hipError_t err = hipSuccess;
  auto go = [&](auto tpr_c) {
    constexpr int T = decltype(tpr_c)::value;
    const int resident = use_shfl ? resident_grid<T, true>() : resident_grid<T, false>();
    if (resident < 1) {
      err = hipErrorInvalidDeviceFunction;
      return;
    }
    const uint32_t grid = static_cast<uint32_t>(std::min<int64_t>(items, resident));
    if (use_shfl) {
      err = launch_kernel(qk_prologue_kernel<T, true>, dim3(grid), dim3(kThreads), stream, p);
    } else {
      err = launch_kernel(qk_prologue_kernel<T, false>, dim3(grid), dim3(kThreads), stream, p);
    }
  };
  switch (a.dim >> 3) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 8: go(std::integral_constant<int, 8>{}); break;
    case 16: go(std::integral_constant<int, 16>{}); break;
    case 32: go(std::integral_constant<int, 32>{}); break;
    case 64: go(std::integral_constant<int, 64>{}); break;
    default: return hipErrorNotSupported;
  }
  return err;
}

}  // namespace ga
