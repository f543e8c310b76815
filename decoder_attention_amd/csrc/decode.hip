// Split-KV decode attention over a contiguous KV cache (gfx950).
//
// q_len query tokens per sequence (1 for the decode step of generate(); more
// for chunked prefill or draft verification), at positions ctx - q_len ..
// ctx - 1, each causal and windowed on its own position.  The keys a sequence
// reads -- back to the window of its first query on local layers, [0, ctx) on
// global layers -- are laid end to end over all sequences (a plan kernel
// writes the prefix sums); the P workgroups of each (KV head, block of 16
// (token, head) columns) take equal consecutive ranges of that line, so every
// workgroup does the same work whatever the mix of context lengths.  A range
// that crosses sequence boundaries yields one unnormalised partial (m, l, o)
// per sequence it touches, stored at slot w + b (unique: along the monotone
// path of (workgroup, sequence) pairs w + b increases at every step); a
// combine kernel merges each (sequence, token, head)'s partials in order.
//
// Inside a workgroup (2 waves) tiles of 16 cache rows stream HBM -> LDS with
// the direct-to-LDS loads into two slots per team (one tile in flight while
// the other is computed), rows XOR-swizzled by 16-byte chunk:
//   * S^T[16 keys x 16 cols] = K . Q^T (v_mfma_f32_16x16x32_bf16) with the g
//     heads as columns (padded to 16), so each lane owns one head and the
//     softmax reductions are over the four lanes that share it;
//   * O^T += V^T . P^T with V^T read transposed from the row-major tile
//     (ds_read_b64_tr_b16); with keys-as-values the one tile is both.
// Cache rows outside the sequence's range are never loaded.
//
// Sources: generate() decoding over cached keys and values (Gemma 4 page, API;
// the atlas summary on KV caches bounded by the window on local layers), the
// window, soft cap, scaling and keys-as-values as for prefill.
#include <type_traits>
#include <utility>

#include "ga_device.h"
#include "ga_kernels.h"

namespace ga {

namespace {

constexpr int kTK = 16;     // keys per wave tile
// Cache policy of the cache copies: non-temporal (each cache row is read once
// per call; a plain streaming read measured ~8% slower than a non-temporal one).
constexpr int kStreamAux = 2;

// s_waitcnt vmcnt(N) (gfx9 encoding: low 4 bits and bits 14-15), leaving the
// export and LDS counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* ctx_len;
  const int32_t* kv_start;    // first cache row each sequence may read (null: 0)
  uint16_t* out;
  float* lse;
  float* ws_o;
  float* ws_m;
  float* ws_l;
  const float* ks;            // int8 caches: scales [B, Hkv, max_ctx] of keys and values
  const float* vs;
  int64_t* prefix;            // workspace: [B + 1] prefix sums of the readable spans
  int32_t* lo;                // workspace: [B] first readable key of each sequence
  int32_t batch, max_ctx, hq, hkv, window, n_wg;   // n_wg: workgroups per (KV head, column block)
  int32_t per_seq;            // workgroup w takes sequence w whole (n_wg = batch)
  int32_t q_len, n_cb;        // query tokens per sequence; 16-column blocks per KV head
  int32_t xcd_log2;           // the dispatcher deals linear block ids round-robin over 2^xcd_log2 XCDs
  float scale_log2, cap_in2, cap_log2;
};

// Keys sequence b can read: [lo, ctx).  With q_len query tokens at positions
// ctx - q_len .. ctx - 1, a local layer reads back to the window of the first;
// a left-padded cache starts at kv_start[b].
__device__ __forceinline__ void seq_range(const DecodeParams& p, int32_t b, int32_t& lo, int32_t& ctx) {
  int32_t c = p.ctx_len[b];
  c = c < 0 ? 0 : (c > p.max_ctx ? p.max_ctx : c);
  const int32_t span = p.window > 0 ? min(c, p.window + p.q_len - 1) : c;
  ctx = c;
  lo = c - span;
  if (p.kv_start) lo = min(max(lo, p.kv_start[b]), c);
}

// One workgroup: the readable span of every sequence and their exclusive
// prefix sums (int64), written to the workspace.
constexpr int kPlanThreads = 256;
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodeParams p) {
  __shared__ int64_t wsum[kPlanThreads / 64];
  lds_poison(wsum);
  const int32_t t = threadIdx.x;
  const int32_t per = (p.batch + kPlanThreads - 1) / kPlanThreads;
  const int32_t b0 = min(p.batch, t * per), b1 = min(p.batch, b0 + per);
  int64_t mine = 0;
  for (int32_t b = b0; b < b1; ++b) {
    int32_t lo, ctx;
    seq_range(p, b, lo, ctx);
    p.lo[b] = lo;
    mine += ctx - lo;
  }
  // inclusive scan of the per-thread sums: within the wave, then across waves
  int64_t inc = mine;
  const int32_t lane = t & 63, wave = t >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t up = __shfl_up(inc, d, 64);
    if (lane >= d) inc += up;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int64_t base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  // exclusive prefix of this thread's first sequence; the spans are
  // recomputed rather than held
  int64_t run = base + inc - mine;
  for (int32_t b = b0; b < b1; ++b) {
    int32_t lo, ctx;
    seq_range(p, b, lo, ctx);
    p.prefix[b] = run;
    run += ctx - lo;
  }
  if (t == kPlanThreads - 1) p.prefix[p.batch] = base + inc;
}

// Workgroup w of P covers keys [w*T/P, (w+1)*T/P) of the line (integer division).
__device__ __forceinline__ int64_t wg_start(int64_t w, int64_t total, int64_t n_wg) { return (w * total) / n_wg; }

// The workgroup whose range holds key x of the line (0 <= x < total).
__device__ __forceinline__ int64_t wg_of(int64_t x, int64_t total, int64_t n_wg) {
  int64_t w = (x * n_wg) / total;
  while (w + 1 < n_wg && wg_start(w + 1, total, n_wg) <= x) ++w;
  while (w > 0 && wg_start(w, total, n_wg) > x) --w;
  return w;
}

// Block placement.  Work item (KV head, key range w) is kvh + Hkv * w; its
// n_cb column blocks take linear ids nx apart (nx = the XCD count), so they run
// on one XCD (linear ids are dealt round-robin to the XCDs) at about the same
// time, and that XCD's L2 serves the cache rows they all read.  With one
// column block the order is the item order: the KV heads of one range side by
// side.
struct DecodeBlock {
  int32_t kvh, cb, w;
  bool valid;
};
__device__ __forceinline__ DecodeBlock decode_block(const DecodeParams& p) {
  const int32_t L = static_cast<int32_t>(blockIdx.x);
  const int32_t nx = 1 << p.xcd_log2;
  const int32_t per = nx * p.n_cb;
  const int32_t g = L / per;
  const int32_t r = L - g * per;
  const int32_t item = g * nx + (r & (nx - 1));
  DecodeBlock d;
  d.valid = item < p.hkv * p.n_wg;
  d.kvh = item % p.hkv;
  d.w = item / p.hkv;
  d.cb = r >> p.xcd_log2;
  return d;
}
inline int64_t decode_grid(int32_t hkv, int32_t n_wg, int32_t n_cb, int32_t xcd_log2) {
  const int64_t items = static_cast<int64_t>(hkv) * n_wg;
  const int64_t nx = int64_t{1} << xcd_log2;
  return n_cb == 1 ? items : (items + nx - 1) / nx * nx * n_cb;
}

// Calls f(b, s_lo, s_hi, ctx) for every sequence b that this workgroup's range
// touches, with [s_lo, s_hi) the sequence's keys in the range; uniform across
// the workgroup.  The caller separates consecutive calls with a barrier.  One
// workgroup per sequence: f runs for the sequence even when it has no keys
// to read (s_lo == s_hi), since that workgroup writes the sequence's output.
template <class F>
__device__ __forceinline__ void for_each_segment(const DecodeParams& p, int32_t wg, F&& f) {
  if (p.per_seq) {
    const int32_t b = wg;
    int32_t lo, ctx;
    seq_range(p, b, lo, ctx);
    f(b, lo, ctx, ctx);
    return;
  }
  const int64_t total = p.prefix[p.batch];
  const int64_t w = wg;
  const int64_t x0 = wg_start(w, total, p.n_wg);
  const int64_t x1 = wg_start(w + 1, total, p.n_wg);
  if (x0 >= x1) return;
  // first sequence: the last b with prefix[b] <= x0
  int32_t lo_b = 0, hi_b = p.batch - 1;
  while (lo_b < hi_b) {
    const int32_t mid = (lo_b + hi_b + 1) >> 1;
    if (p.prefix[mid] <= x0) lo_b = mid;
    else hi_b = mid - 1;
  }
  for (int32_t b = lo_b; b < p.batch; ++b) {
    const int64_t pb = p.prefix[b], pe = p.prefix[b + 1];
    const int64_t a = x0 > pb ? x0 : pb;
    const int64_t e = x1 < pe ? x1 : pe;
    if (a < e) {
      const int32_t base = p.lo[b];
      f(b, base + static_cast<int32_t>(a - pb), base + static_cast<int32_t>(e - pb),
        base + static_cast<int32_t>(pe - pb));
    }
    if (pe >= x1) break;
  }
}

// XOR pattern f(r) of the 16-byte chunks of LDS row r in [0, 16).  The
// score product's ds_read_b128 phase (16 lanes) reads rows 0-15 at one chunk:
// f must take 16 distinct values (D >= 128: one row spans whole bank cycles),
// or 8 distinct values within each row parity (D = 64: two rows per 256-byte
// cycle).  The value transpose read's 32-lane phase reads rows 0-7 (or 8-15)
// at an aligned chunk pair {c, c+1}: the pairs {c ^ f(r), (c+1) ^ f(r)} must
// be disjoint, i.e. f(r) >> 1 distinct over those rows (within a parity at
// D = 64).  Bits 1-3 from r & 7 and bit 0 from r >> 3 satisfy both.
template <int D>
__device__ __forceinline__ int32_t dswz(int32_t r) {
  if constexpr (D >= 128) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

// The lane index, hidden from loop-invariant code motion, so lane-derived
// offsets are recomputed per tile instead of held in registers.
__device__ __forceinline__ int32_t lane_here() {
  int32_t l = static_cast<int32_t>(threadIdx.x);
  asm volatile("" : "+v"(l));
  return l & 63;
}

// Workgroup shape.  One 16-column block (CBW = 1): 2 waves.  Head width 512:
// the two waves are one team that streams the same tiles; both compute the
// full scores (QK^T is a third of the matrix work) and each accumulates O^T
// for its half of D, so neither holds more than 128 accumulator/query
// registers.  Narrower heads: each wave is a team of its own and streams its
// own tiles.  CBW column blocks per workgroup (CBW > 1): one wave per block
// (a D-split pair at width 512), all in one team that streams every tile once
// for all the blocks, through a deeper ring.
template <int D, int CBW>
struct DecodeShape {
  static constexpr int kSplitD = D > 256 ? 2 : 1;          // waves per column block splitting D
  static constexpr int kWaves = CBW == 1 ? 2 : CBW * kSplitD;
  static constexpr int kTeam = CBW == 1 ? kSplitD : kWaves;  // waves streaming one tile sequence
  static constexpr int kTeams = kWaves / kTeam;
};

// f(integral_constant<int, I>) for I = 0, 1, ... in order; static_all stops
// at the first call that returns false.
template <class F, int... I>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <class F, int... I>
__device__ __forceinline__ bool static_all(F&& f, std::integer_sequence<int, I...>) {
  return (f(std::integral_constant<int, I>{}) && ...);
}

// s_waitcnt for tile copies: at most n tiles of K ops each still in flight
// (n runtime, 0 <= n <= N).
template <int N, int K>
__device__ __forceinline__ void wait_tiles(int32_t n) {
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vmcnt<N * K>();
      return;
    }
    wait_tiles<N - 1, K>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// Write the partial (m, l, o) of this workgroup's 16 columns.  One team: both
// waves hold the same (m, l) and disjoint slices of D.  Two teams (one wave
// each, over different keys): merged through LDS first; merge_buf is
// [16 columns][D] fp32 and reuses a slot (both waves are past their last
// tile when the first barrier returns).
// One workgroup per sequence (p.per_seq) at head width <= 256: that
// workgroup's (m, l, o) is the whole attention of its columns, so it writes
// the output o / l (bf16) and the lse itself and no combine kernel runs; a
// sequence with no keys gets zeros and -inf.  (Width 512 keeps the partial and
// the combine: the extra code spilled registers in its kernels.)  `row` is the
// output row (b*q_len + tok)*Hq + head, `lrow` the lse index
// (b*Hq + head)*q_len + tok.
template <int D>
constexpr bool kFinalInKernel = D <= 256;
template <int D>
__device__ __forceinline__ void store_final4(const DecodeParams& p, int64_t row, int32_t d, f32x4 v, float inv) {
  uint16_t* dst = p.out + row * D + d;
  const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(v[0] * inv)) | (static_cast<uint32_t>(f32_to_bf16(v[1] * inv)) << 16);
  const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(v[2] * inv)) | (static_cast<uint32_t>(f32_to_bf16(v[3] * inv)) << 16);
  *reinterpret_cast<u32x2*>(dst) = u32x2{w0, w1};
}
__device__ __forceinline__ void store_final_lse(const DecodeParams& p, int64_t lrow, float m, float l) {
  if (p.lse) p.lse[lrow] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

template <int D, int kTeams, int kDB>
__device__ __forceinline__ void write_partial(const DecodeParams& p, int64_t part, bool col_ok, const f32x4 (&o)[kDB],
                                              float m_run, float l_run, int32_t wave, int32_t member, int32_t dlo,
                                              int32_t grp, int32_t col, float* merge_buf, float (*m_w)[16],
                                              float (*l_w)[16], int64_t row, int64_t lrow) {
  if constexpr (kTeams == 1) {
    if (kFinalInKernel<D> && p.per_seq) {
      if (col_ok) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
        for (int db = 0; db < kDB; ++db) store_final4<D>(p, row, dlo + db * 16 + grp * 4, o[db], inv);
        if (member == 0 && grp == 0) store_final_lse(p, lrow, m_run, l_run);
      }
    } else if (col_ok) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        float* dst = p.ws_o + part * D + dlo + db * 16 + grp * 4;
        *reinterpret_cast<f32x4*>(dst) = o[db];
      }
      if (member == 0 && grp == 0) {
        p.ws_m[part] = m_run;
        p.ws_l[part] = l_run;
      }
    }
  } else {
    __syncthreads();
    if (grp == 0) {
      m_w[wave][col] = m_run;
      l_w[wave][col] = l_run;
    }
    __syncthreads();
    const float m_all = fmaxf(m_w[0][col], m_w[1][col]);
    const float m_ref = m_all == -INFINITY ? 0.f : m_all;
    const float f = __builtin_amdgcn_exp2f(m_run - m_ref);
    // Column col's 16-byte chunk q = db*4 + grp sits at chunk q ^ col of its
    // row, so the 16 columns of a lane group hit 16 different bank groups.
    if (wave == 0) {
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        *reinterpret_cast<f32x4*>(merge_buf + col * D + (((db * 4 + grp) ^ col) << 2)) = o[db] * f;
    }
    __syncthreads();
    if (wave == 1 && col_ok) {
      const float l_all =
          l_w[0][col] * __builtin_amdgcn_exp2f(m_w[0][col] - m_ref) + l_w[1][col] * __builtin_amdgcn_exp2f(m_w[1][col] - m_ref);
      const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const f32x4 prev = *reinterpret_cast<const f32x4*>(merge_buf + col * D + (((db * 4 + grp) ^ col) << 2));
        if (kFinalInKernel<D> && p.per_seq) {
          store_final4<D>(p, row, db * 16 + grp * 4, prev + o[db] * f, inv);
        } else {
          float* dst = p.ws_o + part * D + db * 16 + grp * 4;
          *reinterpret_cast<f32x4*>(dst) = prev + o[db] * f;
        }
      }
      if (grp == 0) {
        if (kFinalInKernel<D> && p.per_seq) {
          store_final_lse(p, lrow, m_all, l_all);
        } else {
          p.ws_m[part] = m_all;
          p.ws_l[part] = l_all;
        }
      }
    }
  }
}

template <int D, int G, bool KEQV, bool CAP, int CBW>
__global__ __launch_bounds__((DecodeShape<D, CBW>::kWaves * 64)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_kernel(DecodeParams p) {
  using Sh = DecodeShape<D, CBW>;
  constexpr int kTeam = Sh::kTeam;
  constexpr int kTeams = Sh::kTeams;
  constexpr int kDW = D / Sh::kSplitD;   // D slice of one wave's accumulators
  constexpr int kDS = D / 32;        // k-steps of QK^T (16x16x32)
  constexpr int kDB = kDW / 16;      // 16-row blocks of this wave's O^T
  constexpr int kRowChunks = D / 8;  // 16-byte chunks per cache row
  constexpr int kSlotElems = kTK * D;
  constexpr int kOps = kTK * kRowChunks / 64;   // 1 KB copy ops per tensor per tile
  constexpr int kWaveOps = kOps / kTeam;        // issued by each wave of a team
  constexpr int kOpsPerTile = kWaveOps * (KEQV ? 1 : 2);
  static_assert(G <= 16, "at most 16 query heads per KV head");
  static_assert(kTK * kRowChunks % (64 * kTeam) == 0, "tile must split into whole 1 KB ops");

  // Ring of slots per team, one LDS array per slot (so reads of one slot are
  // not ordered behind the copies landing in the others).  One column block:
  // two slots, one tile in flight while one is computed.  (At head width 512
  // with keys as values the launch reserves LDS for three workgroups per CU;
  // a three-slot ring that kept two tiles in flight per workgroup was 4%
  // slower on the Gemma-4 global layer, 408 against 392 us.)
  // Several column blocks: one or two workgroups fill a CU (two waves per
  // SIMD), so the ring deepens to keep as many tiles in flight per CU.
  constexpr int kSlotBytes = kSlotElems * 2 * (KEQV ? 1 : 2);
  constexpr int kWgPerCu = 8 / Sh::kWaves;
  constexpr int kSlotsFit = (160 * 1024) / (kWgPerCu * kTeams * kSlotBytes);
  constexpr int kSlots = CBW == 1 ? 2 : (kSlotsFit < 6 ? kSlotsFit : 6);
  static_assert(kSlots >= 2 && kSlots <= 6, "ring depth");
  constexpr int kKE = kTeams * kSlotElems;
  __shared__ __attribute__((aligned(16))) uint16_t ks0[kKE];
  __shared__ __attribute__((aligned(16))) uint16_t ks1[kKE];
  __shared__ __attribute__((aligned(16))) uint16_t ks2[kSlots > 2 ? kKE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t ks3[kSlots > 3 ? kKE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t ks4[kSlots > 4 ? kKE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t ks5[kSlots > 5 ? kKE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t vs0[KEQV ? 8 : kKE];
  __shared__ __attribute__((aligned(16))) uint16_t vs1[KEQV ? 8 : kKE];
  __shared__ __attribute__((aligned(16))) uint16_t vs2[(KEQV || kSlots < 3) ? 8 : kKE];
  __shared__ __attribute__((aligned(16))) uint16_t vs3[(KEQV || kSlots < 4) ? 8 : kKE];
  __shared__ __attribute__((aligned(16))) uint16_t vs4[(KEQV || kSlots < 5) ? 8 : kKE];
  __shared__ __attribute__((aligned(16))) uint16_t vs5[(KEQV || kSlots < 6) ? 8 : kKE];
  __shared__ float m_w[2][16];
  __shared__ float l_w[2][16];
  static_assert(kTeams == 1 || kSlotElems * kTeams * 2 >= 16 * D * 4, "merge buffer reuses slot 0");
  lds_poison(ks0, ks1, ks2, ks3, ks4, ks5, vs0, vs1, vs2, vs3, vs4, vs5, m_w, l_w);

  const DecodeBlock blk = decode_block(p);
  if (!blk.valid) return;                                        // padding block (uniform)
  const int32_t kvh = blk.kvh;
  const int32_t tid = threadIdx.x;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t team = wave / kTeam;
  const int32_t member = wave % kTeam;                           // copy share within the team
  const int32_t dmem = wave % Sh::kSplitD;                       // D slice within the column block
  const int32_t cb = blk.cb * CBW + (CBW == 1 ? 0 : wave / Sh::kSplitD);   // 16-column block
  const int32_t dlo = dmem * kDW;
  const int32_t lane = tid & 63;
  const int32_t col = lane & 15;     // column of the block: (token, head) = divmod(cb*16 + col, g)
  const int32_t grp = lane >> 4;     // 16-lane group
  const int32_t gcol = cb * 16 + col;
  const bool col_ok = gcol < G * p.q_len;
  const int32_t tok = col_ok ? gcol / G : 0;
  const int32_t head = kvh * G + (col_ok ? gcol % G : 0);


  // Each sequence segment of this workgroup's key range: [s_lo, s_hi) of
  // sequence b, whose context is ctx.
  for_each_segment(p, blk.w, [&](int32_t b, int32_t s_lo, int32_t s_hi, int32_t ctx) __attribute__((always_inline)) {
  const int32_t n_t = (s_hi - s_lo + kTK - 1) / kTK;
  // Keys this column may see: [key_lo, key_hi] (its own position and the window).
  const int32_t key_hi = col_ok ? ctx - p.q_len + tok : -1;
  const int32_t key_lo = p.window > 0 ? key_hi - p.window + 1 : 0;
  // Q^T operand: lane holds d = ds*32 + grp*8 + [0, 8) of its (token, head).
  bf16x8 qf[kDS];
  {
    const uint16_t* qrow = p.q + ((static_cast<int64_t>(b) * p.q_len + tok) * p.hq + head) * D + grp * 8;
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) {
      qf[ds] = col_ok ? *reinterpret_cast<const bf16x8*>(qrow + ds * 32) : bf16x8{};
    }
  }

  f32x4 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x4{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const uint32_t row_pitch = static_cast<uint32_t>(p.hkv) * D * 2;    // bytes between cache rows
  const char* kseq = reinterpret_cast<const char*>(p.kc) + (static_cast<int64_t>(b) * p.max_ctx * p.hkv + kvh) * D * 2;
  const char* vseq = KEQV ? kseq : reinterpret_cast<const char*>(p.vc) + (static_cast<int64_t>(b) * p.max_ctx * p.hkv + kvh) * D * 2;

  // Copy this wave's share of tile ti (keys s_lo + 16*ti ...) into a slot.
  // Rows past s_hi repeat row s_hi - 1, so no row outside the sequence's
  // range is read.  A tile that is not live (past the range) gets a zero-byte
  // resource: its copies read no memory and write zeros into the slot.
  auto copy_tile = [&](int32_t ti, uint16_t* kdst, uint16_t* vdst, bool live) __attribute__((always_inline)) {
    const int32_t k0 = live ? s_lo + ti * kTK : 0;
    const int32_t last = s_hi - 1 - k0;
    const uint32_t nbytes = live ? kTK * row_pitch : 0u;
    const __amdgpu_buffer_rsrc_t krs = raw_rsrc(kseq + static_cast<int64_t>(k0) * row_pitch, nbytes);
    const __amdgpu_buffer_rsrc_t vrs = raw_rsrc(vseq + static_cast<int64_t>(k0) * row_pitch, nbytes);
    const int32_t ln = lane_here();
#pragma unroll
    for (int i = 0; i < kWaveOps; ++i) {
      const int32_t op = member * kWaveOps + i;
      const int32_t pc = op * 64 + ln;
      const int32_t row = pc / kRowChunks;
      const int32_t lc = (pc % kRowChunks) ^ dswz<D>(row);
      const uint32_t off = static_cast<uint32_t>(min(row, last)) * row_pitch + static_cast<uint32_t>(lc) * 16u;
      copy_to_lds<16, kStreamAux>(krs, off, kdst + op * 512);
      if (!KEQV) copy_to_lds<16, kStreamAux>(vrs, off, vdst + op * 512);
    }
  };

  // One tile from slot (kb, vb).
  auto compute = [&](int32_t ti, const uint16_t* kb, const uint16_t* vb) __attribute__((always_inline)) {
    const int32_t k0 = s_lo + ti * kTK;
    // S^T[16 keys x 16 heads] = K . Q^T; lane: key row li16, d chunk ds*4 + lgrp.
    // The chunk's bits (ds, lgrp, swizzle) sit in byte-address bits 4-9, clear
    // of the row bits, and ds*4 + lgrp = (ds << 2) ^ lgrp, so step ds reads at
    // one XOR of the lane's base: kaddr ^ (ds << 6).
    f32x4 sacc = f32x4{};
    const int32_t ln = lane_here();
    const int32_t li16 = ln & 15;
    const int32_t lgrp = ln >> 4;
    const uint32_t kaddr = static_cast<uint32_t>(li16 * D * 2 + ((lgrp ^ dswz<D>(li16)) << 4));
    const char* kbc = reinterpret_cast<const char*>(kb);
    // kLA operand reads in flight ahead of the product that consumes them
    // (fenced, so the order holds): the LDS latency spans several products.
    constexpr int kLA = kDS < 4 ? kDS : 4;
    bf16x8 ka[kLA];
#pragma unroll
    for (int ds = 0; ds < kLA; ++ds) ka[ds] = *reinterpret_cast<const bf16x8*>(kbc + (kaddr ^ static_cast<uint32_t>(ds << 6)));
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) {
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ds % kLA], qf[ds], sacc, 0, 0, 0);
      if (ds + kLA < kDS)
        ka[ds % kLA] = *reinterpret_cast<const bf16x8*>(kbc + (kaddr ^ static_cast<uint32_t>((ds + kLA) << 6)));
      __builtin_amdgcn_sched_barrier(0);
    }
    // Lane holds keys k0 + grp*4 + r for head `col`.
    float x[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t;
      if (CAP) {
        const float e = __builtin_amdgcn_exp2f(sacc[r] * p.cap_in2);
        t = fmaf(-2.f * p.cap_log2, __builtin_amdgcn_rcpf(e + 1.f), p.cap_log2);
      } else {
        t = sacc[r] * p.scale_log2;
      }
      const int32_t key = k0 + grp * 4 + r;
      t = ((key < s_hi) & (key <= key_hi) & (key >= key_lo)) ? t : -INFINITY;
      x[r] = t;
      mx = fmaxf(mx, t);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool grow = mx > m_run + 8.f;          // lazily updated running max
    const float m_next = grow ? mx : m_run;
    const float m_use = m_next == -INFINITY ? 0.f : m_next;
    if (__builtin_amdgcn_ballot_w64(grow && m_run != -INFINITY) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
      for (int db = 0; db < kDB; ++db) o[db] *= alpha;
    }
    m_run = m_next;
    const uint32_t pk0 = pack_bf16x2(__builtin_amdgcn_exp2f(x[0] - m_use), __builtin_amdgcn_exp2f(x[1] - m_use));
    const uint32_t pk1 = pack_bf16x2(__builtin_amdgcn_exp2f(x[2] - m_use), __builtin_amdgcn_exp2f(x[3] - m_use));
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk0), ones, l_run, false);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk1), ones, l_run, false);
    // O^T += V^T . P^T with the 16-deep product (16 keys per tile).  P^T
    // operand: lane group grp holds keys grp*4 + [0,4).  V^T operand: the
    // transpose read of rows grp*4 + [0,4) at d = dlo + db*16 + li16.  The
    // chunk (dlo/8 + 2*db + (li16&3)/2) ^ swizzle again has its db bits clear
    // of the rest, so block db reads at vaddr ^ (db << 5).
    const i16x4 pb = __builtin_bit_cast(i16x4, u32x2{pk0, pk1});
    const int32_t r0 = lgrp * 4 + (li16 >> 2);
    const uint32_t vaddr = static_cast<uint32_t>(r0 * D * 2 + ((((dlo >> 3) + ((li16 & 3) >> 1)) ^ dswz<D>(r0)) << 4) +
                                                 (li16 & 1) * 8);
    const char* vbc = reinterpret_cast<const char*>(vb);
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const i16x4 a0 = lds_read_tr16(vbc + (vaddr ^ static_cast<uint32_t>(db << 5)));
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, pb, o[db], 0, 0, 0);
    }
  };

  // Slot I of this team (compile-time I, so each access names one LDS array).
  auto kslot = [&](auto I) -> uint16_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return ks0 + team * kSlotElems;
    else if constexpr (i == 1) return ks1 + team * kSlotElems;
    else if constexpr (i == 2) return ks2 + team * kSlotElems;
    else if constexpr (i == 3) return ks3 + team * kSlotElems;
    else if constexpr (i == 4) return ks4 + team * kSlotElems;
    else return ks5 + team * kSlotElems;
  };
  auto vslot = [&](auto I) -> uint16_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (KEQV) return kslot(I);
    else if constexpr (i == 0) return vs0 + team * kSlotElems;
    else if constexpr (i == 1) return vs1 + team * kSlotElems;
    else if constexpr (i == 2) return vs2 + team * kSlotElems;
    else if constexpr (i == 3) return vs3 + team * kSlotElems;
    else if constexpr (i == 4) return vs4 + team * kSlotElems;
    else return vs5 + team * kSlotElems;
  };
  // A team of several waves shares its slots: a barrier publishes every
  // wave's part of a tile and fences the slot being refilled (every wave
  // runs the same trips).
  auto team_sync = [&]() {
    if constexpr (kTeam > 1) lds_barrier();
  };
  // The team's tiles are ti = team, team + kTeams, ...; tile k of the team
  // sits in slot k % kSlots, and up to kSlots - 1 tiles are copied ahead.
  // Before computing a tile, its copies must have landed; the newer tiles'
  // copies (kOpsPerTile per wave each) may stay in flight.
  //
  // With two slots a copy is issued only for a live tile and each step waits
  // for all copies.  With three or more (several column blocks), every step
  // issues one tile's copies (dead tiles past the range copy nothing), so the
  // wait is one constant count, and no copy sits under a branch: behind such
  // a branch the compiler lost track of which slot the copy writes and made
  // the next read of that slot wait for every copy in flight.
  constexpr bool kAlwaysIssue = kSlots > 2;
  static_assert((kSlots - 2) * kOpsPerTile <= 63, "vmcnt range");
  int32_t ti = team;
  static_for([&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    const bool live = ti + i * kTeams < n_t;
    if (kAlwaysIssue || live) copy_tile(ti + i * kTeams, kslot(I), vslot(I), live);
  }, std::make_integer_sequence<int, kSlots - 1>{});
  // With tiles left in flight across steps, Q^T (loaded before these copies)
  // must be complete before the loop: a load still pending on its registers
  // at the loop head made the compiler wait for every copy in flight before
  // the first product of each pass over the ring.
  if constexpr (kAlwaysIssue) wait_vmcnt<0>();
  auto step = [&](auto I) __attribute__((always_inline)) -> bool {
    constexpr int kCur = decltype(I)::value;
    using Next = std::integral_constant<int, (kCur + kSlots - 1) % kSlots>;
    if constexpr (kAlwaysIssue) {
      wait_vmcnt<(kSlots - 2) * kOpsPerTile>();
    } else {
      const int32_t after = (n_t - 1 - ti) / kTeams;          // team tiles issued after this one, capped below
      wait_tiles<kSlots - 2, kOpsPerTile>(after < kSlots - 2 ? after : kSlots - 2);
    }
    team_sync();
    const int32_t ta = ti + (kSlots - 1) * kTeams;
    if (kAlwaysIssue || ta < n_t) copy_tile(ta, kslot(Next{}), vslot(Next{}), ta < n_t);
    compute(ti, kslot(I), vslot(I));
    ti += kTeams;
    return ti < n_t;
  };
  while (ti < n_t) {
    if (!static_all(step, std::make_integer_sequence<int, kSlots>{})) break;
  }
  // The dead tiles' copies write their slots: they land before the merge
  // buffer (slot 0) is written.
  if constexpr (kAlwaysIssue) wait_vmcnt<0>();

  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  // Partial of (sequence b, token tok, head) from workgroup w: slot w + b.
  const int64_t part = ((static_cast<int64_t>(blk.w) + b) * p.q_len + tok) * p.hq + head;
  write_partial<D, kTeams, kDB>(p, part, col_ok, o, m_run, l_run, wave, dmem, dlo, grp, col,
                                reinterpret_cast<float*>(ks0), m_w, l_w,
                                (static_cast<int64_t>(b) * p.q_len + tok) * p.hq + head,
                                (static_cast<int64_t>(b) * p.hq + head) * p.q_len + tok);
  __syncthreads();   // LDS slots (and the merge buffer) are reused by the next segment
  });
}

// ---------------------------------------------------------------------------
// int8 cache: codes [B, max_ctx, Hkv, D] int8 with one fp32 scale per (token,
// KV head), scales laid out [B, Hkv, max_ctx] so a tile's scales are one
// contiguous run.  Tiles hold 32 keys (the bytes of a 16-row bf16 tile).  The
// key scale multiplies the score and the value scale folds into the
// probability, so both products run on the matrix cores:
//   s_j = ks_j * (q . c_j),   o = sum_j (p_j * vs_j) c'_j,   l = sum_j p_j.
// The products are fp16: a code c enters as the exact fp16 value 1152 + c
// (one XOR and one byte permute per two codes; bf16 needs a normalising
// conversion per code), so each product carries 1152 times the sum of its
// other operand, which is subtracted per column -- 1152 * sum(q') from the
// scores (q' = q * 2^-e, scaled so every bf16 q converts to fp16 exactly) and
// 1152 * sum(p * vs) from the outputs, summed over the same fp16-rounded
// weights the product used.  Value columns reach the PV operand with
// ds_read_b64_tr_b8.
constexpr int kTK8 = 32;    // keys per int8 tile

// XOR pattern of the 16-byte chunks of int8 LDS row r in [0, 32).  A 16-lane
// b128 phase of the score product reads the 16 rows of one half at one chunk;
// a transposed value read covers rows {0-7, 16-23} (lanes 0-31) or
// {8-15, 24-31} (lanes 32-63) at one chunk.  Both sets land on 16 distinct
// 16-byte bank groups (D = 64: four rows share one 256-byte bank cycle).
template <int D>
__device__ __forceinline__ int32_t qswz(int32_t r) {
  if constexpr (D >= 256) return (r & 15) ^ (((r >> 4) & 1) << 3);
  else return ((r >> 2) & 3) ^ (((r >> 4) & 1) << 1);
}

template <int D, int G, bool KEQV, bool CAP>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_split_i8_kernel(DecodeParams p) {
  using Sh = DecodeShape<D, 1>;
  constexpr int kTeam = Sh::kTeam;
  constexpr int kTeams = Sh::kTeams;
  constexpr int kDW = D / kTeam;     // D slice of one wave's accumulators
  constexpr int kDS = D / 64;        // 16-byte key chunks per lane per half (two MFMAs each)
  constexpr int kDSW = kDS / kTeam;  // of them, this wave's share (a team splits the score product by D)
  constexpr int kDB = kDW / 16;      // 16-row blocks of this wave's O^T
  constexpr int kRowChunks = D / 16; // 16-byte chunks per cache row
  constexpr int kSlotBytes = kTK8 * D;
  constexpr int kOps = kTK8 * kRowChunks / 64;  // 1 KB copy ops per tensor per tile
  constexpr int kWaveOps = kOps / kTeam;
  static_assert(G <= 16, "at most 16 query heads per KV head");
  static_assert(kOps % kTeam == 0, "tile must split into whole 1 KB ops");
  static_assert(kTeams == 1 || kSlotBytes * kTeams >= 16 * D * 4, "merge buffer reuses slot 0");
  // Ring depth.  Two slots (one tile in flight while one is computed), four
  // workgroups per CU at head width 512 with keys as values.  Fewer
  // workgroups per CU were slower on the Gemma-4 global layer, with the same
  // ring and LDS reserved at launch (three per CU 284-296 us, two 602 us,
  // against 245-272 us), and so was a three-slot ring (two tiles in flight,
  // three per CU: 468 us): the code conversion makes each tile's work long,
  // and the other workgroups' waves are what hide it.
  constexpr int kSlots = 2;
  // Copy ops each wave issues per tile (codes, then scales): the wait for the
  // oldest tile leaves the newer tile's ops outstanding.
  constexpr int kCodeOps = kWaveOps * (KEQV ? 1 : 2);
  constexpr int kOpsPerTile = kCodeOps + (KEQV ? 1 : 2);

  __shared__ __attribute__((aligned(16))) uint8_t ks0[kTeams * kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ks1[kTeams * kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ks2[kSlots > 2 ? kTeams * kSlotBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ks3[kSlots > 3 ? kTeams * kSlotBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t vs0[KEQV ? 16 : kTeams * kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vs1[KEQV ? 16 : kTeams * kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vs2[(KEQV || kSlots < 3) ? 16 : kTeams * kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vs3[(KEQV || kSlots < 4) ? 16 : kTeams * kSlotBytes];
  __shared__ __attribute__((aligned(16))) float ksc0[kTeams * 64];
  __shared__ __attribute__((aligned(16))) float ksc1[kTeams * 64];
  __shared__ __attribute__((aligned(16))) float ksc2[kSlots > 2 ? kTeams * 64 : 4];
  __shared__ __attribute__((aligned(16))) float ksc3[kSlots > 3 ? kTeams * 64 : 4];
  __shared__ __attribute__((aligned(16))) float vsc0[KEQV ? 4 : kTeams * 64];
  __shared__ __attribute__((aligned(16))) float vsc1[KEQV ? 4 : kTeams * 64];
  __shared__ __attribute__((aligned(16))) float vsc2[(KEQV || kSlots < 3) ? 4 : kTeams * 64];
  __shared__ __attribute__((aligned(16))) float vsc3[(KEQV || kSlots < 4) ? 4 : kTeams * 64];
  __shared__ float m_w[2][16];
  __shared__ float l_w[2][16];
  // Partial scores of a two-wave team: [member][half][lane].
  __shared__ f32x4 sx[kTeam > 1 ? 2 * 2 * 64 : 1];
  lds_poison(ks0, ks1, ks2, ks3, vs0, vs1, vs2, vs3, ksc0, ksc1, ksc2, ksc3, vsc0, vsc1, vsc2, vsc3, m_w, l_w, sx);

  const DecodeBlock blk = decode_block(p);
  if (!blk.valid) return;                                        // padding block (uniform)
  const int32_t kvh = blk.kvh;
  const int32_t cb = blk.cb;                                     // 16-column block
  const int32_t tid = threadIdx.x;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t team = wave / kTeam;
  const int32_t member = wave % kTeam;
  const int32_t dlo = member * kDW;
  const int32_t lane = tid & 63;
  const int32_t col = lane & 15;
  const int32_t grp = lane >> 4;
  const int32_t gcol = cb * 16 + col;
  const bool col_ok = gcol < G * p.q_len;
  const int32_t tok = col_ok ? gcol / G : 0;
  const int32_t head = kvh * G + (col_ok ? gcol % G : 0);


  // Each sequence segment of this workgroup's key range: [s_lo, s_hi) of
  // sequence b, whose context is ctx.
  for_each_segment(p, blk.w, [&](int32_t b, int32_t s_lo, int32_t s_hi, int32_t ctx) __attribute__((always_inline)) {
  const int32_t n_t = (s_hi - s_lo + kTK8 - 1) / kTK8;
  // Keys this column may see: [key_lo, key_hi] (its own position and the window).
  const int32_t key_hi = col_ok ? ctx - p.q_len + tok : -1;
  const int32_t key_lo = p.window > 0 ? key_hi - p.window + 1 : 0;
  // Q^T operand: step ds, MFMA m: lane holds d = (ds*4 + grp)*16 + m*8 + [0, 8),
  // the d range of the key chunk (ds*4 + grp) that the K operand lane reads;
  // this wave's steps are ds = member*kDSW + [0, kDSW).  The products run in
  // fp16 against offset-fp16 codes: q is scaled by 2^-e (e from the largest
  // |q| of this wave's share of the column, so the scaled values stay below 2
  // and every bf16 value converts exactly), and the offset term 1152 * sum(q')
  // comes off each score before it is scaled back by 2^e.
  f16x8 qh[kDSW][2];
  float q_unscale, q_off;
  {
    const uint16_t* qrow = p.q + ((static_cast<int64_t>(b) * p.q_len + tok) * p.hq + head) * D + grp * 16;
    u32x4 qr[kDSW][2];
    float qmax = 0.f;
#pragma unroll
    for (int i = 0; i < kDSW; ++i) {
      const int ds = member * kDSW + i;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        qr[i][m] = col_ok ? *reinterpret_cast<const u32x4*>(qrow + ds * 64 + m * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) qmax = fmaxf(qmax, fmaxf(fabsf(lo_bf16(qr[i][m][e])), fabsf(hi_bf16(qr[i][m][e]))));
      }
    }
    qmax = fmaxf(qmax, __shfl_xor(qmax, 16, 64));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
    const int32_t qe = qmax > 0.f ? __builtin_amdgcn_frexp_expf(qmax) : 0;
    const float qin = __builtin_ldexpf(1.f, -qe);
    q_unscale = __builtin_ldexpf(1.f, qe);
    float qsum = 0.f;
    const f16x2 ones_h = f16x2{static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
#pragma unroll
    for (int i = 0; i < kDSW; ++i) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        u32x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // (pack into a scalar first: the dot of a just-inserted vector
          // element, bit-cast, was compiled as the dot of element 0)
          const uint32_t w = pack_f16x2(lo_bf16(qr[i][m][e]) * qin, hi_bf16(qr[i][m][e]) * qin);
          qsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), ones_h, qsum, false);
          h[e] = w;
        }
        qh[i][m] = __builtin_bit_cast(f16x8, h);
      }
    }
    qsum += __shfl_xor(qsum, 16, 64);
    qsum += __shfl_xor(qsum, 32, 64);
    q_off = kI8Offset * qsum;
  }

  f32x4 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x4{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  float lp_run = 0.f;   // sum of the fp16 value-product weights p * vs (offset term of O)

  const uint32_t row_pitch = static_cast<uint32_t>(p.hkv) * D;     // bytes between cache rows
  const int64_t seq_off = (static_cast<int64_t>(b) * p.max_ctx * p.hkv + kvh) * D;
  const char* kseq = reinterpret_cast<const char*>(p.kc) + seq_off;
  const char* vseq = KEQV ? kseq : reinterpret_cast<const char*>(p.vc) + seq_off;
  const int64_t sc_off = (static_cast<int64_t>(b) * p.hkv + kvh) * p.max_ctx;
  const float* kscale = p.ks + sc_off;
  const float* vscale = KEQV ? kscale : p.vs + sc_off;

  // Copy this wave's share of tile ti into a slot, and the tile's key (and
  // value) scales (64 lanes, key lane & 31, so the upper half repeats the
  // lower).  Every member of a team copies the scales, the same bytes to the
  // same place: with the copy under a branch on the member, the compiler lost
  // track of which LDS array it writes and waited for every copy in flight
  // before the next LDS read.  Rows past s_hi repeat row s_hi - 1.
  auto copy_tile = [&](int32_t ti, uint8_t* kdst, uint8_t* vdst, float* kscd, float* vscd) __attribute__((always_inline)) {
    const int32_t k0 = s_lo + ti * kTK8;
    const int32_t last = s_hi - 1 - k0;
    const __amdgpu_buffer_rsrc_t krs = raw_rsrc(kseq + static_cast<int64_t>(k0) * row_pitch, kTK8 * row_pitch);
    const __amdgpu_buffer_rsrc_t vrs = raw_rsrc(vseq + static_cast<int64_t>(k0) * row_pitch, kTK8 * row_pitch);
    // The lane index is visible to loop-invariant code motion here (not
    // lane_here()): the lane-derived copy offsets and LDS addresses are held
    // across the tile loop, which fits the int8 kernel's registers (keys as
    // values: 216 VGPRs) and saves their per-tile arithmetic.
    const int32_t ln = static_cast<int32_t>(threadIdx.x) & 63;
#pragma unroll
    for (int i = 0; i < kWaveOps; ++i) {
      const int32_t op = member * kWaveOps + i;
      const int32_t pc = op * 64 + ln;
      const int32_t row = pc / kRowChunks;
      const int32_t lc = (pc % kRowChunks) ^ qswz<D>(row);
      const uint32_t off = static_cast<uint32_t>(min(row, last)) * row_pitch + static_cast<uint32_t>(lc) * 16u;
      copy_to_lds<16, kStreamAux>(krs, off, kdst + op * 1024);
      if (!KEQV) copy_to_lds<16, kStreamAux>(vrs, off, vdst + op * 1024);
    }
    const uint32_t koff = static_cast<uint32_t>(min(ln & 31, last)) * 4u;
    copy_to_lds<4, kStreamAux>(raw_rsrc(kscale + k0, kTK8 * 4), koff, kscd);
    if (!KEQV) copy_to_lds<4, kStreamAux>(raw_rsrc(vscale + k0, kTK8 * 4), koff, vscd);
  };

  auto compute = [&](int32_t ti, const uint8_t* kb, const uint8_t* vb, const float* kscs, const float* vscs) __attribute__((always_inline)) {
    const int32_t k0 = s_lo + ti * kTK8;
    const int32_t ln = static_cast<int32_t>(threadIdx.x) & 63;   // hoistable, as in copy_tile
    const int32_t li16 = ln & 15;
    const int32_t lgrp = ln >> 4;
    // S^T[32 keys x 16 columns] in two 16-key halves (this wave's share of D).
    f32x4 sacc[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      sacc[h2] = f32x4{};
      const int32_t row = h2 * 16 + li16;
      const int32_t sw = qswz<D>(row);
#pragma unroll
      for (int i = 0; i < kDSW; ++i) {
        const int32_t c = (member * kDSW + i) * 4 + lgrp;
        const u32x4 raw = *reinterpret_cast<const u32x4*>(kb + row * D + ((c ^ sw) << 4));
        sacc[h2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(i8x8_to_f16x8_off(raw[0], raw[1]), qh[i][0], sacc[h2], 0, 0, 0);
        sacc[h2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(i8x8_to_f16x8_off(raw[2], raw[3]), qh[i][1], sacc[h2], 0, 0, 0);
      }
      sacc[h2] = (sacc[h2] - q_off) * q_unscale;   // this wave's share of q . c
    }
    if constexpr (kTeam > 1) {
      // Add the partner's half of D.  Both members form p0 + p1 (fp32 addition
      // commutes), so they hold bit-identical scores.  The buffer is rewritten
      // only after the next tile's team barrier, which follows this read.
      sx[(member * 2 + 0) * 64 + ln] = sacc[0];
      sx[(member * 2 + 1) * 64 + ln] = sacc[1];
      lds_barrier();   // the next tile's copies stay in flight
      sacc[0] += sx[((1 - member) * 2 + 0) * 64 + ln];
      sacc[1] += sx[((1 - member) * 2 + 1) * 64 + ln];
    }
    // Lane holds keys k0 + h2*16 + grp*4 + r as x[h2*4 + r].
    const f32x4 ksa = *reinterpret_cast<const f32x4*>(kscs + grp * 4);
    const f32x4 ksb = *reinterpret_cast<const f32x4*>(kscs + 16 + grp * 4);
    const f32x4 vsa = *reinterpret_cast<const f32x4*>(vscs + grp * 4);
    const f32x4 vsb = *reinterpret_cast<const f32x4*>(vscs + 16 + grp * 4);
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = sacc[e >> 2][e & 3] * (e < 4 ? ksa[e & 3] : ksb[e & 3]);
      float t;
      if (CAP) {
        const float ex = __builtin_amdgcn_exp2f(sv * p.cap_in2);
        t = fmaf(-2.f * p.cap_log2, __builtin_amdgcn_rcpf(ex + 1.f), p.cap_log2);
      } else {
        t = sv * p.scale_log2;
      }
      const int32_t key = k0 + (e >> 2) * 16 + grp * 4 + (e & 3);
      t = ((key < s_hi) & (key <= key_hi) & (key >= key_lo)) ? t : -INFINITY;
      x[e] = t;
      mx = fmaxf(mx, t);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool grow = mx > m_run + 8.f;
    const float m_next = grow ? mx : m_run;
    const float m_use = m_next == -INFINITY ? 0.f : m_next;
    if (__builtin_amdgcn_ballot_w64(grow && m_run != -INFINITY) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
      lp_run *= alpha;
      for (int db = 0; db < kDB; ++db) o[db] *= alpha;
    }
    m_run = m_next;
    float pe[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
      l_run += pe[e];
    }
    // P^T operand (fp16): slot e = key (e/4)*16 + grp*4 + e%4, scaled by its
    // value scale; lp_run sums the same rounded weights for the offset term.
    const uint32_t pw0 = pack_f16x2(pe[0] * vsa[0], pe[1] * vsa[1]);
    const uint32_t pw1 = pack_f16x2(pe[2] * vsa[2], pe[3] * vsa[3]);
    const uint32_t pw2 = pack_f16x2(pe[4] * vsb[0], pe[5] * vsb[1]);
    const uint32_t pw3 = pack_f16x2(pe[6] * vsb[2], pe[7] * vsb[3]);
    const f16x2 ones_h = f16x2{static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
    lp_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pw0), ones_h, lp_run, false);
    lp_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pw1), ones_h, lp_run, false);
    lp_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pw2), ones_h, lp_run, false);
    lp_run = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pw3), ones_h, lp_run, false);
    const f16x8 pb = __builtin_bit_cast(f16x8, u32x4{pw0, pw1, pw2, pw3});
    // V^T operand: lane j of group lgrp addresses key row of slot j/2 at
    // columns d0 + 8*(j%2); the transpose read hands lane i the 8 keys at d0 + i.
    const int32_t e2 = li16 >> 1;
    const int32_t vrow = (e2 >> 2) * 16 + lgrp * 4 + (e2 & 3);
    const int32_t vsw = qswz<D>(vrow);
    const uint8_t* vbase = vb + vrow * D + (li16 & 1) * 8;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const int32_t c = (dlo >> 4) + db;
      const v2i32 raw = lds_read_tr8(vbase + ((c ^ vsw) << 4));
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          i8x8_to_f16x8_off(static_cast<uint32_t>(raw[0]), static_cast<uint32_t>(raw[1])), pb, o[db], 0, 0, 0);
    }
  };

  // Slot I of this team (compile-time I, so each access names one LDS array).
  auto kslot = [&](auto I) -> uint8_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return ks0 + team * kSlotBytes;
    else if constexpr (i == 1) return ks1 + team * kSlotBytes;
    else if constexpr (i == 2) return ks2 + team * kSlotBytes;
    else return ks3 + team * kSlotBytes;
  };
  auto vslot = [&](auto I) -> uint8_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (KEQV) return kslot(I);
    else if constexpr (i == 0) return vs0 + team * kSlotBytes;
    else if constexpr (i == 1) return vs1 + team * kSlotBytes;
    else if constexpr (i == 2) return vs2 + team * kSlotBytes;
    else return vs3 + team * kSlotBytes;
  };
  auto kscl = [&](auto I) -> float* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return ksc0 + team * 64;
    else if constexpr (i == 1) return ksc1 + team * 64;
    else if constexpr (i == 2) return ksc2 + team * 64;
    else return ksc3 + team * 64;
  };
  auto vscl = [&](auto I) -> float* {
    constexpr int i = decltype(I)::value;
    if constexpr (KEQV) return kscl(I);
    else if constexpr (i == 0) return vsc0 + team * 64;
    else if constexpr (i == 1) return vsc1 + team * 64;
    else if constexpr (i == 2) return vsc2 + team * 64;
    else return vsc3 + team * 64;
  };
  auto team_sync = [&]() {
    if constexpr (kTeam > 1) lds_barrier();
  };
  // The team's tiles are ti = team, team + kTeams, ...; tile k of the team
  // sits in slot k % kSlots, and up to kSlots - 1 tiles are copied ahead.
  // Before computing a tile its copies must have landed; the newer tiles'
  // copies (kOpsPerTile per wave each) may stay in flight.
  int32_t ti = team;
  static_for([&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    if (ti + i * kTeams < n_t) copy_tile(ti + i * kTeams, kslot(I), vslot(I), kscl(I), vscl(I));
  }, std::make_integer_sequence<int, kSlots - 1>{});
  auto step = [&](auto I) __attribute__((always_inline)) -> bool {
    constexpr int kCur = decltype(I)::value;
    using Next = std::integral_constant<int, (kCur + kSlots - 1) % kSlots>;
    const int32_t after = (n_t - 1 - ti) / kTeams;          // team tiles issued after this one, capped below
    const int32_t newer = after < kSlots - 2 ? after : kSlots - 2;
    wait_tiles<kSlots - 2, kOpsPerTile>(newer);
    team_sync();
    const int32_t ta = ti + (kSlots - 1) * kTeams;
    if (ta < n_t) copy_tile(ta, kslot(Next{}), vslot(Next{}), kscl(Next{}), vscl(Next{}));
    compute(ti, kslot(I), vslot(I), kscl(I), vscl(I));
    ti += kTeams;
    return ti < n_t;
  };
  while (ti < n_t) {
    if (!static_all(step, std::make_integer_sequence<int, kSlots>{})) break;
  }

  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  // The value codes entered the products as 1152 + c: remove 1152 * sum(p * vs).
  lp_run += __shfl_xor(lp_run, 16, 64);
  lp_run += __shfl_xor(lp_run, 32, 64);
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] -= kI8Offset * lp_run;
  // Partial of (sequence b, token tok, head) from workgroup w: slot w + b.
  const int64_t part = ((static_cast<int64_t>(blk.w) + b) * p.q_len + tok) * p.hq + head;
  write_partial<D, kTeams, kDB>(p, part, col_ok, o, m_run, l_run, wave, member, dlo, grp, col,
                                reinterpret_cast<float*>(ks0), m_w, l_w,
                                (static_cast<int64_t>(b) * p.q_len + tok) * p.hq + head,
                                (static_cast<int64_t>(b) * p.hq + head) * p.q_len + tok);
  __syncthreads();   // LDS slots (and the merge buffer) are reused by the next segment
  });
}

// Merge the partials of one (sequence, token, query head), in workgroup order.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeParams p) {
  constexpr int kPer = D / 64 > 0 ? D / 64 : 1;   // elements per lane
  const int32_t tok = static_cast<int32_t>(blockIdx.x) / p.hq;
  const int32_t head = static_cast<int32_t>(blockIdx.x) % p.hq;
  const int32_t b = blockIdx.y;
  const int32_t lane = threadIdx.x;
  // workgroups whose ranges hold this sequence's keys (none when it has none)
  int64_t total = 0, wa = 1, wb = 0;
  if (p.per_seq) {
    int32_t lo, ctx;
    seq_range(p, b, lo, ctx);
    if (ctx > lo) wa = wb = b;
  } else {
    total = p.prefix[p.batch];
    const int64_t pb = p.prefix[b], pe = p.prefix[b + 1];
    if (pe > pb) {
      wa = wg_of(pb, total, p.n_wg);
      wb = wg_of(pe - 1, total, p.n_wg);
    }
  }
  const int64_t row = (static_cast<int64_t>(b) * p.q_len + tok) * p.hq + head;
  auto part_of = [&](int64_t w) { return ((w + b) * p.q_len + tok) * p.hq + head; };
  // a workgroup with an empty range (fewer keys than workgroups) wrote nothing
  auto empty = [&](int64_t w) {
    return !p.per_seq && wg_start(w, total, p.n_wg) == wg_start(w + 1, total, p.n_wg);
  };
  // The largest partial max: the lanes take the partials in turn (their
  // loads independent), then a reduction across the wave.
  float m_all = -INFINITY;
  for (int64_t w = wa + lane; w <= wb; w += 64) {
    if (!empty(w)) m_all = fmaxf(m_all, p.ws_m[part_of(w)]);
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) m_all = fmaxf(m_all, __shfl_xor(m_all, sh, 64));
  // The weighted sum, in partial order; kAhead partials are loaded before
  // the first of them is used, so their loads are in flight together.
  constexpr int kAhead = 4;
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float l_all = 0.f;
  const int32_t d0 = lane * kPer;
  for (int64_t w0 = wa; w0 <= wb; w0 += kAhead) {
    bool use[kAhead];
    float ms[kAhead], ls[kAhead], os[kAhead][kPer];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int64_t w = w0 + i;
      use[i] = w <= wb && !empty(w);
      ms[i] = -INFINITY;
      ls[i] = 0.f;
#pragma unroll
      for (int e = 0; e < kPer; ++e) os[i][e] = 0.f;
      if (use[i]) {
        const int64_t part = part_of(w);
        ms[i] = p.ws_m[part];
        ls[i] = p.ws_l[part];
        if (d0 < D) {
          const float* src = p.ws_o + part * D + d0;
#pragma unroll
          for (int e = 0; e < kPer; ++e) os[i][e] = src[e];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      if (!use[i]) continue;
      const float f = ms[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[i] - m_all);
      l_all = fmaf(ls[i], f, l_all);
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] = fmaf(os[i][e], f, acc[e]);
    }
  }
  const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
  if (d0 < D) {
    uint16_t* dst = p.out + row * D + d0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) dst[e] = f32_to_bf16(acc[e] * inv);
  }
  if (p.lse && lane == 0) {
    p.lse[(static_cast<int64_t>(b) * p.hq + head) * p.q_len + tok] =
        l_all > 0.f ? (m_all + __log2f(l_all)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Many query columns per KV head at head width 512 with keys as values (the
// query heads of an MQA global layer times several new tokens): dense enough
// for the prefill's tile structure.  A workgroup is four waves, two D-split
// pairs of 32 columns, so 64 columns, (token, head) = divmod(cg*64 + c, g).
// Each wave holds half of Q^T and O^T.  Per 32-key tile of the cache:
//   * S^T over the wave's half of D (v_mfma_f32_32x32x16_bf16, K operands
//     read four products ahead);
//   * the partial scores exchanged through LDS, so both waves of a pair hold
//     the same fp32 sums (a + b == b + a);
//   * the softmax (masked on boundary tiles only, lazily updated running max);
//   * O^T += V^T . P^T over the wave's half (V operands read two ahead;
//     with keys as values the same LDS tile is both).
// Work items, key ranges, the partial layout and the combine are those of
// the split kernel above.
namespace tile {
constexpr int kD = 512;
constexpr int kKeys = 32;
constexpr int kDW = kD / 2;                     // D half per wave
constexpr int kDS = kDW / 16;                   // k-steps of S^T
constexpr int kDB = kDW / 32;                   // 32-row blocks of O^T
constexpr int kRowChunks = kD / 8;              // 16-byte chunks per cache row
constexpr int kTileElems = kKeys * kD;
constexpr int kOps = kKeys * kRowChunks / 64;   // 1 KB copy ops per tile
constexpr int kWaveOps = kOps / 4;
constexpr float kTau = 8.f;                     // lazy-rescale threshold (log2 units)

// XOR pattern of LDS row r's 16-byte chunks (a 4-bit rotate of r): the S^T
// reads (16 rows at one chunk per ds_read_b128 phase) and the V^T transpose
// reads (4 rows x 4 chunks per half-wave) are free of bank conflicts.
__device__ __forceinline__ int32_t swz(int32_t r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_min(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
}  // namespace tile

template <int G, bool CAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_tile_kernel(DecodeParams p) {
  using namespace tile;
  __shared__ __attribute__((aligned(16))) uint16_t ts0[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t ts1[kTileElems];
  __shared__ __attribute__((aligned(16))) f32x4 sx[4 * 4 * 64];   // [wave][r/4][lane] partial scores
  lds_poison(ts0, ts1, sx);

  const DecodeBlock blk = decode_block(p);
  if (!blk.valid) return;                                        // padding block (uniform)
  const int32_t kvh = blk.kvh;
  const int32_t tid = threadIdx.x;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t lane = tid & 63;
  const int32_t j = lane & 31;       // column within the pair
  const int32_t h = lane >> 5;       // half of the wave
  const int32_t dlo = (wave & 1) * kDW;
  const int32_t ncols = G * p.q_len;
  const int32_t g0 = blk.cb * 64 + (wave >> 1) * 32;                // the pair's first column
  const int32_t gcol = g0 + j;
  const bool col_ok = gcol < ncols;
  const int32_t tok = col_ok ? gcol / G : 0;
  const int32_t head = kvh * G + (col_ok ? gcol % G : 0);
  // First and last token among the pair's columns (for the unmasked-tile test).
  const int32_t tok_first = g0 / G;
  const int32_t tok_last = (min(g0 + 31, ncols - 1)) / G;
  const uint32_t row_pitch = static_cast<uint32_t>(p.hkv) * kD * 2;

  for_each_segment(p, blk.w, [&](int32_t b, int32_t s_lo, int32_t s_hi, int32_t ctx) __attribute__((always_inline)) {
  const int32_t n_t = (s_hi - s_lo + kKeys - 1) / kKeys;
  // Keys this column may see: [key_lo, key_hi] (its own position and the window).
  const int32_t key_hi = col_ok ? ctx - p.q_len + tok : -1;
  const int32_t key_lo = p.window > 0 ? key_hi - p.window + 1 : 0;
  const int32_t first_hi = ctx - p.q_len + tok_first;
  const int32_t last_lo = ctx - p.q_len + tok_last - p.window + 1;
  const char* kseq = reinterpret_cast<const char*>(p.kc) + (static_cast<int64_t>(b) * p.max_ctx * p.hkv + kvh) * kD * 2;

  // Copy tile ti (keys s_lo + 32*ti ...) into dst.  Rows past s_hi repeat
  // row s_hi - 1 (masked), so no row outside the sequence's range is read.
  auto issue = [&](int32_t ti, uint16_t* dst) __attribute__((always_inline)) {
    const int32_t k0 = s_lo + ti * kKeys;
    const int32_t last = s_hi - 1 - k0;
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(kseq + static_cast<int64_t>(k0) * row_pitch, kKeys * row_pitch);
    const int32_t ln = lane_here();
#pragma unroll
    for (int i = 0; i < kWaveOps; ++i) {
      // op i of this wave covers one row: 64 lanes x 16 bytes = 1 KB
      const int32_t first = (wave * kWaveOps + i) * 64;
      const int32_t row = first / kRowChunks;
      const int32_t lc = ln ^ swz(row);
      const uint32_t off = static_cast<uint32_t>(min(row, last)) * row_pitch + static_cast<uint32_t>(lc) * 16u;
      copy_to_lds<16, kStreamAux>(rs, off, dst + first * 8);
    }
  };

  // Q^T operand: lane holds d = dlo + ds*16 + h*8 + [0, 8) of its column.
  bf16x8 qf[kDS];
  {
    const uint16_t* qrow = p.q + ((static_cast<int64_t>(b) * p.q_len + tok) * p.hq + head) * kD + dlo + h * 8;
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) qf[ds] = col_ok ? *reinterpret_cast<const bf16x8*>(qrow + ds * 16) : bf16x8{};
  }
  f32x16 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  if (n_t > 0) issue(0, ts0);
  wait_vmcnt<0>();   // Q^T and the first tile
  __syncthreads();

  // Tile ti from slot cur, while tile ti + 1 is copied into nxt.
  auto step = [&](int32_t ti, const uint16_t* cur, uint16_t* nxt) __attribute__((always_inline)) {
    if (ti + 1 < n_t) issue(ti + 1, nxt);
    const int32_t kt = s_lo + ti * kKeys;
    const int32_t ln = lane_here();
    // S^T over this wave's half of D.  Lane (jj, hh) reads chunk
    // dlo/8 + 2*ds + hh of key row jj; step ds is one XOR of the base.
    f32x16 sacc = f32x16{};
    {
      const int32_t jj = ln & 31;
      const int32_t hh = ln >> 5;
      const uint32_t kaddr = static_cast<uint32_t>(jj * kD * 2 + dlo * 2 + ((hh ^ swz(jj)) << 4));
      const char* kbc = reinterpret_cast<const char*>(cur);
      constexpr int kLA = 4;
      // Address bit 8 of kaddr is clear, so the step's top bit is an addition,
      // which folds into the instruction's offset.
      auto kread = [&](int ds) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(kbc + (kaddr ^ static_cast<uint32_t>((ds & 7) * 32)) + (ds >> 3) * 256);
      };
      bf16x8 a[kLA];
#pragma unroll
      for (int ds = 0; ds < kLA; ++ds) a[ds] = kread(ds);
#pragma unroll
      for (int ds = 0; ds < kDS; ++ds) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ds % kLA], qf[ds], sacc, 0, 0, 0);
        if (ds + kLA < kDS) a[ds % kLA] = kread(ds + kLA);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // The pair's two halves of D: consecutive lanes, consecutive 16 bytes.
    {
      f32x4* mine = sx + wave * 256 + ln;
      const f32x4* other = sx + (wave ^ 1) * 256 + ln;
#pragma unroll
      for (int r = 0; r < 16; r += 4) mine[(r / 4) * 64] = f32x4{sacc[r], sacc[r + 1], sacc[r + 2], sacc[r + 3]};
      lds_barrier();   // the next tile's copies stay in flight
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const f32x4 t4 = other[(r / 4) * 64];
        sacc[r] += t4[0];
        sacc[r + 1] += t4[1];
        sacc[r + 2] += t4[2];
        sacc[r + 3] += t4[3];
      }
    }
    // Lane holds keys kt + (r/4)*8 + h*4 + r%4 of its column.  With a cap,
    // x = 1/(exp(2*s*scale/cap) + 1) and the capped logit is cap*(1 - 2x)
    // (log2 units): the row max comes from the smallest x, a masked key gets
    // +inf.  Without a cap x = s and a masked key gets -inf.
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (CAP) x[r] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(sacc[r] * p.cap_in2) + 1.f);
      else x[r] = sacc[r];
    }
    const bool full = kt + kKeys - 1 < s_hi && kt + kKeys - 1 <= first_hi && (p.window <= 0 || kt >= last_lo);
    if (__builtin_expect(!full, 0)) {
      const int32_t kb0 = kt + h * 4;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t key = kb0 + (r >> 2) * 8 + (r & 3);
        const bool ok = (key < s_hi) & (key <= key_hi) & (key >= key_lo);
        x[r] = ok ? x[r] : (CAP ? INFINITY : -INFINITY);
      }
    }
    float mx;
    if (CAP) {
      float mr = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mr = fminf(mr, x[r]);
      mr = xhalf_min(mr);
      mx = fmaf(-2.f * p.cap_log2, mr, p.cap_log2);
    } else {
      mx = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
      mx = xhalf_max(mx) * p.scale_log2;
    }
    const bool grow = mx > m_run + kTau;
    const float m_next = grow ? mx : m_run;
    const float m_use = m_next == -INFINITY ? 0.f : m_next;
    if (__builtin_amdgcn_ballot_w64(grow && m_run != -INFINITY) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db) o[db] *= alpha;
    }
    m_run = m_next;

    // Probabilities rounded to bf16; the row sum adds the same rounded values.
    uint32_t pk[8];
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    const float cap_m = p.cap_log2 - m_use;
    const float neg2cap = -2.f * p.cap_log2;
    auto prob_pair = [&](int r) {
      float e0, e1;
      if (CAP) {
        e0 = __builtin_amdgcn_exp2f(fmaf(neg2cap, x[2 * r], cap_m));
        e1 = __builtin_amdgcn_exp2f(fmaf(neg2cap, x[2 * r + 1], cap_m));
      } else {
        e0 = __builtin_amdgcn_exp2f(fmaf(x[2 * r], p.scale_log2, -m_use));
        e1 = __builtin_amdgcn_exp2f(fmaf(x[2 * r + 1], p.scale_log2, -m_use));
      }
      pk[r] = pack_bf16x2(e0, e1);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[r]), ones, l_run, false);
    };
#pragma unroll
    for (int r = 0; r < 4; ++r) prob_pair(r);

    // O^T += V^T . P^T: product v is half v / kDB (16 keys), block v % kDB.
    // Lane (lgrp, li16) reads chunk dlo/8 + 4*db + 2*(lgrp&1) + (li16&3)/2 of
    // rows r0 and r0 + 8 (transpose reads); block db is one XOR of the base.
    {
      const int32_t lgrp = ln >> 4;
      const int32_t li16 = ln & 15;
      const int32_t cl = 2 * (lgrp & 1) + ((li16 & 3) >> 1);
      const char* vbc = reinterpret_cast<const char*>(cur);
      const uint32_t rest = static_cast<uint32_t>(dlo * 2 + (li16 & 1) * 8);
      // One per-lane base for every read (as in the prefill kernel): the
      // swizzle reads only row bits 0-3, so half t is the immediate offset
      // t * 16 rows, and row r0 + 8 is the base XOR 32 plus 8 rows.
      const int32_t rb = 4 * (ln >> 5) + (li16 >> 2);
      const uint32_t vb0 = static_cast<uint32_t>(rb * kD * 2 + ((cl ^ swz(rb)) << 4)) + rest;
      auto vread = [&](int v) -> bf16x8 {
        const int t = v / kDB;
        const int db = v % kDB;
        // bit 8 of the base is clear: db's top bit is an offset addition
        const uint32_t x = static_cast<uint32_t>((db & 3) * 64);
        const int32_t imm = t * 16 * kD * 2 + (db >> 2) * 256;
        const i16x4 a0 = lds_read_tr16(vbc + (vb0 ^ x) + imm);
        const i16x4 a1 = lds_read_tr16(vbc + (vb0 ^ (x ^ 32u)) + imm + 8 * kD * 2);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int kV = 2 * kDB;
      constexpr int kLV = 2;
      bf16x8 va[kLV];
#pragma unroll
      for (int v = 0; v < kLV; ++v) va[v] = vread(v);
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int t = v / kDB;
        const int db = v % kDB;
        const bf16x8 bop = __builtin_bit_cast(bf16x8, u32x4{pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]});
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[v % kLV], bop, o[db], 0, 0, 0);
        if (v + kLV < kV) va[v % kLV] = vread(v + kLV);
        if (t == 0) {
#pragma unroll
          for (int r = 4; r < 8; ++r)
            if ((r - 4) * kDB / 4 == db) prob_pair(r);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // The next tile must have landed before it is read, and this slot and the
    // score buffer are rewritten only after every wave is done with them.
    wait_vmcnt<0>();
    __syncthreads();
  };
  for (int32_t ti = 0; ti < n_t; ti += 2) {
    step(ti, ts0, ts1);
    if (ti + 1 < n_t) step(ti + 1, ts1, ts0);
  }

  const float l_tot = xhalf_sum(l_run);
  // Partial of (sequence b, token tok, head) from workgroup w: slot w + b.
  if (col_ok) {
    const int64_t part = ((static_cast<int64_t>(blk.w) + b) * p.q_len + tok) * p.hq + head;
    float* dst = p.ws_o + part * kD + dlo;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        *reinterpret_cast<f32x4*>(dst + db * 32 + a * 8 + h * 4) =
            f32x4{o[db][4 * a], o[db][4 * a + 1], o[db][4 * a + 2], o[db][4 * a + 3]};
      }
    }
    if ((wave & 1) == 0 && h == 0) {
      p.ws_m[part] = m_run;
      p.ws_l[part] = l_tot;
    }
  }
  __syncthreads();   // LDS slots are reused by the next segment
  });
}

template <int D, int G, bool KEQV, bool CAP>
hipError_t launch_t(const DecodeArgs& a, const DecodeParams& prm, hipStream_t stream) {
  if (!a.per_seq) {   // the balanced ranges need the prefix sums of the spans
    const hipError_t e0 = launch_kernel(decode_plan_kernel, dim3(1), dim3(kPlanThreads), stream, prm);
    if (e0 != hipSuccess) return e0;
  }
  // Three or more 16-column blocks per KV head (many query heads per KV
  // head times several tokens): four blocks per workgroup share one stream
  // of cache tiles (bf16 caches, head width 256 or 512).
  constexpr int kCBW = 4;
  const bool tile = a.tile != 0;
  const bool wide = !tile && !prm.ks && D >= 256 && prm.n_cb >= 3;
  DecodeParams pp = prm;
  if (wide) pp.n_cb = (prm.n_cb + kCBW - 1) / kCBW;
  if (tile) pp.n_cb = (a.group * a.q_len + 63) / 64;   // 64-column groups
  const int64_t nblocks = decode_grid(a.hkv, a.n_wg, pp.n_cb, pp.xcd_log2);
  if (nblocks > 0x7fffffff) return hipErrorNotSupported;
  const dim3 grid(static_cast<uint32_t>(nblocks), 1u, 1u);
  hipError_t e = hipSuccess;
  if (tile) {
    if constexpr (D == 512 && KEQV) {
      e = launch_kernel(decode_tile_kernel<G, CAP>, grid, dim3(256), stream, pp);
    } else {
      return hipErrorNotSupported;   // the plan selects the tile kernel only for keys as values at width 512
    }
  } else if (prm.ks) {
    e = launch_kernel(decode_split_i8_kernel<D, G, KEQV, CAP>, grid, dim3(DecodeShape<D, 1>::kWaves * 64), stream, pp);
  } else if (wide) {
    if constexpr (D >= 256) {
      e = launch_kernel(decode_split_kernel<D, G, KEQV, CAP, kCBW>, grid, dim3(DecodeShape<D, kCBW>::kWaves * 64),
                        stream, pp);
    }
  } else {
    // Keys as values at width 512: the two-slot ring holds 32 KB, so four
    // workgroups would share a CU; 16 KB more of LDS per workgroup makes it
    // three, the round the plan sizes the grid for (Gemma-4 global layer:
    // 393 us at four per CU, 388 at three, 387 at two, 525 at one).
    constexpr uint32_t kReserve = (KEQV && D == 512) ? 16384u : 0u;
    e = launch_kernel(decode_split_kernel<D, G, KEQV, CAP, 1>, grid, dim3(DecodeShape<D, 1>::kWaves * 64), stream, pp,
                      kReserve);
  }
  if (e != hipSuccess) return e;
  if (a.per_seq && kFinalInKernel<D>) return hipSuccess;   // each sequence's only workgroup wrote its output
  return launch_kernel(decode_combine_kernel<D>,
                       dim3(static_cast<uint32_t>(a.hq * a.q_len), static_cast<uint32_t>(a.batch)), dim3(64), stream,
                       prm);
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
    default: return hipErrorNotSupported;
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
  prm.kv_start = a.kv_start;
  prm.prefix = a.ws_prefix;
  prm.lo = a.ws_lo;
  prm.batch = a.batch;
  prm.out = static_cast<uint16_t*>(a.out);
  prm.lse = a.lse;
  prm.ws_o = a.ws_o;
  prm.ws_m = a.ws_m;
  prm.ws_l = a.ws_l;
  prm.ks = a.k_scales;
  prm.vs = a.k_eq_v ? a.k_scales : a.v_scales;
  prm.max_ctx = a.max_ctx;
  prm.hq = a.hq;
  prm.hkv = a.hkv;
  prm.window = a.window;
  prm.n_wg = a.n_wg;
  prm.per_seq = a.per_seq;
  prm.q_len = a.q_len;
  prm.n_cb = (a.group * a.q_len + 15) / 16;
  // XCD-aware block placement needs a power-of-two XCD count; otherwise plain order.
  prm.xcd_log2 = 0;
  if (a.xcds > 1 && (a.xcds & (a.xcds - 1)) == 0)
    while ((1 << prm.xcd_log2) < a.xcds) ++prm.xcd_log2;
  const double log2e = 1.4426950408889634;
  prm.scale_log2 = static_cast<float>(a.scale * log2e);
  prm.cap_in2 = a.softcap > 0.0 ? static_cast<float>(2.0 * a.scale * log2e / a.softcap) : 0.f;
  prm.cap_log2 = static_cast<float>(a.softcap * log2e);
  switch (a.dim) {
    case 64: return dispatch_group<64>(a, prm, stream);
    case 256: return dispatch_group<256>(a, prm, stream);
    case 512: return dispatch_group<512>(a, prm, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace ga
