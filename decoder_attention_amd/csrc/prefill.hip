// Causal / sliding-window prefill attention for the Gemma family (gfx950).
//
// Work decomposition
//   One workgroup = 4 waves = 128 query "columns" of one (sequence, KV head):
//   the g query heads of the KV group times 128/g consecutive positions
//   (column c -> position p0 + c/g, head kvh*g + c%g).  Stacking the group's
//   heads makes every K/V tile staged in LDS serve 128 query rows, whatever g.
//   Grid = (q-blocks, KV heads, batch); q-blocks are issued last-first so the
//   longest causal rows start first.
//
// Head width 512 does not fit one wave's registers (Q^T 128 + O^T 256 per
// lane), so there the two waves of a pair share 32 columns and split D: each
// holds half of Q^T and O^T, computes a partial S^T over its half and the pair
// exchanges the partials through LDS (fp32 a+b == b+a, so both waves see the
// same scores bit for bit).  A workgroup then covers 64 columns.
//
// Per wave (32 columns), per tile of 32 keys:
//   S^T[32 keys x 32 cols] = K_tile . Q^T   (v_mfma_f32_32x32x16_bf16, fp32 acc)
//     A = K rows from LDS (ds_read_b128), B = Q^T held in registers.
//   In this orientation every lane owns ONE query column (lane % 32) and 16 of
//   the tile's keys, so the row max and row sum are in-lane plus one exchange
//   with lane ^ 32, and the output rescale is a per-lane scalar.
//   Scale, tanh soft cap, causal/window mask (boundary tiles only), online
//   softmax in the exp2 domain with a lazily updated running max (the
//   accumulators are rescaled only when a row's max grows by more than 2^8);
//   probabilities rounded to bf16 and the row sum taken over the same
//   rounded values.
//   The next K/V tile is loaded into registers while the current one is
//   computed and written to the second LDS buffer: one barrier per tile.
//   O^T[D x 32 cols] += V^T . P^T           (same MFMA)
//     A = V^T read straight from the row-major LDS tile with the gfx950
//     transpose read (ds_read_b64_tr_b16), B = P^T from the score registers.
//     With keys-as-values the same LDS tile is both K and V.
//   Tiles outside a wave's causal/window band are skipped by that wave.
//
// Sources: causal decoder attention (Gemma page), sliding-window local layers
// and the tanh logit soft cap (Gemma 2 page, introduction and Gemma2Model
// table), query_pre_attn_scalar (Gemma 2 / Gemma 3 tables), GQA/MQA head
// sharing (Gemma 2 "Grouped-query attention"; Gemma "multi-query attention"),
// keys-as-values global layers (Gemma 4 "K=V global MQA").
#include "ga_device.h"
#include "ga_kernels.h"

namespace ga {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kCols = 32;                 // query columns per wave
constexpr int kKeys = 32;                 // keys per tile
constexpr int kPad = 8;                   // bf16 elements of padding per LDS row
constexpr float kTau = 8.f;               // lazy-rescale threshold (log2 units)

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  int32_t seq, hq, hkv, window, n_qblocks;
  float scale_log2;   // scale * log2(e)            (no cap)
  float cap_in2;      // 2 * scale * log2(e) / cap  (cap: exp2 argument of tanh)
  float cap_log2;     // cap * log2(e)
};

template <int D>
struct DSplit {
  static constexpr int value = D > 256 ? 2 : 1;
};

template <int D, int G>
constexpr int positions_per_block() {
  return (kWaves / DSplit<D>::value) * kCols / G;
}

template <int D, int G, bool KEQV, bool CAP>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  constexpr int kSplit = DSplit<D>::value;
  constexpr int kDW = D / kSplit;     // D slice of one wave
  constexpr int kP = positions_per_block<D, G>();
  constexpr int kDS = kDW / 16;       // k-steps of QK^T per wave
  constexpr int kDB = kDW / 32;       // 32-row blocks of O^T per wave
  constexpr int kLd = D + kPad;       // LDS row pitch (elements)
  constexpr int kChunks = kKeys * D / 8;   // 16-byte pieces per tile
  constexpr int kPer = kChunks / kThreads;  // pieces per thread
  constexpr int kTile = kKeys * kLd;        // elements per LDS tile buffer
  static_assert(kChunks % kThreads == 0, "tile must split evenly over the workgroup");

  // Two tile buffers: the next tile is written while the current one is read.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2 * kTile];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[KEQV ? 8 : 2 * kTile];
  __shared__ __attribute__((aligned(16))) float sx_lds[kSplit > 1 ? kWaves * 64 * 16 : 4];

  const int32_t S = p.seq;
  const int32_t qb = p.n_qblocks - 1 - static_cast<int32_t>(blockIdx.x);
  const int32_t kvh = blockIdx.y;
  const int32_t b = blockIdx.z;
  const int32_t p0 = qb * kP;
  const int32_t tid = threadIdx.x;
  const int32_t wave = tid >> 6;
  const int32_t lane = tid & 63;
  const int32_t j = lane & 31;       // column within the wave
  const int32_t h = lane >> 5;       // half of the wave
  const int32_t cw = wave / kSplit;  // column group of this wave
  const int32_t dlo = (wave % kSplit) * kDW;  // first d of this wave's slice
  const int32_t c = cw * kCols + j;
  const int32_t pos = p0 + c / G;
  const int32_t head = kvh * G + c % G;
  const bool col_valid = pos < S;
  const int32_t pos_m = col_valid ? pos : S - 1;
  const int32_t W = p.window;

  // Q^T operand: lane holds d = ds*16 + h*8 + [0, 8) of its column.
  bf16x8 qf[kDS];
  {
    const uint16_t* qrow = p.q + ((static_cast<int64_t>(b) * S + pos_m) * p.hq + head) * D + dlo + h * 8;
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) {
      qf[ds] = *reinterpret_cast<const bf16x8*>(qrow + ds * 16);
    }
  }

  const int32_t w_lo = p0 + (cw * kCols) / G;                       // wave's first position
  const int32_t w_hi = min(p0 + (cw * kCols + kCols - 1) / G, S - 1); // wave's last valid position
  const int32_t kv_end = min(S, p0 + kP);
  int32_t kv_begin = W > 0 ? max(0, p0 - W + 1) : 0;
  kv_begin &= ~(kKeys - 1);

  f32x16 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int64_t kv_row0 = static_cast<int64_t>(b) * S;
  const int32_t n_tiles = (kv_end - kv_begin + kKeys - 1) / kKeys;

  // Register staging of one tile: thread tid owns 16-byte pieces tid + i*256.
  u32x4 kreg[kPer];
  u32x4 vreg[KEQV ? 1 : kPer];
  auto load_tile = [&](int32_t kt) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int32_t idx = tid + i * kThreads;
      const int32_t row = idx / (D / 8);
      const int32_t c8 = idx % (D / 8);
      const int32_t key = kt + row;
      kreg[i] = u32x4{0u, 0u, 0u, 0u};
      if (!KEQV) vreg[KEQV ? 0 : i] = u32x4{0u, 0u, 0u, 0u};
      if (key < S) {
        const int64_t off = ((kv_row0 + key) * p.hkv + kvh) * D + c8 * 8;
        kreg[i] = *reinterpret_cast<const u32x4*>(p.k + off);
        if (!KEQV) vreg[KEQV ? 0 : i] = *reinterpret_cast<const u32x4*>(p.v + off);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int32_t idx = tid + i * kThreads;
      const int32_t row = idx / (D / 8);
      const int32_t c8 = idx % (D / 8);
      *reinterpret_cast<u32x4*>(&k_lds[buf * kTile + row * kLd + c8 * 8]) = kreg[i];
      if (!KEQV) *reinterpret_cast<u32x4*>(&v_lds[buf * kTile + row * kLd + c8 * 8]) = vreg[KEQV ? 0 : i];
    }
  };

  if (n_tiles > 0) {
    load_tile(kv_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int32_t it = 0; it < n_tiles; ++it) {
    const int32_t kt = kv_begin + it * kKeys;
    const int32_t buf = it & 1;
    const bool more = it + 1 < n_tiles;
    if (more) load_tile(kt + kKeys);      // in flight while this tile is computed
    const uint16_t* kb = k_lds + buf * kTile;
    const uint16_t* vb = (KEQV ? k_lds : v_lds) + buf * kTile;

    // Does this wave see any key of the tile?  (wave-uniform; equal for both
    // waves of a D-split pair)
    const bool need = kt <= w_hi && (W == 0 || kt + kKeys - 1 >= w_lo - W + 1);
    const bool full = kt + kKeys - 1 <= w_lo && (W == 0 || kt >= w_hi - W + 1);

    // S^T = K . Q^T (partial over this wave's D slice when split)
    f32x16 sacc = f32x16{};
    if (need) {
#pragma unroll
      for (int ds = 0; ds < kDS; ++ds) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kb[j * kLd + dlo + ds * 16 + h * 8]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], sacc, 0, 0, 0);
      }
    }
    if (kSplit > 1) {
      // [wave][r/4][lane] float4 layout: consecutive lanes, consecutive 16 bytes.
      f32x4* mine = reinterpret_cast<f32x4*>(sx_lds) + wave * 256 + lane;
      const f32x4* other = reinterpret_cast<const f32x4*>(sx_lds) + (wave ^ 1) * 256 + lane;
#pragma unroll
      for (int r = 0; r < 16; r += 4) mine[(r / 4) * 64] = f32x4{sacc[r], sacc[r + 1], sacc[r + 2], sacc[r + 3]};
      __syncthreads();
      if (need) {
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const f32x4 t4 = other[(r / 4) * 64];
          sacc[r] += t4[0];
          sacc[r + 1] += t4[1];
          sacc[r + 2] += t4[2];
          sacc[r + 3] += t4[3];
        }
      }
    }

    if (need) {
      // Logits in the exp2 domain; lane holds keys kt + (r/4)*8 + h*4 + r%4.
      float x[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float t;
        if (CAP) {
          // cap * tanh(s*scale/cap) = cap - 2*cap / (exp(2*s*scale/cap) + 1)
          const float e = __builtin_amdgcn_exp2f(sacc[r] * p.cap_in2);
          t = fmaf(-2.f * p.cap_log2, __builtin_amdgcn_rcpf(e + 1.f), p.cap_log2);
        } else {
          t = sacc[r] * p.scale_log2;
        }
        if (!full) {
          const int32_t key = kt + (r >> 2) * 8 + h * 4 + (r & 3);
          const bool ok = key <= pos_m && (W == 0 || pos_m - key < W);
          t = ok ? t : -INFINITY;
        }
        x[r] = t;
        mx = fmaxf(mx, t);
      }
      mx = wave_max_xor32(mx);
      // The running max only moves when the tile exceeds it by more than
      // kTau (log2 units): probabilities then stay <= 2^kTau and the output
      // rescale, a pass over every accumulator, is rare.
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

      uint32_t pk[8];
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float e0 = __builtin_amdgcn_exp2f(x[2 * r] - m_use);
        const float e1 = __builtin_amdgcn_exp2f(x[2 * r + 1] - m_use);
        pk[r] = pack_bf16x2(e0, e1);
        ls += lo_bf16(pk[r]) + hi_bf16(pk[r]);
      }
      l_run += ls;

      // O^T += V^T . P^T, two 16-key halves per tile.
      const int32_t grp = lane >> 4;
      const int32_t i16 = lane & 15;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 pb = u32x4{pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]};
        const bf16x8 bop = __builtin_bit_cast(bf16x8, pb);
        const int32_t r0 = 16 * t + 4 * h + (i16 >> 2);
        const int32_t cbase = (grp & 1) * 16 + 4 * (i16 & 3);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const i16x4 a0 = lds_read_tr16(&vb[r0 * kLd + dlo + db * 32 + cbase]);
          const i16x4 a1 = lds_read_tr16(&vb[(r0 + 8) * kLd + dlo + db * 32 + cbase]);
          const bf16x8 aop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, o[db], 0, 0, 0);
        }
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = wave_sum_xor32(l_run);
  if (col_valid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = p.out + ((static_cast<int64_t>(b) * S + pos) * p.hq + head) * D + dlo;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int32_t d = db * 32 + a * 8 + h * 4;
        u32x2 w2;
        w2[0] = pack_bf16x2(o[db][4 * a] * inv, o[db][4 * a + 1] * inv);
        w2[1] = pack_bf16x2(o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d) = w2;
      }
    }
    if (p.lse && h == 0 && dlo == 0) {
      p.lse[(static_cast<int64_t>(b) * p.hq + head) * S + pos] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int G, bool KEQV, bool CAP>
hipError_t launch_t(const PrefillArgs& a, const PrefillParams& prm, hipStream_t stream) {
  constexpr int kP = positions_per_block<D, G>();
  PrefillParams pp = prm;
  pp.n_qblocks = (a.seq + kP - 1) / kP;
  const dim3 grid(static_cast<uint32_t>(pp.n_qblocks), static_cast<uint32_t>(a.hkv), static_cast<uint32_t>(a.batch));
  hipLaunchKernelGGL((prefill_kernel<D, G, KEQV, CAP>), grid, dim3(kThreads), 0, stream, pp);
  return hipGetLastError();
}

template <int D, int G>
hipError_t dispatch_flags(const PrefillArgs& a, const PrefillParams& prm, hipStream_t s) {
  const bool cap = a.softcap > 0.0;
  if (a.k_eq_v) return cap ? launch_t<D, G, true, true>(a, prm, s) : launch_t<D, G, true, false>(a, prm, s);
  return cap ? launch_t<D, G, false, true>(a, prm, s) : launch_t<D, G, false, false>(a, prm, s);
}

template <int D>
hipError_t dispatch_group(const PrefillArgs& a, const PrefillParams& prm, hipStream_t s) {
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

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.seq == 0) return hipSuccess;
  PrefillParams prm;
  prm.q = static_cast<const uint16_t*>(a.q);
  prm.k = static_cast<const uint16_t*>(a.k);
  prm.v = static_cast<const uint16_t*>(a.v);
  prm.out = static_cast<uint16_t*>(a.out);
  prm.lse = a.lse;
  prm.seq = a.seq;
  prm.hq = a.hq;
  prm.hkv = a.hkv;
  prm.window = a.window;
  prm.n_qblocks = 0;
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
