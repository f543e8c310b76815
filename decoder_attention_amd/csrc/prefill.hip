// Causal / sliding-window prefill attention for the Gemma family (gfx950).
//
// Work decomposition
//   One workgroup = 4 waves covering the query "columns" of one (sequence,
//   KV head): the g query heads of the KV group times consecutive positions
//   (column c -> position p0 + c/g, head kvh*g + c%g).  Stacking the group's
//   heads makes every K/V tile staged in LDS serve 128 query rows, whatever g.
//   Head width 512 does not fit one wave's registers (Q^T 128 + O^T 256 per
//   lane), so there the two waves of a pair share 32 columns and split D: each
//   holds half of Q^T and O^T, computes a partial S^T over its half and the
//   pair exchanges the partials through LDS (fp32 a+b == b+a, so both waves
//   see the same scores bit for bit).  A workgroup then covers 64 columns.
//   Soft-capped global layers of width 256 take the WIDE form: eight waves
//   (256 columns) in one workgroup per CU, each staged tile serving twice the
//   query rows.
//
// Block order
//   The dispatcher deals linear block ids round-robin over the XCDs (8 on a
//   whole MI355X, fewer on a partition; the host passes the count), each with
//   its own L2.  Blocks are renumbered so that the blocks an XCD runs
//   together belong to as few (sequence, KV head) pairs as possible -- they
//   then stream the same K/V tiles through that XCD's L2 -- while every XCD
//   gets the same amount of work; inside a pair, the longest causal rows go
//   first.  On short windows the XCDs sharing a pair take contiguous runs of
//   its blocks, and every block visits its window's tiles in an order shared
//   by all blocks (the tile whose index is congruent to the step), so blocks
//   running together read the same tile at the same time.
//
// K/V staging
//   Tiles of 32 keys are copied HBM -> LDS by the gfx950 direct-to-LDS loads
//   (buffer_load_dwordx4 ... lds, no register round trip) into a ring of three
//   buffers (two when three do not fit), up to two tiles ahead of the one
//   being computed; one barrier per tile.
//   Rows are unpadded and their 16-byte chunks are XOR-swizzled (chunk c of
//   row r sits at c ^ f(r)), which keeps both the K operand reads
//   (ds_read_b128, 16 rows per 256-byte phase) and the transposed V reads
//   (ds_read_b64_tr_b16, 4 rows x 4 chunks per half-wave) free of bank
//   conflicts.
//
// Per wave (32 columns), per tile of 32 keys:
//   S^T[32 keys x 32 cols] = K_tile . Q^T   (v_mfma_f32_32x32x16_bf16, fp32 acc)
//     A = K rows from LDS, B = Q^T held in registers.
//   In this orientation every lane owns ONE query column (lane % 32) and 16 of
//   the tile's keys, so the row max and row sum are in-lane plus one
//   v_permlane32_swap with the other half of the wave.
//   Scale, tanh soft cap, causal/window mask (boundary tiles only), online
//   softmax in the exp2 domain with a lazily updated running max (the
//   accumulators are rescaled only when a row's max grows by more than 2^8)
//   -- or, on soft-capped layers, the cap itself as a fixed maximum, with a
//   recompute for workgroups whose rows lie far below it; probabilities
//   rounded to bf16 and the row sum taken over the same rounded values.
//   O^T[D x 32 cols] += V^T . P^T           (same MFMA)
//     A = V^T read straight from the row-major tile with the transpose read,
//     B = P^T from the score registers.  With keys-as-values the same LDS
//     tile is both K and V.
//   Tiles outside a wave's causal/window band are skipped by that wave.
//   A wave raises its priority while it issues the matrix products, so the
//   SIMD's other wave runs its softmax in the gaps (not on the capped
//   four-wave form, where it measured slower).
//
// Output
//   O^T leaves the accumulators through the idle ring: each wave parks its
//   32 columns in LDS and writes them back in row order, 16 bytes per lane,
//   so a store instruction covers whole cache lines instead of 16-byte
//   pieces of 32 rows.
//
// Sources: causal decoder attention (Gemma page), sliding-window local layers
// and the tanh logit soft cap (Gemma 2 page, introduction and Gemma2Model
// table), query_pre_attn_scalar (Gemma 2 / Gemma 3 tables), GQA/MQA head
// sharing (Gemma 2 "Grouped-query attention"; Gemma "multi-query attention"),
// keys-as-values global layers (Gemma 4 "K=V global MQA").
#include <type_traits>

#include "ga_device.h"
#include "ga_kernels.h"

namespace ga {

namespace {

constexpr int kCols = 32;                 // query columns per wave
constexpr int kKeys = 32;                 // keys per tile
constexpr int kLdsBudget = 160 * 1024;   // bytes of LDS per workgroup
constexpr float kTau = 8.f;               // lazy-rescale threshold (log2 units)

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  const int32_t* seq_start;   // padded batch: sequence b keeps rows [start, end) (null: 0, seq)
  const int32_t* seq_end;
  int32_t seq, hq, hkv, window, n_qblocks, n_qblocks_pad, batch;
  int32_t xcd_log2;   // the dispatcher deals linear block ids round-robin over 2^xcd_log2 XCDs
  int32_t xcd_runs;   // XCDs sharing a pair take contiguous runs of its q-blocks (else interleaved)
  float scale_log2;   // scale * log2(e)            (no cap)
  float cap_in2;      // 2 * scale * log2(e) / cap  (cap: exp2 argument of tanh)
  float cap_log2;     // cap * log2(e)
  // Query rotary inside the kernel (the fused form): position pos0[b] + s
  // (pos0 null: s); pair i turns by (pos0[b] + s) * rot_c0 * rot_w1^i
  // revolutions, rot_w1 = theta^(-2/D), rot_c0 = 1 / (2 pi pos_div).
  const int32_t* pos0;
  double rot_w1, rot_c0;
};

template <int D>
struct DSplit {
  static constexpr int value = D > 256 ? 2 : 1;
};



// XOR pattern of the 16-byte chunks of LDS row r.  The LDS serves 256 bytes
// (64 banks) per cycle: a ds_read_b128 phase is 16 lanes = 16 consecutive K
// rows at one logical chunk, a ds_read_b64_tr_b16 half-wave is 4 rows (aligned
// to 4) x 4 chunks (aligned to 4).  Rows of >= 256 bytes: a 4-bit rotate of
// r, a permutation of 16 consecutive rows whose bits 2-3 differ within every
// aligned group of 4 rows.  128-byte rows (D = 64) pair up in a 256-byte
// window, so the pattern uses 3 bits and separates rows r and r + 2.
template <int D>
__device__ __forceinline__ int32_t swz(int32_t r) {
  if constexpr (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// The lane index, hidden from loop-invariant code motion: lane-derived LDS
// and DMA offsets are recomputed each tile (a few integer ops) instead of
// being held in registers across the loop, which would not fit.
__device__ __forceinline__ int32_t lane_id_here() {
  int32_t l = static_cast<int32_t>(threadIdx.x);
  asm volatile("" : "+v"(l));
  return l & 63;
}

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

// Linear block id -> (pair = b*Hkv + kvh, t = rank in heavy-first order), or
// t >= n_qblocks for padding blocks.
__device__ __forceinline__ void block_work(const PrefillParams& p, int32_t& pair, int32_t& t) {
  const int32_t lin = static_cast<int32_t>(blockIdx.x);
  const int32_t npairs = p.batch * p.hkv;
  const int32_t nq = p.n_qblocks_pad;
  const int32_t nx = 1 << p.xcd_log2;
  const int32_t xcd = lin & (nx - 1);
  const int32_t slot = lin >> p.xcd_log2;
  if ((npairs & (nx - 1)) == 0) {          // every XCD owns npairs/nx pairs, one after another
    pair = xcd + nx * (slot / nq);
    t = slot % nq;
  } else if ((nx % npairs) == 0) {         // nx/npairs XCDs share a pair
    const int32_t k = nx / npairs;
    pair = xcd % npairs;
    // Uniform work (a window much shorter than the sequence): each XCD takes
    // one contiguous run, so the blocks it runs together share their keys in
    // its L2.  Causal rows grow with the position: interleaving keeps the
    // XCDs' shares equal.
    t = p.xcd_runs ? (xcd / npairs) * (nq / k) + slot : slot * k + xcd / npairs;
  } else {
    pair = lin / nq;
    t = lin % nq;
  }
}

// Two waves per SIMD (two workgroups per CU) wherever the LDS ring allows:
// the register budget is then 256 VGPRs per lane and one wave's softmax
// overlaps the other's matrix work.
template <int D, bool KEQV>
constexpr int waves_per_simd() {
  return (D <= 256 || KEQV) ? 2 : 1;
}

// Waves per workgroup: four, one per SIMD; with two waves per SIMD two
// workgroups share a CU.  WIDE: one workgroup of eight (two per SIMD) with a
// three-tile ring, every K/V tile serving twice the columns.  On a
// soft-capped global layer of width 256 it measured 4.6% faster (Gemma-2
// pair, 935 against 894 TFLOP/s); on a 4096-key window it was 16% slower and
// without the cap about even, so it is taken only for the first.
template <int D, bool KEQV, bool WIDE>
constexpr int pf_waves() {
  return WIDE ? 8 : 4;
}

template <int D, int G, bool KEQV, bool WIDE>
constexpr int positions_per_block() {
  return (pf_waves<D, KEQV, WIDE>() / DSplit<D>::value) * kCols / G;
}

template <int D, int G, bool KEQV, bool CAP, bool WIDE, bool QROPE>
__global__ __launch_bounds__((pf_waves<D, KEQV, WIDE>() * 64)) __attribute__((amdgpu_waves_per_eu(waves_per_simd<D, KEQV>(), 2)))
void prefill_kernel(PrefillParams p) {
  constexpr int kWaves = pf_waves<D, KEQV, WIDE>();
  constexpr int kSplit = DSplit<D>::value;
  constexpr int kDW = D / kSplit;            // D slice of one wave
  constexpr int kP = positions_per_block<D, G, KEQV, WIDE>();
  constexpr int kDS = kDW / 16;              // k-steps of QK^T per wave
  constexpr int kDB = kDW / 32;              // 32-row blocks of O^T per wave
  constexpr int kRowChunks = D / 8;          // 16-byte chunks per key row
  constexpr int kTileElems = kKeys * D;
  constexpr int kOps = kKeys * kRowChunks / 64;                  // 1 KB DMA ops per tensor per tile
  constexpr int kWaveLoads = (kOps + kWaves - 1) / kWaves;        // DMA ops per wave per tensor
  constexpr int kLoadsPerTile = kWaveLoads * (KEQV ? 1 : 2);
  static_assert(kKeys * kRowChunks % 64 == 0, "tile must split into whole 1 KB ops");
  // Ring depth: three tiles when the CU's workgroups still fit in LDS, else two.
  constexpr int kSxBytes = kSplit > 1 ? kWaves * 64 * 16 * 4 : 16;
  constexpr int kTileBytes = kTileElems * 2 * (KEQV ? 1 : 2);
  constexpr int kWgPerCu = waves_per_simd<D, KEQV>() * 4 / kWaves;
  constexpr int kBufs = kWgPerCu * (3 * kTileBytes + kSxBytes) <= kLdsBudget ? 3 : 2;
  constexpr int kAhead = kBufs - 1;          // tiles in flight beyond the one computed
  // Wave priority while a wave issues its matrix products (QK^T, PV): when
  // both waves of a SIMD are ready, the one feeding the matrix core goes
  // first and the other's softmax fills the gaps.  Same-box runs: Gemma-4
  // global -4 to -5%, Gemma-3 window 512 -2 to -3%, Gemma-2 global -1 to -2.5%,
  // Gemma-3 global -0.5 to -0.7%; the capped four-wave form (Gemma-2 window
  // 4096) lost about 1%, so it keeps the default priority.
  constexpr int kMatPrio = (CAP && !WIDE) ? 0 : 3;

  // One LDS array per ring slot: every access names its slot at compile time
  // (the loop is unrolled by the ring depth), so the compiler can tell a read
  // of the current tile from the copies still landing in the other slots and
  // does not wait for them.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds1[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds2[kBufs > 2 ? kTileElems : 8];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[KEQV ? 8 : kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[KEQV ? 8 : kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds2[(KEQV || kBufs < 3) ? 8 : kTileElems];
  __shared__ __attribute__((aligned(16))) float sx_lds[kSplit > 1 ? kWaves * 64 * 16 : 4];
  lds_poison(k_lds0, k_lds1, k_lds2, v_lds0, v_lds1, v_lds2, sx_lds);
  auto kslot = [&](auto B) -> uint16_t* {
    if constexpr (decltype(B)::value == 0) return k_lds0;
    else if constexpr (decltype(B)::value == 1) return k_lds1;
    else return k_lds2;
  };
  auto vslot = [&](auto B) -> uint16_t* {
    if constexpr (KEQV) return kslot(B);
    else if constexpr (decltype(B)::value == 0) return v_lds0;
    else if constexpr (decltype(B)::value == 1) return v_lds1;
    else return v_lds2;
  };
  // After the last tile the ring arrays hold each wave's output slice
  // (32 columns x kDW) on its way to memory, whole or, where the ring is too
  // small for every wave's slice, half of it per pass: array n of the ring
  // (K slots, then V slots) holds kSlicePer of them.
  constexpr int kRingArrays = KEQV ? kBufs : 2 * kBufs;
  constexpr int kWhole = kCols * kDW * 2;
  constexpr int kPasses = kRingArrays * (kTileElems * 2 / kWhole) >= kWaves ? 1 : 2;
  constexpr int kSlice = kWhole / kPasses;
  constexpr int kSlicePer = kTileElems * 2 / kSlice;
  constexpr bool kStageO = kSlicePer >= 1 && kRingArrays * kSlicePer >= kWaves && kDB % kPasses == 0;
  auto stage_region = [&](int n) -> uint16_t* {
    if (n == 0) return k_lds0;
    if constexpr (kBufs > 2) {
      if (n == 2) return k_lds2;
    }
    if constexpr (!KEQV) {
      if (n == kBufs) return v_lds0;
      if (n == kBufs + 1) return v_lds1;
      if constexpr (kBufs > 2) {
        if (n == kBufs + 2) return v_lds2;
      }
    }
    return k_lds1;
  };

  int32_t pair, tq;
  block_work(p, pair, tq);
  if (tq >= p.n_qblocks) return;                       // padding block (uniform)
  const int32_t S = p.seq;
  const int32_t qb = p.n_qblocks - 1 - tq;
  const int32_t b = pair / p.hkv;
  const int32_t kvh = pair % p.hkv;
  const int32_t p0 = qb * kP;
  const int32_t tid = threadIdx.x;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar from here on
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
  // Kept rows of this sequence (a padded batch keeps [r_lo, r_hi)); padded
  // rows are neither queries nor keys.
  int32_t r_lo = 0, r_hi = S;
  if (p.seq_start) r_lo = min(max(p.seq_start[b], 0), S);
  if (p.seq_end) r_hi = min(max(p.seq_end[b], r_lo), S);
  const bool kept = pos >= r_lo && pos < r_hi;
  const int32_t key_lo = max(W > 0 ? pos_m - W + 1 : 0, r_lo);   // first key this column may see

  // The wave's kept positions [w_lo, w_hi] (empty when w_lo > w_hi).
  const int32_t w_lo = max(p0 + (cw * kCols) / G, r_lo);
  const int32_t w_hi = min(min(p0 + (cw * kCols + kCols - 1) / G, S - 1), r_hi - 1);
  const int32_t kv_end = min(min(S, p0 + kP), r_hi);
  int32_t kv_begin = max(W > 0 ? max(0, p0 - W + 1) : 0, r_lo);
  kv_begin &= ~(kKeys - 1);
  const int32_t n_tiles = max(0, (kv_end - kv_begin + kKeys - 1) / kKeys);
  // Tile order on a sliding window: step s visits the block's tile whose
  // absolute index is congruent to s modulo n_tiles.  Blocks with the same
  // tile count (every block past the first window) then read the same tile,
  // or tiles n_tiles apart, at the same step, so the blocks an XCD runs
  // together share each K/V tile in its L2 instead of each streaming its own
  // part of the window.  The softmax does not depend on the order; without a
  // window (first key 0) the order is the plain one.
  int32_t rot = 0;
  if (W > 0 && n_tiles > 0) rot = (n_tiles - (kv_begin / kKeys) % n_tiles) % n_tiles;
  auto tile_key = [&](int32_t s) -> int32_t {
    int32_t r = s + rot;
    r -= r >= n_tiles ? n_tiles : 0;
    return kv_begin + r * kKeys;
  };

  // Issue the direct-to-LDS copies of the tile starting at key kt into ring
  // slot B.  Addresses are a wave-uniform tile base (a buffer resource over
  // the tile's 32 rows) plus a 32-bit per-lane byte offset (row * row pitch +
  // chunk), so they need no 64-bit registers.  The buffer form keeps the
  // compiler's LDS-read waits partial (the global-segment form made every
  // consumer of an LDS read wait for all of them).
  const char* kbase = reinterpret_cast<const char*>(p.k) + static_cast<int64_t>(b) * S * p.hkv * D * 2;
  const char* vbase = reinterpret_cast<const char*>(KEQV ? p.k : p.v) + static_cast<int64_t>(b) * S * p.hkv * D * 2;
  const uint32_t row_pitch = static_cast<uint32_t>(p.hkv) * D * 2;
  // Per-lane byte offsets of this wave's copy ops inside a tile (rows not
  // clamped).  Where one wave covers all of D (kHold), only op 0's offset is
  // kept: op i's is (doff[0] ^ dx) + drow with wave-uniform dx and drow (the
  // swizzle of op i's rows differs from op 0's by a pattern that does not
  // depend on the lane, and the row term, a multiple of the row pitch, has no
  // bits in the chunk field), one instruction per op instead of a register
  // per op; the registers go to the LDS read bases held across the loop
  // (below).  At D = 512 every op keeps its register and the read bases are
  // recomputed each tile: holding them there spilled and ran slower.
  constexpr bool kHold = kSplit == 1;
  uint32_t doff[kHold ? 1 : kWaveLoads];
#pragma unroll
  for (int i = 0; i < (kHold ? 1 : kWaveLoads); ++i) {
    const int32_t pc = (wave * kWaveLoads + i) * 64 + lane;
    const int32_t row = pc / kRowChunks;
    const int32_t lc = (pc % kRowChunks) ^ swz<D>(row);       // logical chunk held at pc
    doff[i] = static_cast<uint32_t>(row) * row_pitch + static_cast<uint32_t>(lc) * 16u;
  }
  auto op_dx = [&](int i) -> uint32_t {
    const int32_t r0 = (wave * kWaveLoads * 64) / kRowChunks;
    const int32_t ri = ((wave * kWaveLoads + i) * 64) / kRowChunks;
    return static_cast<uint32_t>(swz<D>(ri) ^ swz<D>(r0)) << 4;
  };
  auto op_drow = [&](int i) -> uint32_t {
    const int32_t r0 = (wave * kWaveLoads * 64) / kRowChunks;
    const int32_t ri = ((wave * kWaveLoads + i) * 64) / kRowChunks;
    return static_cast<uint32_t>(ri - r0) * row_pitch;
  };
  // A dead tile (live = false) gets a zero-byte resource: its copies read no
  // memory and write zeros into the slot.
  auto issue = [&](int32_t kt, auto B, bool live = true) {
    const int64_t tile_off = live ? (static_cast<int64_t>(kt) * p.hkv + kvh) * D * 2 : 0;
    const char* kt_base = kbase + tile_off;
    const char* vt_base = vbase + tile_off;
    // Rows outside the kept range repeat its first or last row (masked), so
    // no padded row is ever read.
    const bool tail = kt < r_lo || kt + kKeys > r_hi;
    uint16_t* kdst = kslot(B);
    uint16_t* vdst = vslot(B);
    const uint32_t nbytes = live ? kKeys * row_pitch : 0u;
    const __amdgpu_buffer_rsrc_t krs = raw_rsrc(kt_base, nbytes);
    const __amdgpu_buffer_rsrc_t vrs = raw_rsrc(vt_base, nbytes);
    // (the pinned base keeps the compiler from hoisting every op's offset
    // out of the loop into a register of its own)
    uint32_t dbase = doff[0];
    if constexpr (kHold) asm volatile("" : "+v"(dbase));
#pragma unroll
    for (int i = 0; i < kWaveLoads; ++i) {
      if (kOps % kWaves != 0 && wave * kWaveLoads + i >= kOps) break;   // uniform per wave
      const int32_t base = (wave * kWaveLoads + i) * 64;     // first physical chunk of this op
      uint32_t off;
      if constexpr (kHold) off = (dbase ^ op_dx(i)) + op_drow(i);
      else off = doff[i];
      if (tail) {
        const int32_t ln = lane_id_here();
        const int32_t pc = base + ln;
        const int32_t row = pc / kRowChunks;
        const int32_t lc = (pc % kRowChunks) ^ swz<D>(row);
        off = static_cast<uint32_t>(min(max(row, r_lo - kt), r_hi - 1 - kt)) * row_pitch +
              static_cast<uint32_t>(lc) * 16u;
      }
      copy_to_lds(krs, off, kdst + base * 8);
      if (!KEQV) copy_to_lds(vrs, off, vdst + base * 8);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  const int32_t pos_base = (QROPE && p.pos0) ? p.pos0[b] : 0;   // first position of sequence b

  // Q^T operand: lane holds d = ds*16 + h*8 + [0, 8) of its column.  With the
  // fused query rotary q is loaded before the first tiles' copies, so that the
  // rotation can start while those are in flight.
  bf16x8 qf[kDS];
  auto load_q = [&]() {
    const uint16_t* qrow = p.q + ((static_cast<int64_t>(b) * S + pos_m) * p.hq + head) * D + dlo + h * 8;
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) qf[ds] = *reinterpret_cast<const bf16x8*>(qrow + ds * 16);
  };
  if constexpr (QROPE) {
    // Every first-tile copy is issued (dead ones copy nothing), so the wait
    // for q below is one constant count.
    load_q();
    issue(tile_key(0), I0{}, 0 < n_tiles);
    if constexpr (kAhead > 1) issue(tile_key(1), I1{}, 1 < n_tiles);
  } else {
    if (0 < n_tiles) issue(tile_key(0), I0{});
    if (kAhead > 1 && 1 < n_tiles) issue(tile_key(1), I1{});
    load_q();
  }

  f32x16 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x16{};
  // Capped layers at one wave per D first run with a fixed maximum: every
  // capped logit is below the cap, so cap (log2 units) bounds the row max
  // and probabilities 2^(logit - cap) need neither a running max nor a
  // rescale.  A row whose logits all lie far below the cap would push its
  // probabilities toward the bottom of the fp32/bf16 range; the workgroup
  // then recomputes with a tracked maximum (below).
  // The fixed maximum is the cap rounded up to an integer, so that the lse
  // can be formed exactly from the sum's exponent (at the end).
  // Caps above 96 log2 units (about 66.5) keep the running maximum from the
  // start: there an ordinary row's probabilities relative to the cap would
  // already sit below the recompute threshold (2^-100).
  constexpr bool kFixedMax = CAP && kSplit == 1;
  const bool fixed = kFixedMax && p.cap_log2 <= 96.f;   // uniform
  const float m_fix = kFixedMax ? ceilf(p.cap_log2) : 0.f;
  float m_run = fixed ? m_fix : -INFINITY;
  bool tracked = !fixed;   // uniform: the running maximum is in use
  float l_run = 0.f;

  if constexpr (!QROPE) wait_vmcnt<0>();   // Q^T and the first tiles
  if constexpr (QROPE) {
    // Wait for q only: the copies of the first tiles, issued after it, stay
    // in flight during the rotation.
    static_assert(kOps % kWaves == 0, "every wave issues kLoadsPerTile copies per tile");
    wait_vmcnt<(kAhead > 1 ? 2 : 1) * kLoadsPerTile>();
    // The fused form: q arrives before rotary, and each lane turns its own
    // column in registers.  Rotate-half pairs (i, i + D/2): the lane holds
    // i = ds*16 + h*8 + [0, 8) at step ds < kDS/2 and its partner at step
    // ds + kDS/2.  The frequencies follow rotary_rev_freq's chain of products
    // (c0, times w8 for h = 1, times w16 per step, times w1 per element) and
    // the angle, cosine, sine and turn are rotary_cos_sin and rotary_turn, the
    // prologue's own arithmetic, so the rotated query rounds to the same bf16
    // values as the prologue's output.
    static_assert(kSplit == 1, "the rotary partner of a dim must sit in the same lane");
    const double pd = static_cast<double>(pos_base) + static_cast<double>(pos_m);
    const double w1 = p.rot_w1;
    const double w2 = w1 * w1, w4 = w2 * w2, w8 = w4 * w4, w16 = w8 * w8;
    double f_ds = h ? p.rot_c0 * w8 : p.rot_c0;
#pragma unroll
    for (int ds = 0; ds < kDS / 2; ++ds) {
      u32x4 lo = __builtin_bit_cast(u32x4, qf[ds]);
      u32x4 hi = __builtin_bit_cast(u32x4, qf[ds + kDS / 2]);
      double f = f_ds;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 cs0 = rotary_cos_sin(pd, f);
        f *= w1;
        const float2 cs1 = rotary_cos_sin(pd, f);
        f *= w1;
        const float a0 = lo_bf16(lo[e]), a1 = hi_bf16(lo[e]);
        const float b0 = lo_bf16(hi[e]), b1 = hi_bf16(hi[e]);
        lo[e] = pack_bf16x2(rotary_turn(a0, b0, cs0.x, -cs0.y), rotary_turn(a1, b1, cs1.x, -cs1.y));
        hi[e] = pack_bf16x2(rotary_turn(b0, a0, cs0.x, cs0.y), rotary_turn(b1, a1, cs1.x, cs1.y));
      }
      qf[ds] = __builtin_bit_cast(bf16x8, lo);
      qf[ds + kDS / 2] = __builtin_bit_cast(bf16x8, hi);
      f_ds *= w16;
    }
    // Pin the rotated values here, before the wait for the tiles: left alone,
    // the compiler moved the whole rotation (register-only work) past that
    // wait and the barrier, next to its first use.
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) asm volatile("" : "+v"(qf[ds]));
    wait_vmcnt<0>();   // the first tiles
  }
  __syncthreads();

  // Per-lane LDS read bases of the K and V^T operands (the addressing is
  // described at their reads).  kHold: computed once and held across the
  // tile loop; at D = 512 they are recomputed from the lane index each tile.
  const uint32_t kaddr_h = static_cast<uint32_t>((lane & 31) * D * 2 + dlo * 2 + (((lane >> 5) ^ swz<D>(lane & 31)) << 4));
  const uint32_t vb0_h = static_cast<uint32_t>((4 * (lane >> 5) + ((lane & 15) >> 2)) * D * 2 +
      (((2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ swz<D>(4 * (lane >> 5) + ((lane & 15) >> 2))) << 4)) +
      static_cast<uint32_t>(dlo * 2 + (lane & 1) * 8);
  int32_t it = 0;
  // One tile: compute from ring slot B while the copies for slot
  // (B + kAhead) % kBufs are issued.
  auto step = [&](auto B, auto TRACK) {
    constexpr int kB = decltype(B)::value;
    constexpr bool kTrack = decltype(TRACK)::value;   // running maximum (else the cap)
    const int32_t kt = tile_key(it);
    if (it + kAhead < n_tiles) issue(tile_key(it + kAhead), std::integral_constant<int, (kB + kAhead) % kBufs>{});
    const uint16_t* kb = kslot(B);
    const uint16_t* vb = vslot(B);

    // Does this wave see any key of the tile?  (wave-uniform; equal for both
    // waves of a D-split pair)
    const bool need = w_lo <= w_hi && kt <= w_hi && kt + kKeys - 1 >= max(r_lo, W > 0 ? w_lo - W + 1 : 0);
    const bool full = kt >= r_lo && kt + kKeys - 1 <= w_lo && (W == 0 || kt >= w_hi - W + 1);

    // V^T operand addressing (used after the softmax; set up here so that the
    // first operand can be read while the softmax runs).  Lane (lgrp, li16)
    // reads chunk dlo/8 + 4*db + 2*(lgrp&1) + (li16&3)/2 of rows r0 and
    // r0 + 8; as for K, the chunk bits are clear of the row, slice and
    // half-chunk bits, so block db's address is one XOR: base ^ (64 * db).
    const int32_t ln = lane_id_here();
    const int32_t lgrp = ln >> 4;
    const int32_t li16 = ln & 15;
    const int32_t cl = 2 * (lgrp & 1) + ((li16 & 3) >> 1);
    const char* vbc = reinterpret_cast<const char*>(vb);
    const uint32_t rest = static_cast<uint32_t>(dlo * 2 + (li16 & 1) * 8);
    // Rows r0 = 16*t + rb and r0 + 8 of half t, rb = 4*(ln>>5) + (li16>>2).
    // The swizzle reads only row bits 0-3 and t moves bit 4, so one
    // per-lane base serves both halves (half t is the immediate offset t *
    // 16 rows).  Row r0 + 8 differs from r0 in swizzle bit 1 alone (rb's
    // bits 2-3 are 0 or 1, and 8 adds 2 to them), and the row, chunk and
    // slice fields of the base do not overlap, so its address is the base
    // XOR 32 plus the immediate offset 8 rows.
    const int32_t rb = 4 * (ln >> 5) + (li16 >> 2);
    const uint32_t vb0 = kHold ? vb0_h : static_cast<uint32_t>(rb * D * 2 + ((cl ^ swz<D>(rb)) << 4)) + rest;
    auto vread = [&](int v) -> bf16x8 {
      const int t = v / kDB;
      const int db = v % kDB;
      // as for K: bit 8 of the base is clear from D = 256 up, so db's top
      // bit is an offset addition (at D = 64, db < 2 never reaches it)
      const uint32_t x = static_cast<uint32_t>((db & 3) * 64);
      const int32_t imm = t * 16 * D * 2 + (db >> 2) * 256;
      const i16x4 a0 = lds_read_tr16(vbc + (vb0 ^ x) + imm);
      const i16x4 a1 = lds_read_tr16(vbc + (vb0 ^ (x ^ 32u)) + imm + 8 * D * 2);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int kV = 2 * kDB;
    constexpr int kLV = 3;
    bf16x8 va[kLV];

    // S^T = K . Q^T (partial over this wave's D slice when split).  Lane
    // (jj, hh) reads chunk dlo/8 + 2*ds + hh of key row jj.  The chunk's bits
    // (ds, hh, swizzle) sit in address bits 4-8, clear of the row and slice
    // bits, so the address of step ds is one XOR: kaddr ^ (32 * ds).
    f32x16 sacc = f32x16{};
    if (need) {
      const int32_t ln = lane_id_here();
      const int32_t jj = ln & 31;
      const int32_t hh = ln >> 5;
      const uint32_t kaddr = kHold ? kaddr_h : static_cast<uint32_t>(jj * D * 2 + dlo * 2 + ((hh ^ swz<D>(jj)) << 4));
      const char* kbc = reinterpret_cast<const char*>(kb);
      // kLA operand reads in flight ahead of the matrix instruction that
      // consumes them (fenced, so the order holds): the LDS latency is several
      // matrix instructions long.
      constexpr int kLA = kDS < 4 ? kDS : 4;
      bf16x8 a[kLA];
      // From D = 256 up the row pitch is a multiple of 512 bytes and the chunk
      // bits are 4-7 (plus the slice's bit 9 at D = 512), so bit 8 of kaddr is
      // clear and the step's top bit is an addition, folded into the
      // instruction's offset.  At D = 64 the steps never reach bit 8.
      auto kread = [&](int ds) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(kbc + (kaddr ^ static_cast<uint32_t>((ds & 7) * 32)) + (ds >> 3) * 256);
      };
#pragma unroll
      for (int ds = 0; ds < kLA; ++ds) a[ds] = kread(ds);
      if constexpr (kMatPrio > 0) __builtin_amdgcn_s_setprio(kMatPrio);
#pragma unroll
      for (int ds = 0; ds < kDS; ++ds) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ds % kLA], qf[ds], sacc, 0, 0, 0);
        if (ds + kLA < kDS) a[ds % kLA] = kread(ds + kLA);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (kMatPrio > 0) __builtin_amdgcn_s_setprio(0);
      // The first value operand is read now, so that its LDS latency passes
      // under the softmax instead of stalling the first PV product
      // (measured: global layers 0.6-1.9% faster, windows unchanged).
      va[0] = vread(0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kSplit > 1) {
      // [wave][r/4][lane] float4 layout: consecutive lanes, consecutive 16 bytes.
      const int32_t ln = lane_id_here();
      f32x4* mine = reinterpret_cast<f32x4*>(sx_lds) + wave * 256 + ln;
      const f32x4* other = reinterpret_cast<const f32x4*>(sx_lds) + (wave ^ 1) * 256 + ln;
#pragma unroll
      for (int r = 0; r < 16; r += 4) mine[(r / 4) * 64] = f32x4{sacc[r], sacc[r + 1], sacc[r + 2], sacc[r + 3]};
      lds_barrier();   // the copies issued for later tiles stay in flight
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
      // Lane holds keys kt + (r/4)*8 + h*4 + r%4.  Each score is kept in the
      // form that needs the fewest instructions per element:
      //  * with a cap, x = 1/(exp(2*s*scale/cap) + 1): the capped logit
      //    cap*tanh(s*scale/cap) is cap*(1 - 2x) (log2 units below), which
      //    falls as x rises, so the row max comes from the smallest x and a
      //    masked key gets x = +inf;
      //  * without a cap, x = s and the scale folds into the exponent,
      //    exp2(s*scale*log2e - m); a masked key gets -inf.
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (CAP) x[r] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(sacc[r] * p.cap_in2) + 1.f);
        else x[r] = sacc[r];
      }
      if (__builtin_expect(!full, 0)) {
        // boundary tile: allowed iff key_lo <= key <= pos
        const int32_t kb0 = kt + h * 4;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t key = kb0 + (r >> 2) * 8 + (r & 3);
          const bool ok = (key <= pos_m) & (key >= key_lo);
          x[r] = ok ? x[r] : (CAP ? INFINITY : -INFINITY);
        }
      }
      float m_use = m_fix;
      if constexpr (kTrack) {
        float mx;
        if (CAP) {
          float mr = x[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mr = fminf(mr, x[r]);
          mr = xhalf_min(mr);
          mx = fmaf(-2.f * p.cap_log2, mr, p.cap_log2);     // -inf when every key is masked
        } else {
          mx = x[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
          mx = xhalf_max(mx) * p.scale_log2;
        }
        // The running max only moves when the tile exceeds it by more than
        // kTau (log2 units): probabilities then stay <= 2^kTau and the output
        // rescale, a pass over every accumulator, is rare.
        const bool grow = mx > m_run + kTau;
        const float m_next = grow ? mx : m_run;
        m_use = m_next == -INFINITY ? 0.f : m_next;
        if (__builtin_amdgcn_ballot_w64(grow && m_run != -INFINITY) != 0) {
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < kDB; ++db) o[db] *= alpha;
        }
        m_run = m_next;
      }

      // Probabilities rounded to bf16; the row sum adds the same rounded
      // values (v_dot2_f32_bf16 against (1, 1)), in key order.
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
      for (int r = 0; r < 4; ++r) prob_pair(r);   // keys 0-15: the first half's operand

      // O^T += V^T . P^T, two 16-key halves per tile (product v: half
      // v / kDB, 32-row block v % kDB).  The operands of kLV products are
      // read ahead (fenced; the first one before the softmax), and the
      // second half's probabilities are computed during the first half's
      // products.
#pragma unroll
      for (int v = 1; v < kLV; ++v) va[v] = vread(v);
      if constexpr (kMatPrio > 0) __builtin_amdgcn_s_setprio(kMatPrio);
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
      if constexpr (kMatPrio > 0) __builtin_amdgcn_s_setprio(0);
    }
    // The next tile's copies must have landed before anyone reads them; the
    // copies of the tile after it may stay in flight.
    if (kAhead > 1 && it + 2 < n_tiles) wait_vmcnt<(kAhead > 1 ? kLoadsPerTile : 0)>(); else wait_vmcnt<0>();
    lds_barrier();
    ++it;
  };
  auto run_tiles = [&](auto TRACK) {
    while (it < n_tiles) {
      step(I0{}, TRACK);
      if (it >= n_tiles) break;
      step(I1{}, TRACK);
      if constexpr (kBufs > 2) {
        if (it >= n_tiles) break;
        step(I2{}, TRACK);
      }
    }
  };
  if (!fixed) {
    run_tiles(std::true_type{});
  } else if constexpr (kFixedMax) {
    run_tiles(std::false_type{});
    // A kept row always sees its own key, so its sum holds 2^(max logit -
    // cap) or more; below 2^-100 every logit of the row is within about 28
    // (log2 units) of -cap, where the terms near the bottom of the fp32 and
    // bf16 range would lose precision or flush to zero.  Then the whole
    // workgroup (it shares the K/V tiles) recomputes with a running maximum.
    // The decision goes through the idle ring: every copy has landed and
    // every wave has passed the last tile's barrier.
    const float l_chk = xhalf_sum(l_run);
    const bool low = kept && !(l_chk >= 0x1p-100f);
    uint32_t* flag = reinterpret_cast<uint32_t*>(k_lds0);
    const bool wave_low = __builtin_amdgcn_ballot_w64(low) != 0;
    if (lane == 0) flag[wave] = wave_low ? 1u : 0u;
    __syncthreads();
    uint32_t any_low = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any_low |= flag[w];
    __syncthreads();   // every wave has read the flags before the ring is written again
    if (any_low != 0) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) o[db] = f32x16{};
      l_run = 0.f;
      m_run = -INFINITY;
      tracked = true;
      it = 0;
      if (0 < n_tiles) issue(tile_key(0), I0{});
      if (kAhead > 1 && 1 < n_tiles) issue(tile_key(1), I1{});
      wait_vmcnt<0>();
      __syncthreads();
      run_tiles(std::true_type{});
    }
  }

  const float l_tot = xhalf_sum(l_run);
  // Padded rows are written as exact zeros (their accumulators are not
  // meaningful: a padded query row may hold anything).
  const bool live = kept && l_tot > 0.f;
  const float inv = live ? 1.f / l_tot : 0.f;
  auto out_pair = [&](int db, int a) -> u32x2 {
    u32x2 w2;
    w2[0] = pack_bf16x2(o[db][4 * a] * inv, o[db][4 * a + 1] * inv);
    w2[1] = pack_bf16x2(o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
    return kept ? w2 : u32x2{0u, 0u};
  };
  if constexpr (kStageO) {
    // The accumulators hold O^T: a lane owns one column and 8-byte pieces of
    // its row, so stores straight from them would write 16 bytes into each
    // of 32 rows per instruction.  Instead each wave parks its slice (or half
    // of it per pass) in its own region of the now idle ring, then reads it
    // back in row order and writes whole 16-byte chunks: one instruction
    // covers 1 KB of rows.
    wait_vmcnt<0>();
    __syncthreads();                 // every wave is done with the ring
    char* st = reinterpret_cast<char*>(stage_region(wave / kSlicePer)) + (wave % kSlicePer) * kSlice;
    constexpr int kRowCh = kDW / 8 / kPasses;   // 16-byte chunks per staged row
    constexpr int kSwz = (kRowCh < 16 ? kRowCh : 16) - 1;
    constexpr int kPassDB = kDB / kPasses;
    const int32_t ln = lane_id_here();
#pragma unroll
    for (int hp = 0; hp < kPasses; ++hp) {
#pragma unroll
      for (int db = 0; db < kPassDB; ++db) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int32_t ch = (db * 4 + a) ^ (j & kSwz);
          *reinterpret_cast<u32x2*>(st + j * (kRowCh * 16) + ch * 16 + h * 8) = out_pair(hp * kPassDB + db, a);
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kCols * kRowCh / 64; ++i) {
        const int32_t q = i * 64 + ln;
        const int32_t col = q / kRowCh;
        const int32_t dc = q % kRowCh;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(st + col * (kRowCh * 16) + ((dc ^ (col & kSwz)) * 16));
        const int32_t cc = cw * kCols + col;
        const int32_t cpos = p0 + cc / G;
        if (cpos < S) {
          uint16_t* dst = p.out + ((static_cast<int64_t>(b) * S + cpos) * p.hq + kvh * G + cc % G) * D + dlo +
                          hp * (kDW / kPasses) + dc * 8;
          *reinterpret_cast<bf16x8*>(dst) = v;
        }
      }
      if (kPasses > 1) __syncthreads();   // the next pass rewrites the region
    }
  } else if (col_valid) {
    uint16_t* orow = p.out + ((static_cast<int64_t>(b) * S + pos) * p.hq + head) * D + dlo;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) *reinterpret_cast<u32x2*>(orow + db * 32 + a * 8 + h * 4) = out_pair(db, a);
    }
  }
  if (col_valid && p.lse && h == 0 && dlo == 0) {
    // With the fixed (integer) maximum, m + log2(l) is formed as the integer
    // m + exponent(l) plus log2 of l's mantissa, which keeps the precision a
    // large offset would cost.
    float lse2;
    if (!tracked) {
      const int32_t e = __builtin_amdgcn_frexp_expf(l_tot);     // l_tot = mant * 2^e, mant in [0.5, 1)
      lse2 = static_cast<float>(static_cast<int32_t>(m_fix) + e) + __log2f(__builtin_amdgcn_frexp_mantf(l_tot));
    } else {
      lse2 = m_run + __log2f(l_tot);
    }
    p.lse[(static_cast<int64_t>(b) * p.hq + head) * S + pos] = live ? lse2 * kLn2 : -INFINITY;
  }
}

template <int D, int G, bool KEQV, bool CAP, bool WIDE = false, bool QROPE = false>
hipError_t launch_t(const PrefillArgs& a, const PrefillParams& prm, hipStream_t stream) {
  constexpr int kP = positions_per_block<D, G, KEQV, WIDE>();
  PrefillParams pp = prm;
  pp.n_qblocks = (a.seq + kP - 1) / kP;
  const int32_t npairs = a.batch * a.hkv;
  const int32_t nx = 1 << pp.xcd_log2;
  int32_t pad = pp.n_qblocks;
  if ((npairs & (nx - 1)) != 0 && (nx % npairs) == 0) {
    const int32_t k = nx / npairs;
    pad = (pp.n_qblocks + k - 1) / k * k;
  }
  pp.n_qblocks_pad = pad;
  // Contiguous runs only where every block does about the same work: the
  // lighter blocks before the first full window are at most 1/8 of the rows.
  pp.xcd_runs = a.window > 0 && static_cast<int64_t>(a.window) * 8 <= a.seq;
  const int64_t blocks = static_cast<int64_t>(npairs) * pad;
  if (blocks > 0x7fffffff) return hipErrorNotSupported;
  return launch_kernel(prefill_kernel<D, G, KEQV, CAP, WIDE, QROPE>, dim3(static_cast<uint32_t>(blocks)),
                       dim3(pf_waves<D, KEQV, WIDE>() * 64), stream, pp);
}

template <int D, int G>
hipError_t dispatch_flags(const PrefillArgs& a, const PrefillParams& prm, hipStream_t s) {
  const bool cap = a.softcap > 0.0;
  if (a.q_rope) {
    // The fused query rotary: width 256, keys and values separate.
    if constexpr (D == 256) {
      if (a.k_eq_v) return hipErrorNotSupported;
      const bool global = a.window <= 0 || a.window >= a.seq;
      if (cap && global) return launch_t<D, G, false, true, true, true>(a, prm, s);
      return cap ? launch_t<D, G, false, true, false, true>(a, prm, s) : launch_t<D, G, false, false, false, true>(a, prm, s);
    }
    return hipErrorNotSupported;
  }
  if (a.k_eq_v) return cap ? launch_t<D, G, true, true>(a, prm, s) : launch_t<D, G, true, false>(a, prm, s);
  if constexpr (D == 256) {
    const bool global = a.window <= 0 || a.window >= a.seq;
    if (cap && global) return launch_t<D, G, false, true, true>(a, prm, s);
  }
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
    default: return hipErrorNotSupported;
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
  prm.seq_start = a.seq_start;
  prm.seq_end = a.seq_end;
  prm.seq = a.seq;
  prm.hq = a.hq;
  prm.hkv = a.hkv;
  prm.window = a.window;
  prm.batch = a.batch;
  prm.n_qblocks = 0;
  prm.n_qblocks_pad = 0;
  prm.xcd_runs = 0;
  // XCD-aware block order needs a power-of-two XCD count; otherwise plain order.
  prm.xcd_log2 = 0;
  if (a.xcds > 1 && (a.xcds & (a.xcds - 1)) == 0)
    while ((1 << prm.xcd_log2) < a.xcds) ++prm.xcd_log2;
  const double log2e = 1.4426950408889634;
  prm.scale_log2 = static_cast<float>(a.scale * log2e);
  prm.cap_in2 = a.softcap > 0.0 ? static_cast<float>(2.0 * a.scale * log2e / a.softcap) : 0.f;
  prm.cap_log2 = static_cast<float>(a.softcap * log2e);
  prm.pos0 = a.pos0;
  prm.rot_w1 = a.q_rope ? rotary_w1(a.rope_theta, a.dim) : 0.0;
  prm.rot_c0 = a.q_rope ? rotary_c0(a.rope_pos_div) : 0.0;
  switch (a.dim) {
    case 64: return dispatch_group<64>(a, prm, stream);
    case 256: return dispatch_group<256>(a, prm, stream);
    case 512: return dispatch_group<512>(a, prm, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace ga
