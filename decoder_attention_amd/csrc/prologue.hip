// Fused QK-norm + dual-base partial rotary prologue (gfx950).
//
// One workgroup per token (b, s).  The token's rotary table cos/sin(p * w_i)
// is built once in LDS (angle formed and reduced modulo 2*pi in fp64, then
// fp32 sincos) and shared by every q and k head of that token.  Each head row
// of width D is handled by D/8 lanes holding 8 contiguous bf16 (one 16-byte
// load); the RMS reduction is a butterfly inside those lanes; the rotate-half
// partner element comes through an LDS copy of the normalised row.
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
constexpr double kTwoPi = 6.283185307179586476925286766559;

__global__ __launch_bounds__(kThreads) void qk_prologue_kernel(
    const uint16_t* q_in, const uint16_t* k_in,
    uint16_t* q_out, uint16_t* k_out,
    const float* __restrict__ qw, const float* __restrict__ kw,
    const int32_t* __restrict__ pos0, int32_t seq, int32_t hq, int32_t hkv, int32_t dim,
    int32_t rotary_dim, double theta, float eps, float offset) {
  __shared__ float2 cs_tab[256];
  __shared__ float rowbuf[kThreads * 8];

  const int64_t token = blockIdx.x;
  const int32_t b = static_cast<int32_t>(token / seq);
  const int32_t s = static_cast<int32_t>(token % seq);
  const int32_t tid = threadIdx.x;
  const int32_t half = rotary_dim >> 1;

  const int64_t pos = static_cast<int64_t>(pos0 ? pos0[b] : 0) + s;
  for (int32_t i = tid; i < half; i += kThreads) {
    const double w = pow(theta, -2.0 * i / rotary_dim);
    double ang = fmod(static_cast<double>(pos) * w, kTwoPi);
    if (ang < 0) ang += kTwoPi;
    float sn, cn;
    sincosf(static_cast<float>(ang), &sn, &cn);
    cs_tab[i] = make_float2(cn, sn);
  }
  __syncthreads();

  const int32_t tpr = dim >> 3;                 // lanes per row (power of two <= 64)
  const int32_t rows_per_pass = kThreads / tpr;
  const int32_t rows = hq + (k_in ? hkv : 0);
  const int32_t sub = tid / tpr;
  const int32_t lane = tid % tpr;
  const int32_t d0 = lane * 8;

  for (int32_t row0 = 0; row0 < rows; row0 += rows_per_pass) {
    const int32_t row = row0 + sub;
    const bool active = row < rows;
    const bool is_q = row < hq;
    const uint16_t* src = nullptr;
    uint16_t* dst = nullptr;
    const float* w = nullptr;
    if (active) {
      if (is_q) {
        const int64_t off = (token * hq + row) * dim + d0;
        src = q_in + off;
        dst = q_out + off;
        w = qw;
      } else {
        const int64_t off = (token * hkv + (row - hq)) * dim + d0;
        src = k_in + off;
        dst = k_out + off;
        w = kw;
      }
    }
    float x[8];
    if (active) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = lo_bf16(raw[e]);
        x[2 * e + 1] = hi_bf16(raw[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    // RMSNorm (only when this side has a weight); the flag is uniform per row.
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    for (int m = tpr >> 1; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (active && w) {
      const float inv = 1.0f / sqrtf(ss / static_cast<float>(dim) + eps);
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + d0);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + d0 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = x[e] * inv * (w0[e] + offset);
        x[e + 4] = x[e + 4] * inv * (w1[e] + offset);
      }
    }
    float* rb = rowbuf + sub * dim;
#pragma unroll
    for (int e = 0; e < 8; ++e) rb[d0 + e] = x[e];
    __syncthreads();
    if (active) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int32_t d = d0 + e;
        if (d < half) {
          const float2 c = cs_tab[d];
          y[e] = x[e] * c.x - rb[d + half] * c.y;
        } else if (d < rotary_dim) {
          const float2 c = cs_tab[d - half];
          y[e] = x[e] * c.x + rb[d - half] * c.y;
        } else {
          y[e] = x[e];
        }
      }
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
      *reinterpret_cast<u32x4*>(dst) = o;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_qk_prologue(const PrologueArgs& a, hipStream_t stream) {
  const int64_t tokens = static_cast<int64_t>(a.batch) * a.seq;
  if (tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(qk_prologue_kernel, dim3(static_cast<uint32_t>(tokens)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a.q_in), static_cast<const uint16_t*>(a.k_in),
                     static_cast<uint16_t*>(a.q_out), static_cast<uint16_t*>(a.k_out), a.q_norm_w, a.k_norm_w,
                     a.pos0, a.seq, a.hq, a.hkv, a.dim, a.rotary_dim, a.theta, a.eps, a.offset);
  return hipGetLastError();
}

}  // namespace ga
