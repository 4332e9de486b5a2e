// scan_time.hpp -- the selective scan with time parallel inside a chunk: a wave64 associative
// scan over (a, b) pairs, for few channels and long sequences (gfx950).
//
// The recurrence h_t = abar_t h_{t-1} + u_t ("Mamba 论文精读" sec. 2.2 and 3.3) composes with the
// associative operator (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) ("mamba->jamba" sec. 2.3,
// parallel scan).  One workgroup per (batch row, channel), four waves of four state chains each
// (N = 16).  The sequence runs in chunks of 64 K steps; lane l of a wave owns steps
// l K .. l K + K - 1 of the chunk:
//   1. each lane runs its K steps from a zero state, keeping abar_t and u_t = B_t dt_t x_t in
//      VGPRs, and forms its block's pair (prod abar, h from zero);
//   2. an inclusive scan of the 64 pairs with DPP: row_shr 1, 2, 4, 8 inside each 16-lane row,
//      then row_bcast:15 and row_bcast:31 across rows; a lane without a source keeps the
//      identity (1, 0), which DPP leaves in place of the missing operand;
//   3. the state entering lane l's block is the pair of lanes 0 .. l-1 applied to the carry of
//      the chunk before (wave_shr:1 of the inclusive scan), and the carry of the next chunk is
//      lane 63's pair applied to it;
//   4. each lane reruns its K steps from its entering state with the stored abar_t, u_t and reads
//      out its four states' share of y_t into LDS; after a barrier the 256 threads add the four
//      waves' shares, D x and the gate, and store y.
// Every step costs the sequential recurrence's work plus a scan level per pair and an extra FMA
// to rerun the block; rows past the sequence carry dt = 0, B = 0, C = 0 (identities).
#pragma once

#include "scan_fwd.hpp"

namespace ssm {

constexpr int kTimeWaves = 4;

// DPP controls (GFX9 encoding)
constexpr int kDppRowShr = 0x110;     // + shift 1..15
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
constexpr int kDppWaveShr1 = 0x138;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or(float identity, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, identity),
                                                               __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                                               false));
}

// one level of the inclusive scan: the pair of the lane CTRL names (identity where there is
// none) composed before this lane's pair
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void scan_level(float& P, float& hl) {
  const float Pp = dpp_or<CTRL, ROW_MASK>(1.0f, P);
  const float hp = dpp_or<CTRL, ROW_MASK>(0.0f, hl);
  hl = fmaf(P, hp, hl);
  P = P * Pp;
}

template <bool BF16, int K>
__global__ __launch_bounds__(64 * kTimeWaves) void scan_time_kernel(const ScanArgs p) {
  constexpr int N = 16, NPL = 4, CH = 64 * K;
  __shared__ float s_yp[kTimeWaves][CH];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t bd = blockIdx.x;
  const int64_t b = bd / p.dim, d = bd % p.dim;
  const int64_t L = p.seqlen;
  const int64_t row_base = b * L;
  const int n0 = NPL * wave;
  float A2[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) A2[j] = fmaxf(p.A[d * N + n0 + j] * kLog2e, -3.0e38f);
  const float bias = p.delta_bias ? p.delta_bias[d] : 0.0f;
  const float dsk = p.Dskip ? p.Dskip[d] : 0.0f;
  auto elem = [&](const void* base, int64_t i) -> float {
    if constexpr (BF16) return bf16_lo(static_cast<const uint16_t*>(base)[i]);
    else return static_cast<const float*>(base)[i];
  };
  float carry[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) carry[j] = 0.0f;
  const int64_t nchunks = (L + CH - 1) / CH;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t tb = c * CH + static_cast<int64_t>(lane) * K;
    float a[K][NPL], u[K][NPL], cv[K][NPL];
    float P[NPL], hl[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      P[j] = 1.0f;
      hl[j] = 0.0f;
    }
    // 1. the lane's block from a zero state
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int64_t t = tb + i;
      const bool ok = t < L;
      float dt = 0.0f, w = 0.0f;
      BcRow<BF16, NPL> rb, rc;
      const int64_t e = (row_base + t) * N + n0;
      rb.load(p.B, e, ok);
      rc.load(p.C, e, ok);
      if (ok) {
        const int64_t itd = (row_base + t) * p.dim + d;
        const float v = elem(p.delta, itd) + bias;
        dt = p.softplus ? softplus_f32(v) : v;
        w = dt * elem(p.x, itd);
      }
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        a[i][j] = hw_exp2(dt * A2[j]);
        u[i][j] = rb.get(j) * w;
        cv[i][j] = rc.get(j);
        hl[j] = fmaf(a[i][j], hl[j], u[i][j]);
        P[j] = P[j] * a[i][j];
      }
    }
    // 2. inclusive scan of the lanes' pairs
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      scan_level<kDppRowShr + 1, 0xF>(P[j], hl[j]);
      scan_level<kDppRowShr + 2, 0xF>(P[j], hl[j]);
      scan_level<kDppRowShr + 4, 0xF>(P[j], hl[j]);
      scan_level<kDppRowShr + 8, 0xF>(P[j], hl[j]);
      scan_level<kDppRowBcast15, 0xA>(P[j], hl[j]);
      scan_level<kDppRowBcast31, 0xC>(P[j], hl[j]);
    }
    // 3. entering states and the next carry
    float h[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const float Pe = dpp_or<kDppWaveShr1, 0xF>(1.0f, P[j]);
      const float he = dpp_or<kDppWaveShr1, 0xF>(0.0f, hl[j]);
      h[j] = fmaf(Pe, carry[j], he);
      const float P63 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, P[j]), 63));
      const float h63 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hl[j]), 63));
      carry[j] = fmaf(P63, carry[j], h63);
    }
    // 4. rerun the block from its entering state, reading out this wave's share
#pragma unroll
    for (int i = 0; i < K; ++i) {
      float yp = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        h[j] = fmaf(a[i][j], h[j], u[i][j]);
        yp = fmaf(cv[i][j], h[j], yp);
      }
      s_yp[wave][lane * K + i] = yp;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < CH; e += 64 * kTimeWaves) {
      const int64_t t = c * CH + e;
      if (t >= L) break;
      const int64_t itd = (row_base + t) * p.dim + d;
      float y = ((s_yp[0][e] + s_yp[1][e]) + s_yp[2][e]) + s_yp[3][e];
      y = fmaf(dsk, elem(p.x, itd), y);
      if (p.z) y *= silu_f32(elem(p.z, itd));
      if constexpr (BF16) static_cast<uint16_t*>(p.y)[itd] = to_bf16(y);
      else static_cast<float*>(p.y)[itd] = y;
    }
    __syncthreads();
  }
  if (p.last_state && lane == 0) {
    float* dst = p.last_state + (b * p.dim + d) * N + n0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) dst[j] = carry[j];
  }
}

}  // namespace ssm
