// state_update.hpp -- single-token decode step of the selective SSM for gfx950.
//
// One step of the recurrence ("Mamba 论文精读" sec. 2.2; sec. 6: O(1) work per token with a
// fixed-size state and no cache of past inputs):
//   dt = softplus(delta + bias) (or delta + bias);  h[n] = exp(dt A[n]) h[n] + dt B[n] x;
//   y = sum_n C[n] h[n] + D x;  y *= silu(z).
//
// The state (batch, dim, N) fp32 is read and written once per step: that traffic is the whole
// cost, so the kernel is a streaming one, with non-temporal state accesses.  A thread owns SPT = min(N, 4) consecutive states of
// one channel (one 16-byte load and store), TPC = N / SPT neighbouring lanes share a channel
// and combine their partial read-outs with cross-lane adds.  The per-channel prologue (softplus)
// is recomputed by each of those lanes; it is cheap next to the state traffic.
#pragma once

#include "ssm_device.hpp"

namespace ssm {

struct UpdateArgs {
  float* state;
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* z;
  const float* delta_bias;
  void* y;
  int64_t batch;
  int64_t dim;
  int32_t softplus;
  int32_t state_vec_ok;  // state rows allow 16-byte access
  int32_t a_vec_ok;      // rows of A allow 16-byte access
};

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
  if constexpr (BF16) return bf16_lo(static_cast<const uint16_t*>(base)[idx]);
  else return static_cast<const float*>(base)[idx];
}

// Quads (SPT consecutive states of one channel) handled per thread: all their loads are issued
// before any arithmetic, so each wave keeps several 1 KB state reads in flight.
constexpr int kQuadsPerThread = 1;
constexpr int kUpdateThreads = 256;

// ZOH: exact zero-order-hold input term (zoh_factor) instead of Delta B
template <bool BF16, int N, bool ZOH = false>
__global__ __launch_bounds__(kUpdateThreads) void state_update_kernel(const UpdateArgs p) {
  constexpr int SPT = N < 4 ? N : 4;
  constexpr int TPC = N / SPT;
  constexpr int Q = kQuadsPerThread;
  static_assert(TPC <= 64 && (64 % TPC) == 0, "a channel's lanes must share one wave");
  const int64_t nquads = p.batch * p.dim * TPC;
  // quad of slice k: consecutive threads take consecutive quads (coalesced 16-byte accesses)
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kUpdateThreads * Q) + threadIdx.x;

  // optional tensors are read from an always-valid stand-in when absent and zeroed afterwards,
  // so that no load is behind a branch
  const void* zsrc = p.z ? p.z : p.x;
  const float* bsrc = p.delta_bias ? p.delta_bias : p.A;
  const float* dsrc = p.Dskip ? p.Dskip : p.A;
  const float bias_on = p.delta_bias ? 1.0f : 0.0f, d_on = p.Dskip ? 1.0f : 0.0f;

  float hs[Q][SPT], a2[Q][SPT], bv[Q][SPT], cv[Q][SPT];
  float xv[Q], dv[Q], zv[Q], bias[Q], dsk[Q];
  bool ok[Q];
  // 1. loads, all unconditional: a quad past the end reads channel 0 (always in bounds) and its
  //    results are never stored, so no load sits behind a branch and all stay in flight together
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const int64_t q = base + k * kUpdateThreads;
    ok[k] = q < nquads;
    const int64_t ch = ok[k] ? q / TPC : 0;
    const int n0 = static_cast<int>(q % TPC) * SPT;
    const int64_t b = ch / p.dim, d = ch % p.dim;
    const float* st = p.state + ch * N + n0;
    if constexpr (SPT == 4) {
      if (p.state_vec_ok) {
        const float4 v = load_stream(st);
        hs[k][0] = v.x; hs[k][1] = v.y; hs[k][2] = v.z; hs[k][3] = v.w;
      } else {
#pragma unroll
        for (int j = 0; j < SPT; ++j) hs[k][j] = st[j];
      }
      if (p.a_vec_ok) {
        const float4 av = *reinterpret_cast<const float4*>(p.A + d * N + n0);
        a2[k][0] = av.x; a2[k][1] = av.y; a2[k][2] = av.z; a2[k][3] = av.w;
      } else {
#pragma unroll
        for (int j = 0; j < SPT; ++j) a2[k][j] = p.A[d * N + n0 + j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        hs[k][j] = st[j];
        a2[k][j] = p.A[d * N + n0 + j];
      }
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      bv[k][j] = load_elem<BF16>(p.B, b * N + n0 + j);
      cv[k][j] = load_elem<BF16>(p.C, b * N + n0 + j);
    }
    xv[k] = load_elem<BF16>(p.x, ch);
    dv[k] = load_elem<BF16>(p.delta, ch);
    zv[k] = load_elem<BF16>(zsrc, ch);
    bias[k] = bias_on * bsrc[d];
    dsk[k] = d_on * dsrc[d];
  }
  // 2. arithmetic
  float yp[Q];
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const float vb = dv[k] + bias[k];
    const float dt = p.softplus ? softplus_f32(vb) : vb;
    const float w = dt * xv[k];
    yp[k] = 0.0f;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const float tt = dt * (a2[k][j] * kLog2e);
      const float a = hw_exp2(tt);
      const float u = ZOH ? (w * kLog2e) * zoh_factor(tt, a) * bv[k][j] : w * bv[k][j];
      hs[k][j] = fmaf(a, hs[k][j], u);
      yp[k] = fmaf(cv[k][j], hs[k][j], yp[k]);
    }
  }
  // 3. stores: the state, then y from the first lane of each channel after the cross-lane sum
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const int64_t q = base + k * kUpdateThreads;
    const int64_t ch = ok[k] ? q / TPC : 0;
    const int n0 = static_cast<int>(q % TPC) * SPT;
    float* st = p.state + ch * N + n0;
    if (ok[k]) {
      if constexpr (SPT == 4) {
        if (p.state_vec_ok) {
          store_stream(st, make_float4(hs[k][0], hs[k][1], hs[k][2], hs[k][3]));
        } else {
#pragma unroll
          for (int j = 0; j < SPT; ++j) st[j] = hs[k][j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < SPT; ++j) st[j] = hs[k][j];
      }
    }
    float y = yp[k];
#pragma unroll
    for (int off = 1; off < TPC; off <<= 1) y += __shfl_xor(y, off, 64);
    if (ok[k] && n0 == 0) {
      float yv = fmaf(dsk[k], xv[k], y);
      if (p.z) yv *= silu_f32(zv[k]);
      if constexpr (BF16) static_cast<uint16_t*>(p.y)[ch] = to_bf16(yv);
      else static_cast<float*>(p.y)[ch] = yv;
    }
  }
}

}  // namespace ssm
