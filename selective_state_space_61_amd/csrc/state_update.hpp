// state_update.hpp -- single-token decode step of the selective SSM for gfx950.
//
// One step of the recurrence ("Mamba 论文精读" sec. 2.2; sec. 6: O(1) work per token with a
// fixed-size state and no cache of past inputs):
//   dt = softplus(delta + bias) (or delta + bias);  h[n] = exp(dt A[n]) h[n] + dt B[n] x;
//   y = sum_n C[n] h[n] + D x;  y *= silu(z).
//
// The state (batch, dim, N) fp32 is read and written once per step: that traffic is the whole
// cost, so the kernel is a streaming one.  A thread owns SPT = min(N, 4) consecutive states of
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
};

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
  if constexpr (BF16) return bf16_lo(static_cast<const uint16_t*>(base)[idx]);
  else return static_cast<const float*>(base)[idx];
}

template <bool BF16, int N>
__global__ __launch_bounds__(256) void state_update_kernel(const UpdateArgs p) {
  constexpr int SPT = N < 4 ? N : 4;
  constexpr int TPC = N / SPT;
  static_assert(TPC <= 64 && (64 % TPC) == 0, "a channel's lanes must share one wave");
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t ch = gid / TPC;
  const int sub = static_cast<int>(gid % TPC);
  const bool ok = ch < p.batch * p.dim;

  float yp = 0.0f;
  float xv = 0.0f, zv = 0.0f;
  if (ok) {
    const int64_t b = ch / p.dim;
    const int64_t d = ch % p.dim;
    const int n0 = sub * SPT;
    xv = load_elem<BF16>(p.x, ch);
    const float vb = load_elem<BF16>(p.delta, ch) + (p.delta_bias ? p.delta_bias[d] : 0.0f);
    const float dt = p.softplus ? softplus_f32(vb) : vb;
    const float w = dt * xv;
    if (p.z) zv = load_elem<BF16>(p.z, ch);

    float hs[SPT];
    float* st = p.state + ch * N + n0;
    if constexpr (SPT == 4) {
      if (p.state_vec_ok) {
        const float4 v = *reinterpret_cast<const float4*>(st);
        hs[0] = v.x; hs[1] = v.y; hs[2] = v.z; hs[3] = v.w;
      } else {
#pragma unroll
        for (int j = 0; j < SPT; ++j) hs[j] = st[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < SPT; ++j) hs[j] = st[j];
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const float a = hw_exp2(dt * (p.A[d * N + n0 + j] * kLog2e));
      const float bv = load_elem<BF16>(p.B, b * N + n0 + j);
      const float cv = load_elem<BF16>(p.C, b * N + n0 + j);
      hs[j] = fmaf(a, hs[j], w * bv);
      yp = fmaf(cv, hs[j], yp);
    }
    if constexpr (SPT == 4) {
      if (p.state_vec_ok) {
        *reinterpret_cast<float4*>(st) = make_float4(hs[0], hs[1], hs[2], hs[3]);
      } else {
#pragma unroll
        for (int j = 0; j < SPT; ++j) st[j] = hs[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < SPT; ++j) st[j] = hs[j];
    }
  }
  // combine the TPC partial read-outs of a channel (its lanes are adjacent in one wave)
#pragma unroll
  for (int off = 1; off < TPC; off <<= 1) yp += __shfl_xor(yp, off, 64);
  if (ok && sub == 0) {
    const int64_t d = ch % p.dim;
    float yv = fmaf(p.Dskip ? p.Dskip[d] : 0.0f, xv, yp);
    if (p.z) yv *= silu_f32(zv);
    if constexpr (BF16) static_cast<uint16_t*>(p.y)[ch] = to_bf16(yv);
    else static_cast<float*>(p.y)[ch] = yv;
  }
}

}  // namespace ssm
