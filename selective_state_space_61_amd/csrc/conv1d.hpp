// conv1d.hpp -- the depthwise causal convolution that feeds the scan, and its one-token form,
// for gfx950.
//
// "Mamba 论文精读" sec. 3.4 (MambaBlock listing): a Conv1d with one group per channel, kernel
// width K and K-1 zeros of padding, cut back to the first L outputs, then SiLU.  As a
// cross-correlation, for channel d of batch row b:
//   y[t] = bias[d] + sum_k w[d,k] * xin[t-(K-1)+k],  xin[s] = x[s] (s >= 0) or the initial
//   state (s < 0, zeros without one);  out = silu(y) when asked.
// The final state is the last K-1 inputs, oldest first, in x's storage type: the input of the
// next call, or of the one-token update.
//
// Both kernels stream: every input element is read once (plus a K-1 row halo per time tile,
// which the L2 serves) and every output written once (non-temporally), so HBM bandwidth is the
// bound.  A thread owns VEC consecutive channels, one kConvVecBytes-byte (4-byte) access per
// row, and kConvTile consecutive steps; it keeps the K-1 previous inputs in registers and issues
// kConvUnroll row loads before using any of them.
#pragma once

#include "ssm_device.hpp"

namespace ssm {

struct ConvArgs {
  const void* x;        // (batch, seqlen, dim)
  const float* weight;  // (dim, K)
  const float* bias;    // (dim) or NULL
  const void* init;     // (batch, dim, K-1) or NULL
  void* y;              // (batch, seqlen, dim)
  void* final_state;    // (batch, dim, K-1) or NULL
  int64_t batch;
  int64_t seqlen;
  int64_t dim;
  int64_t ncv;     // channel vectors per row: ceil(dim / VEC)
  int64_t ntiles;  // time tiles per batch row (at least 1)
  int32_t silu;
  int32_t vec_ok;  // x / y rows allow the aligned kConvVecBytes-byte access
};

struct ConvUpdateArgs {
  void* state;          // (batch, dim, K-1), updated in place
  const void* x;        // (batch, dim)
  const float* weight;  // (dim, K)
  const float* bias;    // (dim) or NULL
  void* y;              // (batch, dim)
  int64_t batch;
  int64_t dim;
  int32_t silu;
};

constexpr int kConvVecBytes = 4;  // bytes of one thread's channel vector per row
template <bool BF16>
constexpr int kConvVec = kConvVecBytes / (BF16 ? 2 : 4);
constexpr int kConvTile = 32;
constexpr int kConvThreads = 256;
constexpr int kConvUnroll = 16;
static_assert(kConvTile % kConvUnroll == 0, "whole row groups per tile");

template <bool BF16>
__device__ __forceinline__ float load_one(const void* base, int64_t i) {
  if constexpr (BF16) return bf16_lo(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_one(void* base, int64_t i, float v) {
  if constexpr (BF16) static_cast<uint16_t*>(base)[i] = to_bf16(v);
  else static_cast<float*>(base)[i] = v;
}

// One thread's output vector of a row (kConvVecBytes, aligned), stored non-temporally: the
// output is written once and read by the next kernel, not by this one, so it need not displace
// the x rows that the neighbouring time tile still reads as its halo.
template <bool BF16>
__device__ __forceinline__ void store_row_stream(void* base, int64_t idx, const float (&val)[kConvVec<BF16>]) {
  static_assert(kConvVecBytes == 4, "one 32-bit word per thread and row");
  uint32_t word;
  if constexpr (BF16) word = pack_bf16x2(val[0], val[1]);
  else word = __builtin_bit_cast(uint32_t, val[0]);
  __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(static_cast<char*>(base) + idx * (BF16 ? 2 : 4)));
}

template <bool BF16, int K, bool FAST>
__device__ __forceinline__ void conv_tile(const ConvArgs& p, int64_t b, int64_t d0, int nv, int64_t t0, int64_t t1) {
  // FAST: all VEC channels valid, rows allow the aligned vector access, and the tile is whole
  // (no checks)
  constexpr int VEC = kConvVec<BF16>;
  constexpr int W = K > 1 ? K - 1 : 1;  // window slots (unused when K == 1)
  const bool vec = FAST || (p.vec_ok != 0 && nv == VEC);
  float w[K][VEC], bias[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const bool ok = FAST || v < nv;
#pragma unroll
    for (int k = 0; k < K; ++k) w[k][v] = ok ? p.weight[(d0 + v) * K + k] : 0.0f;
    bias[v] = (ok && p.bias) ? p.bias[d0 + v] : 0.0f;
  }
  // win[j] = input at step t - (K-1) + j for the next step t to produce
  float win[W][VEC];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t s = t0 - (K - 1) + j;
    if (s >= 0) {
      RawVec<BF16, VEC> r;
      r.load(p.x, (b * p.seqlen + s) * p.dim + d0, FAST ? VEC : nv, vec);
#pragma unroll
      for (int v = 0; v < VEC; ++v) win[j][v] = r.get(v);
    } else {
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        win[j][v] = (p.init && (FAST || v < nv))
                        ? load_one<BF16>(p.init, (b * p.dim + d0 + v) * (K - 1) + (K - 1) + s) : 0.0f;
    }
  }
  for (int64_t tb = t0; tb < t1; tb += kConvUnroll) {
    RawVec<BF16, VEC> r[kConvUnroll];
#pragma unroll
    for (int u = 0; u < kConvUnroll; ++u) {
      const int64_t t = tb + u;
      if (FAST || t < t1) r[u].load(p.x, (b * p.seqlen + t) * p.dim + d0, FAST ? VEC : nv, vec);
    }
#pragma unroll
    for (int u = 0; u < kConvUnroll; ++u) {
      const int64_t t = tb + u;
      if (!FAST && t >= t1) break;
      float out[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float xv = r[u].get(v);
        float acc = bias[v];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) acc = fmaf(w[j][v], win[j][v], acc);
        acc = fmaf(w[K - 1][v], xv, acc);
        out[v] = p.silu ? silu_f32(acc) : acc;
#pragma unroll
        for (int j = 0; j + 1 < K - 1; ++j) win[j][v] = win[j + 1][v];
        if constexpr (K > 1) win[K - 2][v] = xv;
      }
      if constexpr (FAST) store_row_stream<BF16>(p.y, (b * p.seqlen + t) * p.dim + d0, out);
      else store_vec<BF16, VEC>(p.y, (b * p.seqlen + t) * p.dim + d0, out, nv, vec);
    }
  }
  // the tile that holds the last step leaves the last K-1 inputs behind
  if (p.final_state && t1 == p.seqlen) {
#pragma unroll
    for (int j = 0; j < K - 1; ++j)
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        if (FAST || v < nv) store_one<BF16>(p.final_state, (b * p.dim + d0 + v) * (K - 1) + j, win[j][v]);
  }
}

template <bool BF16, int K>
__global__ __launch_bounds__(kConvThreads) void causal_conv1d_kernel(const ConvArgs p) {
  constexpr int VEC = kConvVec<BF16>;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x;
  if (gid >= p.ncv * p.ntiles * p.batch) return;
  // consecutive threads take consecutive channel vectors of one row: coalesced rows
  const int64_t cv = gid % p.ncv;
  const int64_t rest = gid / p.ncv;
  const int64_t tile = rest % p.ntiles;
  const int64_t b = rest / p.ntiles;
  const int64_t d0 = cv * VEC;
  const int nv = static_cast<int>((p.dim - d0) < VEC ? (p.dim - d0) : VEC);
  const int64_t t0 = tile * kConvTile;
  const int64_t t1 = (t0 + kConvTile < p.seqlen) ? (t0 + kConvTile) : p.seqlen;
  if (p.vec_ok && nv == VEC && t1 - t0 == kConvTile) conv_tile<BF16, K, true>(p, b, d0, nv, t0, t1);
  else conv_tile<BF16, K, false>(p, b, d0, nv, t0, t1);
}

// One token: one thread per (batch row, channel).  The window is the K-1 stored inputs followed
// by x; the state then drops its oldest input and appends x.
template <bool BF16, int K>
__global__ __launch_bounds__(kConvThreads) void conv1d_update_kernel(const ConvUpdateArgs p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x;
  if (i >= p.batch * p.dim) return;
  const int64_t d = i % p.dim;
  const float xv = load_one<BF16>(p.x, i);
  float st[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) st[j] = load_one<BF16>(p.state, i * (K - 1) + j);
  float acc = p.bias ? p.bias[d] : 0.0f;
#pragma unroll
  for (int j = 0; j < K - 1; ++j) acc = fmaf(p.weight[d * K + j], st[j], acc);
  acc = fmaf(p.weight[d * K + K - 1], xv, acc);
  store_one<BF16>(p.y, i, p.silu ? silu_f32(acc) : acc);
#pragma unroll
  for (int j = 0; j + 1 < K - 1; ++j) store_one<BF16>(p.state, i * (K - 1) + j, st[j + 1]);
  if constexpr (K > 1) store_one<BF16>(p.state, i * (K - 1) + K - 2, xv);
}

}  // namespace ssm
