// scan_bwd.hpp -- backward pass of the selective scan for gfx950, with recomputation.
//
// Gradients of sum(dy * y) for the forward of scan_fwd.hpp (zero initial state), by the adjoint
// recurrence.  For one channel with g_t = dL/dh_t:
//   dy0_t = dy_t silu(z_t);  dz_t = dy_t y0_t silu'(z_t)   (y0_t = C_t.h_t + D x_t)
//   g_t = dy0_t C_t + abar_{t+1} g_{t+1}
//   dC_t += dy0_t h_t;  dB_t += g_t dt_t x_t;  dx_t = dy0_t D + sum_n g_t dt_t B_t
//   ddt_t = sum_n g_t (B_t x_t + A abar_t h_{t-1});  dA += g_t dt_t abar_t h_{t-1}
//   ddelta_t = ddt_t sigmoid(delta_t + bias) (softplus on) or ddt_t;  dbias += ddelta_t;  dD += dy0_t x_t
// As the pages' hardware-aware backward does ("mamba->jamba" sec. 2.3: Abar and Bbar are recomputed
// in the backward pass rather than stored), nothing of size (B, L, D, N) is kept: the states are
// recomputed.
//
// One workgroup per (batch row, 64-channel block), with the wave roles of the forward kernel:
//   phase 0 (forward, chunks 0 .. nc-1): IO waves stage (dt, dt x) in LDS, scan waves run the
//     recurrence and store the state at the start of every kBwdChunk-step chunk in scratch
//     (B, nc, N, D) fp32 -- the only O(B L D N / kBwdChunk) memory the pass uses;
//   phase 1 (reverse, chunks nc-1 .. 0), per chunk:
//     A  IO:   load x, delta, z, dy; stage (dt, dt x) in LDS
//     B  scan: recompute the chunk's states from the stored chunk start, keep them in VGPRs, and
//              write the read-out partials C_t.h_t
//     C  IO:   y0 = sum of partials + D x; dz; dy0 = dy silu(z) into LDS; dD partial
//     D  scan: reverse the chunk: adjoint g, dA in registers, per-lane dx / ddt partials into
//              LDS, and the channel sums of dB / dC through an LDS transpose, written per channel
//              block to scratch
//     E  IO:   dx, ddelta from the partials; store dx, ddelta, dz; dbias partial
// A second kernel adds the channel-block partials of dB and dC, and the per-batch-row partials
// of dA, dD and dbias, in a fixed order (deterministic).
#pragma once

#include "ssm_device.hpp"

namespace ssm {

struct BwdArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* z;
  const float* delta_bias;
  const void* dy;
  void* dx;
  void* ddelta;
  void* dz;
  float* hstart;     // (batch, nc, N, dim) chunk-start states
  float* part_bc;    // (2, ncb, batch, L, N): dB then dC partial sums over one channel block
  float* part_a;     // (batch, N, dim)
  float* part_d;     // (batch, kBwdChunk, dim)
  float* part_bias;  // (batch, kBwdChunk, dim)
  int64_t batch;
  int64_t seqlen;
  int64_t dim;
  int64_t nc;        // chunks of kBwdChunk steps
  int32_t ncb;
  int32_t softplus;
  int32_t vec_ok;
};

constexpr int kBwdChunk = 16;
constexpr int kBwdIoWaves = 4;
// steps per dB / dC reduction round: 2 NPL values per step and lane, one column per lane
template <int NPL>
constexpr int kBwdHalf = 32 / NPL < kBwdChunk ? 32 / NPL : kBwdChunk;

// LDS written by some lanes of a wave is visible to all lanes of that wave afterwards
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool BF16, int N, int NPL>
__global__ __launch_bounds__(64 * (N / NPL + kBwdIoWaves)) void scan_bwd_kernel(const BwdArgs p) {
  constexpr int G = N / NPL;
  constexpr int T = kBwdChunk;
  constexpr int IOT = 64 * kBwdIoWaves;
  constexpr int EPT = T * 64 / IOT;  // tile elements per IO thread
  constexpr int VEC = EPT;           // one vector per IO thread: a row segment of EPT channels
  constexpr int TPR = 64 / VEC;      // IO threads per tile row
  static_assert(TPR * T == IOT, "IO threads cover the chunk tile exactly once");
  constexpr int H = kBwdHalf<NPL>;
  constexpr int RED = 2 * NPL * H;  // dB and dC values per lane per reduction round
  static_assert(RED <= 64 && T % H == 0, "one reduction column per lane, whole rounds per chunk");

  __shared__ float2 s_dw[T][64 + 2];        // (dt, dt x)
  __shared__ float s_yp[G][T][64 + 4];      // read-out partials
  __shared__ float s_dy0[T][64 + 2];        // dy * silu(z)
  __shared__ float2 s_part[G][T][64 + 2];   // (dx, ddt) partials
  __shared__ float s_red[G][64][RED + 1];   // per-wave transpose for the dB / dC channel sums

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t blk = blockIdx.x;
  const int cb = static_cast<int>(blk % p.ncb);
  const int64_t b = blk / p.ncb;
  const int64_t L = p.seqlen;
  const int64_t nc = p.nc;
  const int64_t row_base = b * L;
  const bool full_cols = p.vec_ok && (static_cast<int64_t>(cb) * 64 + 64 <= p.dim);
  auto chunk_full = [&](int64_t c) { return full_cols && (c + 1) * T <= L; };

  if (wave < G) {
    // ===================================== scan role ==========================================
    const int64_t d_lane = static_cast<int64_t>(cb) * 64 + lane;
    const bool lane_ok = d_lane < p.dim;
    const int n0 = wave * NPL;
    const int bc_k = lane & 15;
    float A2[NPL], Araw[NPL], h[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      Araw[j] = lane_ok ? p.A[d_lane * N + n0 + j] : 0.0f;
      A2[j] = fmaxf(Araw[j] * kLog2e, -3.0e38f);
      h[j] = 0.0f;
    }
    // B / C of a chunk: lane k of each 16-lane row holds step k
    auto load_bc = [&](int64_t c, BcRow<BF16, NPL>& rb, BcRow<BF16, NPL>& rc) {
      const int64_t t = c * T + bc_k;
      const int64_t e = (row_base + t) * N + n0;
      rb.load(p.B, e, t < L);
      rc.load(p.C, e, t < L);
    };
    auto hstart = [&](int64_t c, int j) -> float* {
      return p.hstart + ((b * nc + c) * N + n0 + j) * p.dim + d_lane;
    };

    // ---- phase 0: forward, storing every chunk-start state ----------------------------------
    for (int64_t c = 0; c < nc; ++c) {
      if (lane_ok) {
#pragma unroll
        for (int j = 0; j < NPL; ++j) *hstart(c, j) = h[j];
      }
      BcRow<BF16, NPL> rb, rc;
      load_bc(c, rb, rc);
      __syncthreads();  // s_dw of chunk c is ready
      float Bv[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) Bv[j] = rb.get(j);
      static_for<T>([&](auto K) {
        constexpr int k = decltype(K)::value;
        const float2 dw = s_dw[k][lane];
#pragma unroll
        for (int j = 0; j < NPL; ++j) h[j] = fmaf(hw_exp2(dw.x * A2[j]), h[j], row_bcast<k>(Bv[j]) * dw.y);
      });
      __syncthreads();  // s_dw may be rewritten
    }

    // ---- phase 1: reverse ---------------------------------------------------------------------
    float g[NPL], an[NPL], dA[NPL];  // adjoint, abar of the step after, dA accumulator
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      g[j] = 0.0f;
      an[j] = 0.0f;
      dA[j] = 0.0f;
    }
    float* const red = &s_red[wave][0][0];
    for (int64_t c = nc - 1; c >= 0; --c) {
      BcRow<BF16, NPL> rb, rc;
      load_bc(c, rb, rc);
      float Bv[NPL], Cv[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        Bv[j] = rb.get(j);
        Cv[j] = rc.get(j);
      }
      float hs[T + 1][NPL];  // hs[k] = state before step k of the chunk; hs[T] after its last step
#pragma unroll
      for (int j = 0; j < NPL; ++j) hs[0][j] = lane_ok ? *hstart(c, j) : 0.0f;
      __syncthreads();  // (A) s_dw of chunk c is ready
      // ---- B: recompute the chunk, read-out partials ----
      static_for<T>([&](auto K) {
        constexpr int k = decltype(K)::value;
        const float2 dw = s_dw[k][lane];
        float yp = 0.0f;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          hs[k + 1][j] = fmaf(hw_exp2(dw.x * A2[j]), hs[k][j], row_bcast<k>(Bv[j]) * dw.y);
          yp = fmaf(row_bcast<k>(Cv[j]), hs[k + 1][j], yp);
        }
        s_yp[wave][k][lane] = yp;
      });
      __syncthreads();  // (B) partials ready
      __syncthreads();  // (C) s_dy0 ready
      // ---- D: reverse the chunk ----
      static_for<T / H>([&](auto R) {
        constexpr int hf = T / H - 1 - decltype(R)::value;  // rounds in reverse
        static_for<H>([&](auto K) {
          constexpr int k = hf * H + H - 1 - decltype(K)::value;  // steps in reverse
          constexpr int r = k - hf * H;                                   // row in the round
          const float2 dw = s_dw[k][lane];
          const float dt = dw.x, w = dw.y;
          const float dy0 = s_dy0[k][lane];
          float gB = 0.0f, pdt = 0.0f;  // sum_j g_j B_j; sum_j g_j A_j abar_j h_{t-1,j}
#pragma unroll
          for (int j = 0; j < NPL; ++j) {
            const float Bk = row_bcast<k>(Bv[j]), Ck = row_bcast<k>(Cv[j]);
            const float a = hw_exp2(dt * A2[j]);  // abar_t
            g[j] = fmaf(an[j], g[j], dy0 * Ck);    // g_t = dy0 C_t + abar_{t+1} g_{t+1}
            const float ah = a * hs[k][j];         // abar_t h_{t-1}
            red[lane * (RED + 1) + r * 2 * NPL + j] = g[j] * w;                  // dB: g dt x
            red[lane * (RED + 1) + r * 2 * NPL + NPL + j] = dy0 * hs[k + 1][j];  // dC: dy0 h_t
            gB = fmaf(g[j], Bk, gB);
            pdt = fmaf(g[j] * Araw[j], ah, pdt);
            dA[j] = fmaf(g[j] * dt, ah, dA[j]);
            an[j] = a;
          }
          // dx partial = dt sum_j g_j B_j; ddt partial = sum_j g_j A_j abar_j h_{t-1,j}.  The
          // x sum_j g_j B_j part of ddt is added by the IO waves, which hold x.
          s_part[wave][k][lane] = make_float2(gB * dt, pdt);
          s_yp[wave][k][lane] = gB;
        });
        // channel sums of this round's dB / dC partials: lane l adds column l over the 64 lanes
        wave_sync();
        if (lane < RED) {
          float s = 0.0f;
          for (int l = 0; l < 64; ++l) s += red[l * (RED + 1) + lane];
          const int r = lane / (2 * NPL), q = lane % (2 * NPL);
          const int64_t t = c * T + hf * H + r;
          const int which = q < NPL ? 0 : 1;  // 0: dB, 1: dC
          const int n = n0 + (q % NPL);
          if (t < L)
            p.part_bc[((((int64_t)which * p.ncb + cb) * p.batch + b) * L + t) * N + n] = s;
        }
        wave_sync();  // the next round rewrites the transpose buffer
      });
      __syncthreads();  // (D) partials ready
      __syncthreads();  // (E) IO done with s_dw, s_part
    }
    if (lane_ok) {
#pragma unroll
      for (int j = 0; j < NPL; ++j) p.part_a[(b * N + n0 + j) * p.dim + d_lane] = dA[j];
    }
    return;
  }

  // ======================================= IO role ==============================================
  const int iot = tid - 64 * G;
  const int col = (iot % TPR) * VEC;
  const int row = iot / TPR;  // one tile row per IO thread
  const int64_t d_col = static_cast<int64_t>(cb) * 64 + col;
  const int nvalid_col = d_col >= p.dim ? 0 : static_cast<int>((p.dim - d_col) < VEC ? (p.dim - d_col) : VEC);
  float bias[VEC], dsk[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    bias[v] = (p.delta_bias && v < nvalid_col) ? p.delta_bias[d_col + v] : 0.0f;
    dsk[v] = (p.Dskip && v < nvalid_col) ? p.Dskip[d_col + v] : 0.0f;
  }
  const bool has_z = p.z != nullptr;
  // stages (dt, dt x) of chunk c into s_dw; returns the values it needs later
  auto stage = [&](int64_t c, float (&xs)[VEC], float (&vs)[VEC], float (&dts)[VEC], bool& row_ok) {
    const int64_t t = c * T + row;
    row_ok = t < L;
    const int nv = row_ok ? nvalid_col : 0;
    const int64_t idx = (row_base + t) * p.dim + d_col;
    const bool vec = chunk_full(c);
    RawVec<BF16, VEC> rx, rd;
    rx.load(p.x, idx, nv, vec);
    rd.load(p.delta, idx, nv, vec);
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const bool ok = v < nv;
      xs[v] = ok ? rx.get(v) : 0.0f;
      vs[v] = rd.get(v) + bias[v];
      const float dt = p.softplus ? softplus_f32(vs[v]) : vs[v];
      dts[v] = ok ? dt : 0.0f;
      s_dw[row][col + v] = make_float2(dts[v], dts[v] * xs[v]);
    }
  };

  // ---- phase 0 ----
  for (int64_t c = 0; c < nc; ++c) {
    float xs[VEC], vs[VEC], dts[VEC];
    bool row_ok;
    stage(c, xs, vs, dts, row_ok);
    __syncthreads();
    __syncthreads();
  }
  // ---- phase 1 ----
  float accD[VEC], accBias[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) accD[v] = accBias[v] = 0.0f;
  for (int64_t c = nc - 1; c >= 0; --c) {
    float xs[VEC], vs[VEC], dts[VEC];
    bool row_ok;
    stage(c, xs, vs, dts, row_ok);  // (A)
    const int64_t t = c * T + row;
    const int nv = row_ok ? nvalid_col : 0;
    const int64_t idx = (row_base + t) * p.dim + d_col;
    const bool vec = chunk_full(c);
    RawVec<BF16, VEC> rz, rdy;
    if (has_z) rz.load(p.z, idx, nv, vec);
    rdy.load(p.dy, idx, nv, vec);
    __syncthreads();  // (A)
    __syncthreads();  // (B) read-out partials ready
    // ---- C ----
    float dy0[VEC], dzv[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      float y0 = fmaf(dsk[v], xs[v], s_yp[0][row][col + v]);
#pragma unroll
      for (int gw = 1; gw < G; ++gw) y0 += s_yp[gw][row][col + v];
      const float dyv = v < nv ? rdy.get(v) : 0.0f;
      if (has_z) {
        const float zv = rz.get(v);
        const float sg = hw_rcp(1.0f + hw_exp2(-zv * kLog2e));
        dzv[v] = dyv * y0 * fmaf(zv * sg, 1.0f - sg, sg);
        dy0[v] = dyv * zv * sg;
      } else {
        dzv[v] = 0.0f;
        dy0[v] = dyv;
      }
      accD[v] = fmaf(dy0[v], xs[v], accD[v]);
      s_dy0[row][col + v] = dy0[v];
    }
    __syncthreads();  // (C)
    __syncthreads();  // (D) partials ready
    // ---- E ----
    float dxo[VEC], ddo[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      float dxv = dy0[v] * dsk[v], ddt = 0.0f, gB = 0.0f;
#pragma unroll
      for (int gw = 0; gw < G; ++gw) {
        const float2 pr = s_part[gw][row][col + v];
        dxv += pr.x;
        ddt += pr.y;
        gB += s_yp[gw][row][col + v];
      }
      ddt = fmaf(gB, xs[v], ddt);  // the B x term of ddt
      const float dd = p.softplus ? ddt * hw_rcp(1.0f + hw_exp2(-vs[v] * kLog2e)) : ddt;
      dxo[v] = dxv;
      ddo[v] = dd;
      if (v < nv) accBias[v] += dd;
    }
    if (nv > 0) {
      store_vec<BF16, VEC>(p.dx, idx, dxo, nv, vec);
      store_vec<BF16, VEC>(p.ddelta, idx, ddo, nv, vec);
      if (has_z) store_vec<BF16, VEC>(p.dz, idx, dzv, nv, vec);
    }
    __syncthreads();  // (E)
  }
  // per-(batch row, tile row) partials of dD and dbias, summed by the reduce kernel
  if (nvalid_col > 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      if (v < nvalid_col) {
        p.part_d[(b * T + row) * p.dim + d_col + v] = accD[v];
        p.part_bias[(b * T + row) * p.dim + d_col + v] = accBias[v];
      }
    }
  }
}

// Second pass: fixed-order sums of the partials.
//   dB / dC (batch, L, N) in the storage type: sum over the ncb channel blocks;
//   dA (dim, N), dD (dim), dbias (dim) in fp32: sum over the batch rows.
struct BwdReduceArgs {
  const float* part_bc;
  const float* part_a;
  const float* part_d;
  const float* part_bias;
  void* dB;
  void* dC;
  float* dA;
  float* dD;
  float* dbias;
  int64_t batch;
  int64_t seqlen;
  int64_t dim;
  int32_t N;
  int32_t ncb;
};

template <bool BF16>
__global__ __launch_bounds__(256) void scan_bwd_reduce_kernel(const BwdReduceArgs p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nbln = p.batch * p.seqlen * p.N;
  const int64_t ndn = p.dim * p.N;
  if (i < 2 * nbln) {
    const int which = i < nbln ? 0 : 1;
    const int64_t e = i - which * nbln;  // (b, t, n)
    float s = 0.0f;
    for (int k = 0; k < p.ncb; ++k) s += p.part_bc[(static_cast<int64_t>(which) * p.ncb + k) * nbln + e];
    void* out = which == 0 ? p.dB : p.dC;
    if constexpr (BF16) static_cast<uint16_t*>(out)[e] = to_bf16(s);
    else static_cast<float*>(out)[e] = s;
    return;
  }
  const int64_t j = i - 2 * nbln;
  if (j < ndn) {  // dA[d, n] = sum_b part_a[b, n, d]
    const int64_t d = j / p.N, n = j % p.N;
    float s = 0.0f;
    for (int64_t bb = 0; bb < p.batch; ++bb) s += p.part_a[(bb * p.N + n) * p.dim + d];
    p.dA[j] = s;
    return;
  }
  const int64_t k = j - ndn;
  if (k < p.dim) {
    float sd = 0.0f, sb = 0.0f;
    for (int64_t r = 0; r < p.batch * kBwdChunk; ++r) {
      sd += p.part_d[r * p.dim + k];
      sb += p.part_bias[r * p.dim + k];
    }
    if (p.dD) p.dD[k] = sd;
    if (p.dbias) p.dbias[k] = sb;
  }
}

}  // namespace ssm
