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
//     recurrence and store the state at the start of every T-step chunk in scratch
//     (B, nc, N, D) fp32 -- the only O(B L D N / T) memory the pass uses;
//   phase 1 (reverse, chunks nc-1 .. 0), per chunk, with two barriers:
//     A  IO:   stage (dt, dt x) and dy0 = dy silu(z) in LDS from the x, delta, z, dy tile fetched
//              a chunk earlier (dy0 needs no read-out, so it is staged up front); dD partial;
//              fetch the next chunk's tile                                      -- barrier (1)
//     B  scan: recompute the chunk's states from the stored chunk start, keep them in VGPRs, and
//              write the read-out partials C_t.h_t
//     D  scan: reverse the chunk: adjoint g, dA in registers, per-lane dx / ddt partials into
//              LDS, and the channel sums of dB / dC through an LDS transpose, written per channel
//              block to scratch                                               -- barrier (2)
//     E  IO:   y0 = sum of partials + D x, dz, and dx, ddelta from the partials; store dx,
//              ddelta, dz; dbias partial
// A second kernel adds the channel-block partials of dB and dC, and the per-batch-row partials
// of dA, dD and dbias, in a fixed order (deterministic).
//
// Exact zero-order hold (ZOH, "Mamba 论文精读" sec. 2.2): the input term is phi B x with
// phi = expm1(dt A) / A = dt fz, fz = log2(e) m, m = zoh_factor.  Its adjoint differs in
//   dB_t += g dt x fz;  dx_t += dt sum_n g fz B;  ddt_t = x sum_n g abar B + sum_n g A abar h_{t-1};
//   dA += g dt (abar h_{t-1} + B dt x psi(dt A)),  psi(z) = ((z - 1) e^z + 1) / z^2
// (the derivative of phi in A over dt^2), so the scan waves hand the IO waves one more sum.
// Wider states (N 32, 64) keep four scan waves with 8 or 16 chains per lane and shorter chunks
// (8 or 4 steps), which keeps a chunk's recomputed states in VGPRs.
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
  float* hstart;     // chunk-start states: (batch, nc, N, dim) channel lanes, (batch, nc, dim, N) state rows
  int32_t have_hstart;  // state rows: hstart holds the forward's checkpoints, so there is no phase 0
  float* part_bc;    // (2, ncb, batch, L, N): dB then dC partial sums over one channel block
  float* part_a;     // (batch, N, dim)
  float* part_d;     // (batch, T, dim), T the chunk length
  float* part_bias;  // (batch, T, dim)
  int64_t batch;
  int64_t seqlen;
  int64_t dim;
  int64_t nc;        // chunks of T steps
  int32_t ncb;
  int32_t softplus;
  int32_t vec_ok;
};

constexpr int kBwdChunk = 16;  // chunk length for dstate <= 16
constexpr int kBwdIoWaves = 4;
// chunk length of an instantiation: 16 steps up to 4 chains per lane, 8 for 8, 4 for 16; the
// exact-ZOH step keeps more values live, so it takes half that (at least 4: one tile row per IO
// thread)
constexpr int bwd_chunk(int npl, bool zoh) {
  const int t = npl <= 4 ? 16 : (npl == 8 ? 8 : 4);
  return zoh ? (t / 2 < 4 ? 4 : t / 2) : t;
}
// steps per dB / dC reduction round: 2 NPL values per step and lane, at most 64 rows per round
template <int NPL, int T>
constexpr int kBwdHalf = 32 / NPL < T ? 32 / NPL : T;

// psi(z) = ((z - 1) e^z + 1) / z^2 = 1/2 + z/3 + z^2/8 + z^3/30 + z^4/144 + ..., with a = e^z
// given.  The closed form cancels for small |z|, where the series (error below 2e-9 relative for
// |z| < 1/8) is used.
__device__ __forceinline__ float zoh_psi(float zz, float a) {
  const float series = fmaf(zz, fmaf(zz, fmaf(zz, fmaf(zz, 1.0f / 144.0f, 1.0f / 30.0f), 0.125f), 1.0f / 3.0f), 0.5f);
  const float closed = fmaf(zz - 1.0f, a, 1.0f) * hw_rcp(zz * zz);
  return fabsf(zz) < 0.125f ? series : closed;
}

// LDS written by some lanes of a wave is visible to all lanes of that wave afterwards
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool BF16, int N, int NPL, bool ZOH = false>
__global__ __launch_bounds__(64 * (N / NPL + kBwdIoWaves)) void scan_bwd_kernel(const BwdArgs p) {
  constexpr int G = N / NPL;
  constexpr int T = bwd_chunk(NPL, ZOH);
  constexpr int IOT = 64 * kBwdIoWaves;
  constexpr int EPT = T * 64 / IOT;  // tile elements per IO thread
  constexpr int VEC = EPT;           // one vector per IO thread: a row segment of EPT channels
  constexpr int TPR = 64 / VEC;      // IO threads per tile row
  static_assert(TPR * T == IOT, "IO threads cover the chunk tile exactly once");
  constexpr int H = kBwdHalf<NPL, T>;
  constexpr int RED = 2 * NPL * H;  // dB and dC values per lane per reduction round
  static_assert(RED <= 64 && T % H == 0, "one reduction row per lane, whole rounds per chunk");

  __shared__ float2 s_dw[2][T][64 + 2];               // (dt, dt x); phase 0 double-buffers
  __shared__ float s_dy0[T][64 + 2];                  // dy * silu(z)
  __shared__ float s_yp[G][T][64 + 4];                // read-out partials C_t.h_t
  // (sum_j g_j B_j fz_j, sum_j g_j A_j abar_j h_{t-1,j}); with ZOH also sum_j g_j abar_j B_j
  __shared__ float2 s_part[G][T][64 + 2];
  __shared__ float s_part_z[ZOH ? G : 1][ZOH ? T : 1][64 + 4];
  __shared__ __align__(16) float s_red[G][RED][64 + 4];  // per-wave transpose for dB / dC sums

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

  // Barriers: phase 0 runs nc + 1 iterations with one barrier each; phase 1 runs nc chunks with
  // two barriers each (after the IO staging, after the scan).  Both roles follow that count.
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

    // ---- phase 0: forward over chunk j-1 while the IO waves stage chunk j --------------------
    BcRow<BF16, NPL> rb0, rc0;
    if (nc > 0) load_bc(0, rb0, rc0);
    for (int64_t j = 0; j <= nc; ++j) {
      if (j >= 1) {
        const int64_t c = j - 1;
        const int sb = static_cast<int>(c & 1);
        if (lane_ok) {
#pragma unroll
          for (int q = 0; q < NPL; ++q) *hstart(c, q) = h[q];
        }
        float Bv[NPL];
#pragma unroll
        for (int q = 0; q < NPL; ++q) Bv[q] = rb0.get(q);
        if (c + 1 < nc) load_bc(c + 1, rb0, rc0);
        static_for<T>([&](auto K) {
          constexpr int k = decltype(K)::value;
          const float2 dw = s_dw[sb][k][lane];
#pragma unroll
          for (int q = 0; q < NPL; ++q) {
            const float tt = dw.x * A2[q];
            const float a = hw_exp2(tt);
            const float u = ZOH ? dw.y * (kLog2e * zoh_factor(tt, a)) : dw.y;
            h[q] = fmaf(a, h[q], row_bcast<k>(Bv[q]) * u);
          }
        });
      }
      __syncthreads();
    }

    // ---- phase 1: reverse ---------------------------------------------------------------------
    float g[NPL], an[NPL], dA[NPL];  // adjoint, abar of the step after, dA accumulator
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      g[q] = 0.0f;
      an[q] = 0.0f;
      dA[q] = 0.0f;
    }
    float* const red = &s_red[wave][0][0];
    for (int64_t c = nc - 1; c >= 0; --c) {
      BcRow<BF16, NPL> rb, rc;
      load_bc(c, rb, rc);
      float hs[T + 1][NPL];  // hs[k] = state before step k of the chunk; hs[T] after its last step
#pragma unroll
      for (int q = 0; q < NPL; ++q) hs[0][q] = lane_ok ? *hstart(c, q) : 0.0f;
      __syncthreads();  // (1) the chunk's (dt, dt x) and dy0 are staged
      float Bv[NPL], Cv[NPL];
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        Bv[q] = rb.get(q);
        Cv[q] = rc.get(q);
      }
      // recompute the chunk's states and read-out partials
      static_for<T>([&](auto K) {
        constexpr int k = decltype(K)::value;
        const float2 dw = s_dw[0][k][lane];
        float yp = 0.0f;
#pragma unroll
        for (int q = 0; q < NPL; ++q) {
          const float tt = dw.x * A2[q];
          const float a = hw_exp2(tt);
          const float u = ZOH ? dw.y * (kLog2e * zoh_factor(tt, a)) : dw.y;
          hs[k + 1][q] = fmaf(a, hs[k][q], row_bcast<k>(Bv[q]) * u);
          yp = fmaf(row_bcast<k>(Cv[q]), hs[k + 1][q], yp);
        }
        s_yp[wave][k][lane] = yp;
      });
      // reverse the chunk, in rounds of H steps for the dB / dC channel sums
      static_for<T / H>([&](auto R) {
        constexpr int hf = T / H - 1 - decltype(R)::value;  // rounds in reverse
        static_for<H>([&](auto K) {
          constexpr int k = hf * H + H - 1 - decltype(K)::value;  // steps in reverse
          constexpr int r = k - hf * H;                             // step within the round
          const float2 dw = s_dw[0][k][lane];
          const float dt = dw.x, w = dw.y;
          const float dy0 = s_dy0[k][lane];
          float gB = 0.0f, pdt = 0.0f, gBa = 0.0f;
#pragma unroll
          for (int q = 0; q < NPL; ++q) {
            g[q] = fmaf(an[q], g[q], dy0 * row_bcast<k>(Cv[q]));  // g_t = dy0 C_t + abar_{t+1} g_{t+1}
            const float tt = dt * A2[q];
            const float a = hw_exp2(tt);                           // abar_t (recomputed)
            const float ah = a * hs[k][q];                         // abar_t h_{t-1}
            const float b = row_bcast<k>(Bv[q]);
            if constexpr (ZOH) {
              const float fz = kLog2e * zoh_factor(tt, a);         // phi / dt
              const float gfz = g[q] * fz;
              red[(r * 2 * NPL + q) * (64 + 4) + lane] = gfz * w;  // dB: g phi x
              gB = fmaf(gfz, b, gB);                                // sum g phi B / dt
              gBa = fmaf(g[q] * a, b, gBa);                         // sum g abar B
              const float gah = g[q] * ah;
              pdt = fmaf(gah, Araw[q], pdt);
              // dA += g dt (abar h_{t-1} + B dt x psi(dt A))
              const float psi = zoh_psi(tt * kLn2, a);
              dA[q] = fmaf(g[q] * dt, fmaf(b * w, psi, ah), dA[q]);
            } else {
              red[(r * 2 * NPL + q) * (64 + 4) + lane] = g[q] * w;  // dB: g dt x
              gB = fmaf(g[q], b, gB);
              const float gah = g[q] * ah;
              pdt = fmaf(gah, Araw[q], pdt);
              dA[q] = fmaf(gah, dt, dA[q]);
            }
            red[(r * 2 * NPL + NPL + q) * (64 + 4) + lane] = dy0 * hs[k + 1][q];  // dC: dy0 h_t
            an[q] = a;
          }
          s_part[wave][k][lane] = make_float2(gB, pdt);
          if constexpr (ZOH) s_part_z[wave][k][lane] = gBa;
        });
        // channel sums of this round's dB / dC values: lane q adds row q of the transpose
        wave_sync();
        if (lane < RED) {
          const float4* rowp = reinterpret_cast<const float4*>(red + lane * (64 + 4));
          float4 acc = rowp[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) {
            const float4 v = rowp[i];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
          }
          const float sum = (acc.x + acc.y) + (acc.z + acc.w);
          const int r = lane / (2 * NPL), qq = lane % (2 * NPL);
          const int64_t t = c * T + hf * H + r;
          const int which = qq < NPL ? 0 : 1;  // 0: dB, 1: dC
          const int n = n0 + (qq % NPL);
          if (t < L) p.part_bc[((((int64_t)which * p.ncb + cb) * p.batch + b) * L + t) * N + n] = sum;
        }
        wave_sync();  // the next round rewrites the transpose buffer
      });
      __syncthreads();  // (2) read-out and adjoint partials are ready
    }
    if (lane_ok) {
#pragma unroll
      for (int q = 0; q < NPL; ++q) p.part_a[(b * N + n0 + q) * p.dim + d_lane] = dA[q];
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
  // Raw tiles are loaded one chunk ahead of their use, so the global-load latency overlaps the
  // scan waves' work on the current chunk.
  struct Raw {
    RawVec<BF16, VEC> x, d, z, dy;
    int nv;
  };
  auto fetch = [&](int64_t c, Raw& r, bool grads) {
    const int64_t t = c * T + row;
    r.nv = t < L ? nvalid_col : 0;
    const int64_t idx = (row_base + t) * p.dim + d_col;
    const bool vec = chunk_full(c);
    r.x.load(p.x, idx, r.nv, vec);
    r.d.load(p.delta, idx, r.nv, vec);
    if (grads) {
      if (has_z) r.z.load(p.z, idx, r.nv, vec);
      r.dy.load(p.dy, idx, r.nv, vec);
    }
  };
  // (dt, dt x) of a fetched tile into s_dw[sb]; x and the pre-softplus value kept
  auto stage = [&](const Raw& r, int sb, float (&xs)[VEC], float (&vs)[VEC]) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const bool ok = v < r.nv;
      xs[v] = ok ? r.x.get(v) : 0.0f;
      vs[v] = r.d.get(v) + bias[v];
      const float dt = ok ? (p.softplus ? softplus_f32(vs[v]) : vs[v]) : 0.0f;
      s_dw[sb][row][col + v] = make_float2(dt, dt * xs[v]);
    }
  };

  // ---- phase 0 ----
  {
    Raw cur;
    if (nc > 0) fetch(0, cur, false);
    for (int64_t j = 0; j <= nc; ++j) {
      if (j < nc) {
        float xs[VEC], vs[VEC];
        stage(cur, static_cast<int>(j & 1), xs, vs);
        if (j + 1 < nc) fetch(j + 1, cur, false);
      }
      __syncthreads();
    }
  }
  // ---- phase 1 ----
  float accD[VEC], accBias[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) accD[v] = accBias[v] = 0.0f;
  Raw nxt;
  if (nc > 0) fetch(nc - 1, nxt, true);
  for (int64_t c = nc - 1; c >= 0; --c) {
    const Raw cur = nxt;
    float xs[VEC], vs[VEC];
    stage(cur, 0, xs, vs);
    const int nv = cur.nv;
    const int64_t idx = (row_base + c * T + row) * p.dim + d_col;
    const bool vec = chunk_full(c);
    float dyv[VEC], zv[VEC], sg[VEC], dy0[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      dyv[v] = v < nv ? cur.dy.get(v) : 0.0f;
      if (has_z) {
        zv[v] = cur.z.get(v);
        sg[v] = hw_rcp(1.0f + hw_exp2(-zv[v] * kLog2e));
        dy0[v] = dyv[v] * zv[v] * sg[v];
      } else {
        zv[v] = sg[v] = 0.0f;
        dy0[v] = dyv[v];
      }
      accD[v] = fmaf(dy0[v], xs[v], accD[v]);
      s_dy0[row][col + v] = dy0[v];
    }
    if (c > 0) fetch(c - 1, nxt, true);
    __syncthreads();  // (1)
    __syncthreads();  // (2) the scan waves' partials are ready
    float dxo[VEC], ddo[VEC], dzo[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      float y0 = dsk[v] * xs[v], gB = 0.0f, pdt = 0.0f, gBa = 0.0f;
#pragma unroll
      for (int gw = 0; gw < G; ++gw) {
        y0 += s_yp[gw][row][col + v];
        const float2 pr = s_part[gw][row][col + v];
        gB += pr.x;
        pdt += pr.y;
        if constexpr (ZOH) gBa += s_part_z[gw][row][col + v];
      }
      const float dt = s_dw[0][row][col + v].x;
      dzo[v] = has_z ? dyv[v] * y0 * fmaf(zv[v] * sg[v], 1.0f - sg[v], sg[v]) : 0.0f;
      dxo[v] = fmaf(dy0[v], dsk[v], dt * gB);
      const float ddt = fmaf(ZOH ? gBa : gB, xs[v], pdt);
      ddo[v] = p.softplus ? ddt * hw_rcp(1.0f + hw_exp2(-vs[v] * kLog2e)) : ddt;
      if (v < nv) accBias[v] += ddo[v];
    }
    if (nv > 0) {
      store_vec<BF16, VEC>(p.dx, idx, dxo, nv, vec);
      store_vec<BF16, VEC>(p.ddelta, idx, ddo, nv, vec);
      if (has_z) store_vec<BF16, VEC>(p.dz, idx, dzo, nv, vec);
    }
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
  int32_t T;  // chunk length of the main kernel (rows of the dD / dbias partials)
};

// Sum of n values base[i * stride], i = 0 .. n-1, with 8 independent accumulators so that the
// loads overlap; the order of the additions is fixed, so the result is reproducible.
__device__ __forceinline__ float strided_sum(const float* base, int64_t n, int64_t stride) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t i = 0;
  for (; i + 8 <= n; i += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += base[(i + u) * stride];
  }
  for (int u = 0; i < n; ++i, ++u) acc[u] += base[i * stride];
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

template <bool BF16>
__global__ __launch_bounds__(256) void scan_bwd_reduce_kernel(const BwdReduceArgs p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nbln = p.batch * p.seqlen * p.N;
  const int64_t ndn = p.dim * p.N;
  if (i < 2 * nbln) {
    const int which = i < nbln ? 0 : 1;
    const int64_t e = i - which * nbln;  // (b, t, n)
    const float s = strided_sum(p.part_bc + static_cast<int64_t>(which) * p.ncb * nbln + e, p.ncb, nbln);
    void* out = which == 0 ? p.dB : p.dC;
    if constexpr (BF16) static_cast<uint16_t*>(out)[e] = to_bf16(s);
    else static_cast<float*>(out)[e] = s;
    return;
  }
  const int64_t j = i - 2 * nbln;
  if (j < ndn) {  // dA[d, n] = sum_b part_a[b, n, d]
    const int64_t d = j / p.N, n = j % p.N;
    p.dA[j] = strided_sum(p.part_a + n * p.dim + d, p.batch, static_cast<int64_t>(p.N) * p.dim);
    return;
  }
  const int64_t k = j - ndn;
  if (k < p.dim) {
    const float sd = strided_sum(p.part_d + k, p.batch * p.T, p.dim);
    const float sb = strided_sum(p.part_bias + k, p.batch * p.T, p.dim);
    if (p.dD) p.dD[k] = sd;
    if (p.dbias) p.dbias[k] = sb;
  }
}

}  // namespace ssm
