// ssd_fwd.hpp -- forward pass of the Mamba-2 state space dual (SSD) layer for gfx950, chunked,
// with every contraction on bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// "Mamba 论文精读" sec. 4.1 gives the recurrence h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t and
// its dual: the same outputs are a product with a lower-triangular (causal) semi-separable
// matrix.  Sec. 4.2 adds heads and larger states (N up to 256); sec. 5.2 gives the layer's
// headdim and d_state.  Per head A is one scalar, Bbar = dt B as in the selective scan, and the
// heads of a group share B and C.  For one head and a chunk of Q = 64 steps, with
// cum_i = sum_{k<=i} dt_k A inside the chunk and S (dstate x headdim) the state entering it:
//
//   Y[i,:] = sum_{j<=i} (C_i . B_j) exp(cum_i - cum_j) dt_j X[j,:]     (the masked matrix form)
//          + exp(cum_i) C_i S                                          (read-out of S)
//   S'     = exp(cum_{Q-1}) S + sum_j B_j^T exp(cum_{Q-1} - cum_j) dt_j X[j,:]
//   y      = (Y + D x) * silu(z)
//
// Unrolling the recurrence over the chunk gives exactly these sums, so the chunked form is the
// recurrence reordered.  Within a chunk the work is four small matrix products: G = C B^T
// (Q x Q, over dstate), the masked product with X (over the chunk's steps), C S (over dstate)
// and B^T X (over the steps).
//
// Work split: one workgroup per (batch row, head, slice of PS = 16*NW head channels).  Wave w
// owns channels [16w, 16w+16) of the slice, so the columns of S it updates are exactly the ones
// it reads out: S never leaves the wave's accumulators.  Each wave forms all of G itself
// (redundant across the waves of a workgroup), which saves a barrier and an LDS round trip.
//
// Operand layouts of the 16x16x32 product D = A B (lane l, q = l / 16, i = 0..7, r = 0..3):
//   A: lane l holds A[l % 16][8q + i];  B: lane l holds B[8q + i][l % 16];
//   D: lane l holds D[4q + r][l % 16].
// A D tile therefore hands each lane four CONSECUTIVE rows of one column.  Two D tiles over
// rows k0..k0+15 and k0+16..k0+31 give lane l the k indices {k0 + 4q + r} and {k0 + 16 + 4q + r}:
// the same eight k values, in a fixed order, that a K = 32 step asks of lane l, up to a
// permutation of k.  A product sums over k, so it is unchanged when both operands use the same
// permutation.  That lets G (computed transposed, so its columns are the output rows) become the
// A operand of the masked product, and S become the B operand of the read-out, with no LDS
// round trip; the other operand is read from LDS in the same permuted order.
#pragma once

#include "ssm_device.hpp"

namespace ssm {

struct SsdArgs {
  const uint16_t* x;     // (batch, seqlen, nheads, headdim) bf16
  const uint16_t* dt;    // (batch, seqlen, nheads) bf16, before bias and softplus
  const float* A;        // (nheads)
  const uint16_t* B;     // (batch, seqlen, ngroups, dstate) bf16
  const uint16_t* C;     // (batch, seqlen, ngroups, dstate) bf16
  const float* D;        // (nheads) or NULL
  const uint16_t* z;     // like x, or NULL
  const float* dt_bias;  // (nheads) or NULL
  uint16_t* y;           // like x
  float* final_state;    // (batch, nheads, headdim, dstate) or NULL
  int64_t batch;
  int64_t seqlen;
  int32_t nheads;
  int32_t headdim;
  int32_t ngroups;
  int32_t nslices;  // headdim / PS
  int32_t softplus;
};

constexpr int kSsdChunk = 64;  // steps per chunk: one per lane of a wave

typedef __bf16 ssd_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float ssd_f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t ssd_u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t ssd_u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ ssd_f32x4_t mfma16x16x32(ssd_u32x4_t a, ssd_u32x4_t b, ssd_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(ssd_bf16x8_t, a),
                                                 __builtin_bit_cast(ssd_bf16x8_t, b), c, 0, 0, 0);
}

// Two 8-byte halves k0..k0+3 and k0+16..k0+19 of a bf16 row: the permuted K = 32 fragment.
__device__ __forceinline__ ssd_u32x4_t load_perm_frag(const uint16_t* row_k0) {
  const ssd_u32x2_t lo = *reinterpret_cast<const ssd_u32x2_t*>(row_k0);
  const ssd_u32x2_t hi = *reinterpret_cast<const ssd_u32x2_t*>(row_k0 + 16);
  return ssd_u32x4_t{lo.x, lo.y, hi.x, hi.y};
}

// Element e of two bf16 rows (low half from `a`, high half from `b`) as one word.
template <int E>
__device__ __forceinline__ uint32_t column_pair(ssd_u32x4_t a, ssd_u32x4_t b) {
  const uint32_t wa = a[E / 2], wb = b[E / 2];
  return (E & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
}

template <int E>
__device__ __forceinline__ float bf16_elem(ssd_u32x4_t v) {
  return (E & 1) ? bf16_hi(v[E / 2]) : bf16_lo(v[E / 2]);
}

// Workgroups of 4 waves (dstate <= 128) keep two workgroups per compute unit: their LDS fits
// twice in 160 KB and the registers are held to 256 per lane.
// Inclusive prefix sum over the 64 lanes of a wave with DPP (gfx9): shifts by 1, 2, 4, 8 within
// each row of 16 (lanes shifted in from outside the row read 0), then lane 15 of each row is
// added to rows 1 and 3 and lane 31 to rows 2 and 3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true));
}
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  v += dpp_or_zero<0x111, 0xF>(v);  // row_shr:1
  v += dpp_or_zero<0x112, 0xF>(v);  // row_shr:2
  v += dpp_or_zero<0x114, 0xF>(v);  // row_shr:4
  v += dpp_or_zero<0x118, 0xF>(v);  // row_shr:8
  v += dpp_or_zero<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_or_zero<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

template <int N, int NW>
constexpr int kSsdWavesPerEu = (NW == 4 && N <= 128) ? 2 : 1;

template <int N, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(kSsdWavesPerEu<N, NW>)))
void ssd_chunk_kernel(const SsdArgs p) {
  constexpr int Q = kSsdChunk;
  constexpr int PS = 16 * NW;  // head channels per workgroup
  constexpr int T = 64 * NW;   // threads
  constexpr int LDB = N + 8;   // row stride (elements) of the row-major B and C tiles
  constexpr int LDT = Q + 8;   // row stride of the step-indexed tiles (B^T, X^T, weighted X^T, M)
  constexpr int NKS = N / 32;  // K = 32 steps over dstate
  constexpr int NT = N / 16;   // 16-row tiles of S per wave
  constexpr int kBTasks = 4 * N;  // (row pair, 8-column group) pieces of B
  constexpr int kBPer = (kBTasks + T - 1) / T;
  constexpr int kCTasks = 8 * N;  // (row, 8-column group) pieces of C
  constexpr int kCPer = (kCTasks + T - 1) / T;
  static_assert(N % 32 == 0, "dstate is a multiple of 32");
  static_assert(4 * PS == T, "one (row pair, 8-column group) piece of X per thread");

  __shared__ __align__(16) uint16_t s_b[Q * LDB];    // B[j][n]
  __shared__ __align__(16) uint16_t s_c[Q * LDB];    // C[i][n]
  __shared__ __align__(16) uint16_t s_bt[N * LDT];   // B^T[n][j]
  __shared__ __align__(16) uint16_t s_xt[PS * LDT];  // X^T[p][j]
  __shared__ __align__(16) uint16_t s_xw[PS * LDT];  // X^T[p][j] * exp(cum_last - cum_j) dt_j
  __shared__ __align__(16) uint16_t s_m[Q * LDT];    // M[i][j] = (C_i . B_j) exp(cum_i - cum_j) dt_j, j <= i
  __shared__ __align__(16) float s_cum[Q];           // cum_j in log2 units
  __shared__ __align__(16) float s_dt[Q];            // dt_j (0 past the end of the sequence)

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t blk = blockIdx.x;
  const int slice = static_cast<int>(blk % p.nslices);
  const int64_t bh = blk / p.nslices;
  const int h = static_cast<int>(bh % p.nheads);
  const int64_t b = bh / p.nheads;
  const int g = h / (p.nheads / p.ngroups);
  const int64_t L = p.seqlen, H = p.nheads, P = p.headdim, G = p.ngroups;
  const int p0 = slice * PS;
  const float A2 = p.A[h] * kLog2e;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const float Dh = p.D ? p.D[h] : 0.0f;
  const int pw = 16 * wave + l16;     // this lane's S column (A-operand row of the products)
  const int pe = 16 * wave + 4 * q;   // first of the 4 channels this lane writes

  const uint16_t* xg = p.x + (b * L * H + h) * P + p0;  // step t at xg + t * H * P
  const uint16_t* zg = p.z ? p.z + (b * L * H + h) * P + p0 + pe : nullptr;
  uint16_t* yg = p.y + (b * L * H + h) * P + p0 + pe;
  const uint16_t* bg = p.B + (b * L * G + g) * N;  // step t at bg + t * G * N
  const uint16_t* cg = p.C + (b * L * G + g) * N;
  const uint16_t* dtg = p.dt + b * L * H + h;       // step t at dtg + t * H
  const int64_t xs = H * P, bs = G * N;

  // Registers that carry the next chunk's inputs while the current one is computed.
  ssd_u32x4_t rb[kBPer][2], rc[kCPer], rx[2];
  ssd_u32x2_t rz[4];
  uint32_t rdt = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) rz[k] = ssd_u32x2_t{0u, 0u};

  // FULL: all 64 steps of the chunk are inside the sequence (no bounds checks).
  auto load_chunk = [&](int64_t t0, auto full) {
    constexpr bool FULL = decltype(full)::value;
#pragma unroll
    for (int u = 0; u < kBPer; ++u) {
      const int k = tid + u * T;
      if (kBPer * T == kBTasks || k < kBTasks) {
        const int rp = k % 32, c8 = k / 32;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int64_t t = t0 + 2 * rp + hb;
          rb[u][hb] = (FULL || t < L) ? *reinterpret_cast<const ssd_u32x4_t*>(bg + t * bs + 8 * c8)
                                      : ssd_u32x4_t{0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCPer; ++u) {
      const int k = tid + u * T;
      if (kCPer * T == kCTasks || k < kCTasks) {
        const int c8 = k % (N / 8), i = k / (N / 8);
        const int64_t t = t0 + i;
        rc[u] = (FULL || t < L) ? *reinterpret_cast<const ssd_u32x4_t*>(cg + t * bs + 8 * c8) : ssd_u32x4_t{0, 0, 0, 0};
      }
    }
    {
      const int rp = tid % 32, p8 = tid / 32;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int64_t t = t0 + 2 * rp + hb;
        rx[hb] = (FULL || t < L) ? *reinterpret_cast<const ssd_u32x4_t*>(xg + t * xs + 8 * p8) : ssd_u32x4_t{0, 0, 0, 0};
      }
    }
    rdt = (FULL || t0 + lane < L) ? dtg[(t0 + lane) * H] : 0u;
    if (zg) {
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const int64_t t = t0 + 16 * ib + l16;
        rz[ib] = (FULL || t < L) ? *reinterpret_cast<const ssd_u32x2_t*>(zg + t * xs) : ssd_u32x2_t{0u, 0u};
      }
    }
  };

  // Writes the chunk held in registers to LDS.
  auto stage_chunk = [&](int64_t t0) {
    // dt and the cumulative decay: lane l of every wave holds step l of the chunk
    float dtv = 0.0f;
    if (t0 + lane < L) {
      const float v = bf16_lo(rdt) + bias;
      dtv = p.softplus ? softplus_f32(v) : v;
    }
    const float cum = wave_inclusive_sum(dtv * A2);
    const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cum), 63));
    const float wgt = hw_exp2(last - cum) * dtv;
    if (wave == 0) {
      s_cum[lane] = cum;
      s_dt[lane] = dtv;
    }
#pragma unroll
    for (int u = 0; u < kBPer; ++u) {
      const int k = tid + u * T;
      if (kBPer * T == kBTasks || k < kBTasks) {
        const int rp = k % 32, c8 = k / 32;
        *reinterpret_cast<ssd_u32x4_t*>(&s_b[(2 * rp) * LDB + 8 * c8]) = rb[u][0];
        *reinterpret_cast<ssd_u32x4_t*>(&s_b[(2 * rp + 1) * LDB + 8 * c8]) = rb[u][1];
        uint32_t* bt = reinterpret_cast<uint32_t*>(&s_bt[(8 * c8) * LDT + 2 * rp]);
        bt[0 * LDT / 2] = column_pair<0>(rb[u][0], rb[u][1]);
        bt[1 * LDT / 2] = column_pair<1>(rb[u][0], rb[u][1]);
        bt[2 * LDT / 2] = column_pair<2>(rb[u][0], rb[u][1]);
        bt[3 * LDT / 2] = column_pair<3>(rb[u][0], rb[u][1]);
        bt[4 * LDT / 2] = column_pair<4>(rb[u][0], rb[u][1]);
        bt[5 * LDT / 2] = column_pair<5>(rb[u][0], rb[u][1]);
        bt[6 * LDT / 2] = column_pair<6>(rb[u][0], rb[u][1]);
        bt[7 * LDT / 2] = column_pair<7>(rb[u][0], rb[u][1]);
      }
    }
#pragma unroll
    for (int u = 0; u < kCPer; ++u) {
      const int k = tid + u * T;
      if (kCPer * T == kCTasks || k < kCTasks) {
        const int c8 = k % (N / 8), i = k / (N / 8);
        *reinterpret_cast<ssd_u32x4_t*>(&s_c[i * LDB + 8 * c8]) = rc[u];
      }
    }
    {
      const int rp = tid % 32, p8 = tid / 32;
      const float w0 = __shfl(wgt, 2 * rp), w1 = __shfl(wgt, 2 * rp + 1);
      uint32_t* xt = reinterpret_cast<uint32_t*>(&s_xt[(8 * p8) * LDT + 2 * rp]);
      uint32_t* xw = reinterpret_cast<uint32_t*>(&s_xw[(8 * p8) * LDT + 2 * rp]);
#define SSD_X_COLUMN(E)                                                                  \
  xt[(E) * LDT / 2] = column_pair<E>(rx[0], rx[1]);                                      \
  xw[(E) * LDT / 2] = pack_bf16x2(bf16_elem<E>(rx[0]) * w0, bf16_elem<E>(rx[1]) * w1);
      SSD_X_COLUMN(0) SSD_X_COLUMN(1) SSD_X_COLUMN(2) SSD_X_COLUMN(3)
      SSD_X_COLUMN(4) SSD_X_COLUMN(5) SSD_X_COLUMN(6) SSD_X_COLUMN(7)
#undef SSD_X_COLUMN
    }
  };

  ssd_f32x4_t S[NT];
#pragma unroll
  for (int nb = 0; nb < NT; ++nb) S[nb] = ssd_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t nchunks = (L + Q - 1) / Q;
  using Full = std::integral_constant<bool, true>;
  using Ragged = std::integral_constant<bool, false>;
  if (nchunks > 0) {
    if (Q <= L) load_chunk(0, Full{});
    else load_chunk(0, Ragged{});
  }
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * Q;
    __syncthreads();  // every wave is done with the previous chunk's tiles
    stage_chunk(t0);
    ssd_u32x2_t zc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) zc[k] = rz[k];
    __syncthreads();
    if (c + 1 < nchunks) {
      if (t0 + 2 * Q <= L) load_chunk(t0 + Q, Full{});
      else load_chunk(t0 + Q, Ragged{});
    }
    // M, split over the waves: G^T tile (j-block jb, i-block ib) = B_j . C_i, masked to j <= i,
    // decayed and stored as M[i][j].  The masked product reads M in K = 32 steps, so besides the
    // ten tiles jb <= ib it needs the two tiles (ib, jb) = (0, 1), (2, 3) just past the diagonal,
    // which the mask zeroes.  Twelve tiles, 12 / NW per wave, in one straight-line block.
#pragma unroll
    for (int s = 0; s < 12 / NW; ++s) {
      const int k = wave + NW * s;
      const int ib = k < 4 ? k / 2 : k / 4 + 1, jb = k < 4 ? k % 2 : k % 4;
      const int irow = 16 * ib + l16;
      ssd_f32x4_t gt = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        gt = mfma16x16x32(*reinterpret_cast<const ssd_u32x4_t*>(&s_b[(16 * jb + l16) * LDB + 32 * ks + 8 * q]),
                          *reinterpret_cast<const ssd_u32x4_t*>(&s_c[irow * LDB + 32 * ks + 8 * q]), gt);
      const float cum_i = s_cum[irow];
      const ssd_f32x4_t cj = *reinterpret_cast<const ssd_f32x4_t*>(&s_cum[16 * jb + 4 * q]);
      const ssd_f32x4_t dj = *reinterpret_cast<const ssd_f32x4_t*>(&s_dt[16 * jb + 4 * q]);
      float m[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) m[r] = (16 * jb + 4 * q + r <= irow) ? gt[r] * hw_exp2(cum_i - cj[r]) * dj[r] : 0.0f;
      *reinterpret_cast<ssd_u32x2_t*>(&s_m[irow * LDT + 16 * jb + 4 * q]) =
          ssd_u32x2_t{pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3])};
    }

    // S entering the chunk as bf16 A operands of the read-out, S^T[p][n] with n permuted as the
    // tiles hold it
    ssd_u32x4_t sf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      sf[ks] = ssd_u32x4_t{pack_bf16x2(S[2 * ks][0], S[2 * ks][1]), pack_bf16x2(S[2 * ks][2], S[2 * ks][3]),
                           pack_bf16x2(S[2 * ks + 1][0], S[2 * ks + 1][1]),
                           pack_bf16x2(S[2 * ks + 1][2], S[2 * ks + 1][3])};
    __syncthreads();  // M complete

    // Y^T tiles (channels 16 wave .. +15, steps 16 ib .. +15): the read-out exp(cum_i) S^T C_i^T
    // plus the masked product X^T M^T over the steps j <= i
    ssd_f32x4_t acc[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const int irow = 16 * ib + l16;  // the output step this lane holds
      acc[ib] = ssd_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        acc[ib] = mfma16x16x32(sf[ks], load_perm_frag(&s_c[irow * LDB + 32 * ks + 4 * q]), acc[ib]);
    }
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const int irow = 16 * ib + l16;
      acc[ib] *= hw_exp2(s_cum[irow]);
#pragma unroll
      for (int ks = 0; ks <= ib / 2; ++ks)
        acc[ib] = mfma16x16x32(*reinterpret_cast<const ssd_u32x4_t*>(&s_xt[pw * LDT + 32 * ks + 8 * q]),
                               *reinterpret_cast<const ssd_u32x4_t*>(&s_m[irow * LDT + 32 * ks + 8 * q]), acc[ib]);
    }
    // skip term, gate, store: channels pe .. pe + 3 of step 16 ib + l16
    const bool full = t0 + Q <= L;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const int irow = 16 * ib + l16;
      float yv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        yv[r] = fmaf(Dh, bf16_lo(s_xt[(pe + r) * LDT + irow]), acc[ib][r]);
        if (zg) yv[r] *= silu_f32((r & 1) ? bf16_hi(zc[ib][r / 2]) : bf16_lo(zc[ib][r / 2]));
      }
      const int64_t t = t0 + irow;
      if (full || t < L)
        *reinterpret_cast<ssd_u32x2_t*>(yg + t * xs) = ssd_u32x2_t{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])};
    }

    // state update: S = exp(cum_last) S + B^T (weighted X)
    const float decay = hw_exp2(s_cum[Q - 1]);
    ssd_u32x4_t xw[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) xw[ks] = *reinterpret_cast<const ssd_u32x4_t*>(&s_xw[pw * LDT + 32 * ks + 8 * q]);
#pragma unroll
    for (int nb = 0; nb < NT; ++nb) {
      S[nb] *= decay;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        S[nb] = mfma16x16x32(*reinterpret_cast<const ssd_u32x4_t*>(&s_bt[(16 * nb + l16) * LDT + 32 * ks + 8 * q]),
                             xw[ks], S[nb]);
    }
  }

  if (p.final_state) {
    float* fs = p.final_state + ((b * H + h) * P + p0 + pw) * N + 4 * q;
#pragma unroll
    for (int nb = 0; nb < NT; ++nb) *reinterpret_cast<ssd_f32x4_t*>(fs + 16 * nb) = S[nb];
  }
}

using SsdKernel = void (*)(const SsdArgs);
// The kernel for (dstate, waves per workgroup), or NULL when that pair is not instantiated.
SsdKernel ssd_kernel(int64_t dstate, int waves);

}  // namespace ssm
