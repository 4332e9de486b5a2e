// scan_fwd.hpp -- the selective-scan forward kernels for gfx950 (wave64, 160 KB LDS per CU).
//
// The recurrence ("Mamba 论文精读" sec. 2.2 and sec. 3.3; "mamba->jamba" sec. 2.3):
//   dt_t = softplus(delta_t + bias)  (or delta_t + bias),  w_t = dt_t * x_t
//   h_t[n] = exp(dt_t A[n]) h_{t-1}[n] + w_t B_t[n],        y_t = sum_n C_t[n] h_t[n] + D x_t,
//   y_t *= silu(z_t).
//
// Work decomposition (one workgroup = 64 channels of one batch row x all N state indices,
// optionally x one segment of the sequence):
//   * wave g of the workgroup owns state indices n in [g*NPL, (g+1)*NPL) of all 64 channels;
//     lane = channel.  Its NPL states live in VGPRs for the whole sequence (never in HBM).
//     B_t[n] and C_t[n] are the same for all 64 lanes: lane k of every 16-lane row loads step
//     k of each 16-step half of the chunk, and each step takes its values with DPP row
//     broadcasts that are operands of the multiply (B_t * w) and of the read-out multiply-adds
//     (C_t * h) -- no memory access and no LDS traffic for B and C.  Each step is one fused,
//     hazard-ordered instruction block that also reads out the previous step.
//   * per chunk of CHUNK time steps, all threads of the workgroup load the x / delta / z tile
//     with coalesced vector loads (a chunk ahead, into registers), compute the per-(t, d)
//     prologue once (softplus, dt * x) into LDS, every wave runs its CHUNK steps of the
//     recurrence reading (dt, w) from LDS, writes its partial read-out sum_{n in group} C h
//     to LDS, and the same threads that loaded the tile sum the G partials, add D x, apply
//     the gate and store y with vector stores.
//   * rows past the end of the sequence and channels past `dim` are carried with
//     dt = w = B = C = 0, which makes those steps exact identities on the state (A is clamped
//     to a finite value, so exp2(0 * A) = 1); their outputs are never stored.  Every chunk
//     therefore runs all CHUNK steps, fully unrolled.
//
// Split sequence (few channels, long L): the sequence is cut into `nseg` segments of seg_len
// steps (a multiple of CHUNK).  Phase 1 (MODE_AGG) runs the recurrence of segments
// 0..nseg-2 from a zero state and stores each segment's end state H_s and its summed step
// S_s = sum dt.  Phase 2 (carry kernel) composes them in order with the scan operator
// (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2), where the segment's decay is
// a = exp(A S_s), giving every segment its incoming state.  Phase 3 (MODE_FULL) reruns
// every segment from its incoming state and writes y.
#pragma once

#include "ssm_device.hpp"

namespace ssm {

enum { MODE_FULL = 0, MODE_AGG = 1 };

struct ScanArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* z;
  const float* delta_bias;
  void* y;
  float* last_state;
  float* seg_state;  // (nseg, batch, dim, N): end state of a segment (AGG) / incoming state (FULL)
  float* seg_dsum;   // (nseg, batch, dim): summed step of a segment (AGG)
  int64_t batch;
  int64_t seqlen;
  int64_t dim;
  int64_t seg_len;   // steps per segment; == seqlen when nseg == 1
  int32_t nseg;
  int32_t ncb;       // channel blocks of 64
  int32_t softplus;
  int32_t vec_ok;    // x / delta / z / y rows allow aligned vector access
};

constexpr int kChunk = 32;
constexpr int kDwPad = 2;   // float2 padding per LDS row of (dt, w)
constexpr int kYpPad = 4;   // float padding per LDS row of partial read-outs

template <int N, int NPL>
struct ScanShape {
  static constexpr int G = N / NPL;           // waves per workgroup
  static constexpr int NT = 64 * G;           // threads per workgroup
  static constexpr int EPT = kChunk * 64 / NT;  // tile elements per thread
};

template <bool BF16, int N, int NPL, int MODE>
__global__ __launch_bounds__(64 * (N / NPL)) void scan_chunk_kernel(const ScanArgs p) {
  using Shape = ScanShape<N, NPL>;
  constexpr int G = Shape::G;
  constexpr int NT = Shape::NT;
  constexpr int EPT = Shape::EPT;
  static_assert(EPT >= 1, "chunk too small for this workgroup");
  constexpr int kMaxVec = BF16 ? 8 : 4;       // 16-byte accesses
  constexpr int VEC = EPT < kMaxVec ? EPT : kMaxVec;
  constexpr int ITEMS = EPT / VEC;
  constexpr int TPR = 64 / VEC;               // threads per tile row
  constexpr int RSTEP = NT / TPR;             // tile rows covered per pass
  static_assert(ITEMS * RSTEP == kChunk, "tile mapping must cover the chunk exactly");
  constexpr bool kFull = (MODE == MODE_FULL);

  __shared__ float2 s_dw[kChunk][64 + kDwPad];
  __shared__ float s_yp[kFull ? G : 1][kChunk][64 + kYpPad];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup -> (channel block, batch row, segment)
  const int64_t blk = blockIdx.x;
  const int cb = static_cast<int>(blk % p.ncb);
  const int64_t rest = blk / p.ncb;
  const int64_t b = rest % p.batch;
  const int seg = static_cast<int>(rest / p.batch);
  const int64_t t_begin = static_cast<int64_t>(seg) * p.seg_len;
  const int64_t t_end = (t_begin + p.seg_len < p.seqlen) ? (t_begin + p.seg_len) : p.seqlen;

  // ---- scan-side state: lane = channel, NPL chains -------------------------------------------
  const int64_t d_lane = static_cast<int64_t>(cb) * 64 + lane;
  const bool lane_ok = d_lane < p.dim;
  const int n0 = wave * NPL;
  float A2[NPL], h[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    // log2(e) * A, clamped to a finite value: a padded step (dt = 0) must give exp2(0) = 1
    A2[j] = lane_ok ? fmaxf(p.A[d_lane * N + n0 + j] * kLog2e, -3.0e38f) : 0.0f;
    h[j] = 0.0f;
  }
  if (kFull && p.nseg > 1 && lane_ok) {
    const float* hin = p.seg_state + ((static_cast<int64_t>(seg) * p.batch + b) * p.dim + d_lane) * N + n0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) h[j] = hin[j];
  }
  float dsum = 0.0f;

  // ---- tile-side mapping: (row, VEC channels) items ------------------------------------------
  const int col = (tid % TPR) * VEC;
  const int row0 = tid / TPR;
  const int64_t d_col = static_cast<int64_t>(cb) * 64 + col;
  const int nvalid_col = d_col >= p.dim ? 0 : static_cast<int>((p.dim - d_col) < VEC ? (p.dim - d_col) : VEC);
  const bool vec_ok = p.vec_ok != 0;
  float bias[VEC], dsk[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    bias[v] = (p.delta_bias && v < nvalid_col) ? p.delta_bias[d_col + v] : 0.0f;
    dsk[v] = (p.Dskip && v < nvalid_col) ? p.Dskip[d_col + v] : 0.0f;
  }
  const bool has_z = kFull && p.z != nullptr;
  const int64_t row_base = b * p.seqlen;  // (b, t) row index = row_base + t

  RawVec<BF16, VEC> nx[ITEMS], nd[ITEMS], nz[ITEMS];
  constexpr int kHalves = kChunk / 16;
  const int bc_k = lane & 15;
  BcRow<BF16, NPL> nb[kHalves], nc[kHalves];
  // loads the x / delta / z tile and the B / C rows of the chunk starting at t0 into registers;
  // `full` (uniform): every row of the chunk exists and the channel block is whole
  auto load_tile = [&](int64_t t0, bool full) {
    if (full) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int64_t idx = (row_base + t0 + row0 + i * RSTEP) * p.dim + d_col;
        nx[i].load(p.x, idx, VEC, true);
        nd[i].load(p.delta, idx, VEC, true);
        if (has_z) nz[i].load(p.z, idx, VEC, true);
      }
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) {
        const int64_t e = (row_base + t0 + hf * 16 + bc_k) * N + n0;
        nb[hf].load(p.B, e, true);
        if constexpr (kFull) nc[hf].load(p.C, e, true);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t t = t0 + row0 + i * RSTEP;
      const int nv = (t < t_end) ? nvalid_col : 0;
      const int64_t idx = (row_base + t) * p.dim + d_col;
      nx[i].load(p.x, idx, nv, vec_ok);
      nd[i].load(p.delta, idx, nv, vec_ok);
      if (has_z) nz[i].load(p.z, idx, nv, vec_ok);
    }
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) {
      const int64_t t = t0 + hf * 16 + bc_k;
      const int64_t e = (row_base + t) * N + n0;
      nb[hf].load(p.B, e, t < t_end);
      if constexpr (kFull) nc[hf].load(p.C, e, t < t_end);
    }
  };

  // whole 64-channel block valid with vector access: chunks away from the sequence end need no
  // per-element masking
  const bool full_cols = vec_ok && (static_cast<int64_t>(cb) * 64 + 64 <= p.dim);
  if (t_begin < t_end) load_tile(t_begin, full_cols && t_begin + kChunk <= t_end);

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const bool full = full_cols && (t0 + kChunk <= t_end);

    // 1. prologue of this chunk: (dt, dt * x) into LDS; keep x and z for the epilogue
    RawVec<BF16, VEC> cx[ITEMS], cz[ITEMS];
    float dts[ITEMS][VEC], xs[ITEMS][VEC];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        dts[i][v] = nd[i].get(v) + bias[v];
        xs[i][v] = nx[i].get(v);
      }
    if (p.softplus) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i)
#pragma unroll
        for (int v = 0; v < VEC; ++v) dts[i][v] = softplus_f32(dts[i][v]);
    }
    if (!full) {  // rows past the end and channels past dim become identity steps
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const bool row_ok = (t0 + row0 + i * RSTEP) < t_end;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const bool ok = row_ok && (v < nvalid_col);
          dts[i][v] = ok ? dts[i][v] : 0.0f;
          xs[i][v] = ok ? xs[i][v] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int row = row0 + i * RSTEP;
#pragma unroll
      for (int v = 0; v < VEC; ++v) s_dw[row][col + v] = make_float2(dts[i][v], dts[i][v] * xs[i][v]);
      cx[i] = nx[i];
      if (has_z) cz[i] = nz[i];
    }
    float Bv[kHalves][NPL], Cv[kHalves][NPL];
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf)
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        Bv[hf][j] = nb[hf].get(j);
        Cv[hf][j] = kFull ? nc[hf].get(j) : 0.0f;
      }
    // 2. prefetch the next chunk's tile into registers
    if (t0 + kChunk < t_end) load_tile(t0 + kChunk, full_cols && t0 + 2 * kChunk <= t_end);
    __syncthreads();

    // 3. the recurrence over this chunk: NPL chains per lane, all kChunk steps unrolled, the
    //    (dt, w) pairs of kBatch steps read from LDS ahead of their use.  In FULL mode each step
    //    t >= 1 is one fused block that also reads out step t - 1; step 31 is read out after the
    //    loop.
    constexpr int kBatch = 8;
    static_for<kChunk / kBatch>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      float2 dw[kBatch];
      static_for<kBatch>([&](auto K) { dw[decltype(K)::value] = s_dw[q * kBatch + decltype(K)::value][lane]; });
      static_for<kBatch>([&](auto K) {
        constexpr int k = decltype(K)::value;
        constexpr int t = q * kBatch + k;
        if constexpr (kFull && t > 0) {
          s_yp[wave][t - 1][lane] =
              step_readout<NPL, t % 16, (t - 1) % 16>(dw[k].x, dw[k].y, A2, Bv[t / 16], Cv[(t - 1) / 16], h);
        } else {
#pragma unroll
          for (int j = 0; j < NPL; ++j)
            h[j] = fmaf(hw_exp2(dw[k].x * A2[j]), h[j], row_bcast<t % 16>(Bv[t / 16][j]) * dw[k].y);
          if constexpr (!kFull) dsum += dw[k].x;
        }
      });
    });
    if constexpr (kFull) {
      float yp = row_bcast<15>(Cv[kHalves - 1][0]) * h[0];
#pragma unroll
      for (int j = 1; j < NPL; ++j) yp = fmaf(row_bcast<15>(Cv[kHalves - 1][j]), h[j], yp);
      s_yp[wave][kChunk - 1][lane] = yp;
    }

    // 4. one barrier: every wave is done with s_dw (the next prologue may overwrite it) and
    //    s_yp is complete.  The next chunk's first barrier orders this epilogue's
    //    reads of s_yp before the next scan's writes.
    __syncthreads();

    // 5. epilogue: y = sum of partials + D x, gated, stored with vector stores
    if constexpr (kFull) {
      float out[ITEMS][VEC];
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int row = row0 + i * RSTEP;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          float acc = s_yp[0][row][col + v];
#pragma unroll
          for (int g = 1; g < G; ++g) acc += s_yp[g][row][col + v];
          out[i][v] = fmaf(dsk[v], cx[i].get(v), acc);
        }
      }
      if (has_z) {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i)
#pragma unroll
          for (int v = 0; v < VEC; ++v) out[i][v] *= silu_f32(cz[i].get(v));
      }
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int64_t t = t0 + row0 + i * RSTEP;
        const int64_t idx = (row_base + t) * p.dim + d_col;
        if (full) {
          store_vec<BF16, VEC>(p.y, idx, out[i], VEC, true);
        } else {
          const int nv = (t < t_end) ? nvalid_col : 0;
          if (nv > 0) store_vec<BF16, VEC>(p.y, idx, out[i], nv, vec_ok);
        }
      }
    }
  }

  // ---- results --------------------------------------------------------------------------------
  if (!lane_ok) return;
  if constexpr (kFull) {
    if (p.last_state && seg == p.nseg - 1) {
      float* dst = p.last_state + (b * p.dim + d_lane) * N + n0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) dst[j] = h[j];
    }
  } else {
    float* dst = p.seg_state + ((static_cast<int64_t>(seg) * p.batch + b) * p.dim + d_lane) * N + n0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) dst[j] = h[j];
    if (wave == 0) p.seg_dsum[(static_cast<int64_t>(seg) * p.batch + b) * p.dim + d_lane] = dsum;
  }
}

// Phase 2 of the split-sequence scan: one thread per (b, d, n) composes the segment summaries
// in order.  On entry seg_state[s] holds segment s's end state from a zero start (s < nseg-1);
// on exit it holds the state entering segment s.
template <int N>
__global__ __launch_bounds__(256) void scan_carry_kernel(const ScanArgs p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_seg = p.batch * p.dim * N;
  if (i >= per_seg) return;
  const int64_t bd = i / N;
  const int n = static_cast<int>(i % N);
  const int64_t d = bd % p.dim;
  const float a2 = p.A[d * N + n] * kLog2e;
  float h = 0.0f;
  for (int s = 0; s + 1 < p.nseg; ++s) {
    const float hs = p.seg_state[s * per_seg + i];
    p.seg_state[s * per_seg + i] = h;
    h = fmaf(hw_exp2(a2 * p.seg_dsum[s * p.batch * p.dim + bd]), h, hs);
  }
  p.seg_state[static_cast<int64_t>(p.nseg - 1) * per_seg + i] = h;
}

}  // namespace ssm
