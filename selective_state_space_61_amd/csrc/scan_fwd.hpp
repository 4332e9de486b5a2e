// scan_fwd.hpp -- the selective-scan forward kernels for gfx950 (wave64, 160 KB LDS per CU).
//
// The recurrence ("Mamba 论文精读" sec. 2.2 and sec. 3.3; "mamba->jamba" sec. 2.3):
//   dt_t = softplus(delta_t + bias)  (or delta_t + bias),  w_t = dt_t * x_t
//   h_t[n] = exp(dt_t A[n]) h_{t-1}[n] + w_t B_t[n],        y_t = sum_n C_t[n] h_t[n] + D x_t,
//   y_t *= silu(z_t).
//
// Work decomposition (one workgroup = 64 channels of one batch row x all N state indices,
// optionally x one segment of the sequence), with two kinds of waves:
//   * scan wave g (G = N / NPL of them) owns state indices n in [g*NPL, (g+1)*NPL) of all 64
//     channels; lane = channel.  Its NPL states live in VGPRs for the whole sequence (never in
//     HBM), and it does nothing but the recurrence and the read-out.
//     B_t[n] and C_t[n] are the same for all 64 lanes: lane k of every 16-lane row loads step
//     k of each 16-step half of the chunk, and each step takes its values with DPP row
//     broadcasts that are operands of the multiply (B_t * w) and of the read-out multiply-adds
//     (C_t * h) -- no memory access and no LDS traffic for B and C.  Each step is one fused,
//     hazard-ordered instruction block that also reads out the previous step.
//   * kIoWaves IO waves, per chunk of CH time steps: they load the x / delta / z tile with
//     coalesced 16-byte loads (two chunks ahead, into registers), compute the per-(t, d)
//     prologue once (softplus, dt * x) into LDS for the scan waves, and, for the chunk the scan
//     waves finished one iteration earlier, sum the G partial read-outs sum_{n in group} C h
//     that those left in LDS, add D x, apply the gate and store y with 16-byte stores.  One
//     barrier per chunk separates the roles; every LDS buffer is double-buffered across it.
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
  float* ckpt;       // (batch, ceil(seqlen / 32), dim, N): the state entering every 32nd step, or NULL
                     // (state rows only)
  int64_t batch;
  int64_t seqlen;
  int64_t dim;
  int64_t seg_len;   // steps per segment; == seqlen when nseg == 1
  int32_t nseg;
  int32_t ncb;       // channel blocks of 64
  int32_t softplus;
  int32_t vec_ok;    // x / delta / z / y rows allow aligned vector access
};

constexpr int kChunk = 32;  // segment lengths are multiples of this (and so of every chunk size)
constexpr int kIoWaves = 4; // waves per workgroup that load, prologue, epilogue and store
// LDS rows are unpadded: every access to them is a whole 64-lane row (a scan wave's step) or a
// contiguous run of one row (an IO thread's 16-byte pieces), so padding buys no bank spread.
// Rows 512 bytes apart let a scan wave read two steps' (dt, dt x) with one ds_read2st64_b64
// whose immediate offsets reach every step of a chunk (no per-pair address arithmetic).
constexpr int kDwPad = 0;   // float2 padding per LDS row of (dt, w)
constexpr int kYpPad = 0;   // float padding per LDS row of partial read-outs

// LDS bytes of one workgroup: double-buffered (dt, dt x) tiles, plus (full scan only) the
// double-buffered partial read-outs of the G scan waves.
constexpr int scan_lds_bytes(int G, bool full, int ch) {
  return ch * (2 * (64 + kDwPad) * 8 + (full ? 2 * G * (64 + kYpPad) * 4 : 0));
}
constexpr int kLdsBudget = 160 * 1024;

// ZOH: exact zero-order-hold input term (zoh_factor) instead of Delta B.  That form runs as
// compiler-scheduled code and reads out each step in the step itself.
template <bool BF16, int N, int NPL, int MODE, int CH, bool ZOH = false>
__global__ __launch_bounds__(64 * (N / NPL + kIoWaves)) void scan_chunk_kernel(const ScanArgs p) {
  constexpr int G = N / NPL;                   // scan waves
  constexpr bool kFull = (MODE == MODE_FULL);
  static_assert(CH == 16 || CH == 32, "chunks of 16 or 32 steps");
  static_assert(scan_lds_bytes(G, kFull, CH) <= kLdsBudget, "LDS tiles exceed a workgroup's share");
  constexpr int kHalves = CH / 16;
  constexpr int IOT = 64 * kIoWaves;           // IO threads
  constexpr int EPT = CH * 64 / IOT;           // tile elements per IO thread
  constexpr int kMaxVec = BF16 ? 8 : 4;        // 16-byte accesses
  constexpr int VEC = EPT < kMaxVec ? EPT : kMaxVec;
  constexpr int ITEMS = EPT / VEC;
  constexpr int TPR = 64 / VEC;                // IO threads per tile row
  constexpr int RSTEP = IOT / TPR;             // tile rows covered per pass
  static_assert(EPT >= 1 && ITEMS * RSTEP == CH, "tile mapping must cover the chunk exactly");

  // double buffers: chunk c uses s_dw[c & 1] and s_yp[c & 1]
  __shared__ float2 s_dw[2][CH][64 + kDwPad];
  __shared__ float s_yp[kFull ? 2 : 1][kFull ? G : 1][CH][64 + kYpPad];

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
  const int64_t nchunks = (t_end - t_begin + CH - 1) / CH;
  const int64_t row_base = b * p.seqlen;  // (b, t) row index = row_base + t
  const bool vec_ok = p.vec_ok != 0;
  // whole 64-channel block valid with vector access, and chunk c entirely inside the sequence
  const bool full_cols = vec_ok && (static_cast<int64_t>(cb) * 64 + 64 <= p.dim);
  auto chunk_full = [&](int64_t c) { return full_cols && t_begin + (c + 1) * CH <= t_end; };

  // Both roles run nchunks + 2 iterations (j = -1 .. nchunks) with one barrier each:
  //   IO waves:   epilogue of chunk j-1 <- s_yp[(j-1) & 1];  prologue of chunk j+1 -> s_dw[(j+1) & 1]
  //   scan waves: recurrence of chunk j:  s_dw[j & 1] -> s_yp[j & 1]
  // Every buffer is written in one iteration, read in the next and rewritten in the one after,
  // each time across a barrier.
  if (wave < G) {
    // ================================ scan role ================================================
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

    // B / C rows: lane k of each 16-lane row holds step k of each 16-step half of a chunk
    const int bc_k = lane & 15;
    BcRow<BF16, NPL> nb[kHalves], nc[kHalves];
    auto load_bc = [&](int64_t c) {
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) {
        const int64_t t = t_begin + c * CH + hf * 16 + bc_k;
        const int64_t e = (row_base + t) * N + n0;
        nb[hf].load(p.B, e, t < t_end);
        if constexpr (kFull) nc[hf].load(p.C, e, t < t_end);
      }
    };
    if (nchunks > 0) load_bc(0);

    for (int64_t j = -1; j <= nchunks; ++j) {
      if (j >= 0 && j < nchunks) {
        const int sb = static_cast<int>(j & 1);
        float Bv[kHalves][NPL], Cv[kHalves][NPL];
#pragma unroll
        for (int hf = 0; hf < kHalves; ++hf)
#pragma unroll
          for (int jj = 0; jj < NPL; ++jj) {
            Bv[hf][jj] = nb[hf].get(jj);
            Cv[hf][jj] = kFull ? nc[hf].get(jj) : 0.0f;
          }
        if (j + 1 < nchunks) load_bc(j + 1);
        // CH steps unrolled; each step t >= 1 is one fused block that also reads out step t-1,
        // step CH-1 is read out at the end
        // (dt, w) of the next batch of steps is read from LDS while the current batch computes
        constexpr int kBatch = 8;
        float2 dwq[2][kBatch];
        static_for<kBatch>([&](auto K) { dwq[0][decltype(K)::value] = s_dw[sb][decltype(K)::value][lane]; });
        static_for<CH / kBatch>([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          if constexpr (q + 1 < CH / kBatch)
            static_for<kBatch>([&](auto K) {
              dwq[(q + 1) & 1][decltype(K)::value] = s_dw[sb][(q + 1) * kBatch + decltype(K)::value][lane];
            });
          float2* dw = dwq[q & 1];
          static_for<kBatch>([&](auto K) {
            constexpr int k = decltype(K)::value;
            constexpr int t = q * kBatch + k;
            if constexpr (ZOH) {
              float yp = 0.0f;
#pragma unroll
              for (int jj = 0; jj < NPL; ++jj) {
                const float tt = dw[k].x * A2[jj];
                const float a = hw_exp2(tt);
                h[jj] = fmaf(a, h[jj], row_bcast<t % 16>(Bv[t / 16][jj]) * (dw[k].y * zoh_factor(tt, a)));
                if constexpr (kFull) yp = fmaf(row_bcast<t % 16>(Cv[t / 16][jj]), h[jj], yp);
              }
              if constexpr (kFull) s_yp[sb][wave][t][lane] = yp;
              else dsum += dw[k].x;
            } else if constexpr (kFull && t > 0) {
              s_yp[sb][wave][t - 1][lane] =
                  step_readout<NPL, t % 16, (t - 1) % 16>(dw[k].x, dw[k].y, A2, Bv[t / 16], Cv[(t - 1) / 16], h);
            } else {
#pragma unroll
              for (int jj = 0; jj < NPL; ++jj)
                h[jj] = fmaf(hw_exp2(dw[k].x * A2[jj]), h[jj], row_bcast<t % 16>(Bv[t / 16][jj]) * dw[k].y);
              if constexpr (!kFull) dsum += dw[k].x;
            }
          });
        });
        if constexpr (kFull && !ZOH) {
          float yp = row_bcast<15>(Cv[kHalves - 1][0]) * h[0];
#pragma unroll
          for (int jj = 1; jj < NPL; ++jj) yp = fmaf(row_bcast<15>(Cv[kHalves - 1][jj]), h[jj], yp);
          s_yp[sb][wave][CH - 1][lane] = yp;
        }
      }
      __syncthreads();
    }

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
    return;
  }

  // ================================== IO role ===================================================
  const int iot = tid - 64 * G;
  const int col = (iot % TPR) * VEC;
  const int row0 = iot / TPR;
  const int64_t d_col = static_cast<int64_t>(cb) * 64 + col;
  const int nvalid_col = d_col >= p.dim ? 0 : static_cast<int>((p.dim - d_col) < VEC ? (p.dim - d_col) : VEC);
  float bias[VEC], dsk[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    bias[v] = (p.delta_bias && v < nvalid_col) ? p.delta_bias[d_col + v] : 0.0f;
    dsk[v] = (p.Dskip && v < nvalid_col) ? p.Dskip[d_col + v] : 0.0f;
  }
  const bool has_z = kFull && p.z != nullptr;
  // without a gate the z tile is read from x (always valid) and never used: a load that runs on
  // every path keeps the tile registers free of merges, whose copies would wait for the load
  const void* zsrc = has_z ? p.z : p.x;

  // tiles of the next two chunks to enter the prologue: chunk c sits in slot c & 1 and is loaded
  // two iterations before its prologue (the compiler's wait before a prologue counts every
  // outstanding load, so it also covers the newer tile; the two slots still measured faster than
  // one, with fixed registers instead of a rotation per iteration)
  RawVec<BF16, VEC> nx[2][ITEMS], nd[2][ITEMS], nz[2][ITEMS];
  // loads the x / delta / z tile of chunk c into slot S
  auto load_tile = [&](int64_t c, auto S) {
    constexpr int sl = decltype(S)::value;
    const int64_t t0 = t_begin + c * CH;
    if (chunk_full(c)) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int64_t idx = (row_base + t0 + row0 + i * RSTEP) * p.dim + d_col;
        nx[sl][i].load(p.x, idx, VEC, true);
        nd[sl][i].load(p.delta, idx, VEC, true);
        nz[sl][i].load(zsrc, idx, VEC, true);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t t = t0 + row0 + i * RSTEP;
      const int nv = (t < t_end) ? nvalid_col : 0;
      const int64_t idx = (row_base + t) * p.dim + d_col;
      nx[sl][i].load(p.x, idx, nv, vec_ok);
      nd[sl][i].load(p.delta, idx, nv, vec_ok);
      nz[sl][i].load(zsrc, idx, nv, vec_ok);
    }
  };
  using Slot0 = std::integral_constant<int, 0>;
  using Slot1 = std::integral_constant<int, 1>;
  if (nchunks > 0) load_tile(0, Slot0{});
  if (nchunks > 1) load_tile(1, Slot1{});

  // x and z of the chunks between prologue and epilogue: at the top of iteration j, [0] holds
  // chunk j (prologued in iteration j-1) and [1] chunk j-1 (its epilogue runs now)
  RawVec<BF16, VEC> ex[2][ITEMS], ez[2][ITEMS];
  // Order inside an iteration: epilogue arithmetic, prologue, the loads of a later tile, and
  // last the y stores.  Vector-memory completions are counted in issue order, so any wait for a
  // load also waits for every store issued before it; in this order no wait in the loop covers a
  // store issued in the same iteration, where storing first cost a full write round trip on
  // every chunk.  Iteration j works on slot (j + 1) & 1, so the loop is unrolled by two.
  auto iteration = [&](int64_t j, auto S) {
    constexpr int sl = decltype(S)::value;
    // ---- epilogue of chunk j-1, arithmetic: y = sum of partials + D x, gated ------------------
    const int64_t e = j - 1;
    const bool epi = kFull && e >= 0;
    [[maybe_unused]] float out[ITEMS][VEC];
    if constexpr (kFull) {
      if (epi) {
        const int eb = static_cast<int>(e & 1);
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
          const int row = row0 + i * RSTEP;
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            float acc = s_yp[eb][0][row][col + v];
#pragma unroll
            for (int g = 1; g < G; ++g) acc += s_yp[eb][g][row][col + v];
            out[i][v] = fmaf(dsk[v], ex[1][i].get(v), acc);
          }
        }
        if (has_z) {
#pragma unroll
          for (int i = 0; i < ITEMS; ++i)
#pragma unroll
            for (int v = 0; v < VEC; ++v) out[i][v] *= silu_f32(ez[1][i].get(v));
        }
      }
    }
    // ---- prologue of chunk j+1 ----------------------------------------------------------------
    const int64_t c = j + 1;
    if (c < nchunks) {
      const int pb = static_cast<int>(c & 1);
      const int64_t t0 = t_begin + c * CH;
      float dts[ITEMS][VEC], xs[ITEMS][VEC];
#pragma unroll
      for (int i = 0; i < ITEMS; ++i)
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          dts[i][v] = nd[sl][i].get(v) + bias[v];
          xs[i][v] = nx[sl][i].get(v);
        }
      if (p.softplus) {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i)
#pragma unroll
          for (int v = 0; v < VEC; ++v) dts[i][v] = softplus_f32(dts[i][v]);
      }
      if (!chunk_full(c)) {  // rows past the end and channels past dim become identity steps
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
        for (int v = 0; v < VEC; ++v)  // ZOH: the scan multiplies by ln2 phi, so w carries log2(e)
          s_dw[pb][row][col + v] = make_float2(dts[i][v], dts[i][v] * (ZOH ? xs[i][v] * kLog2e : xs[i][v]));
        ex[1][i] = ex[0][i];
        ex[0][i] = nx[sl][i];
        ez[1][i] = ez[0][i];
        ez[0][i] = nz[sl][i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        ex[1][i] = ex[0][i];
        ez[1][i] = ez[0][i];
      }
    }
    // ---- tile of chunk j+3, into the slot the prologue just freed -----------------------------
    if (c + 2 < nchunks) load_tile(c + 2, S);
    // ---- epilogue of chunk j-1, stores --------------------------------------------------------
    if constexpr (kFull) {
      if (epi) {
        const int64_t t0 = t_begin + e * CH;
        const bool full = chunk_full(e);
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

    __syncthreads();
  };
  for (int64_t j = -1; j <= nchunks; j += 2) {
    iteration(j, Slot0{});
    if (j + 1 <= nchunks) iteration(j + 1, Slot1{});
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
  const int64_t per_sum = p.batch * p.dim;
  const int last = p.nseg - 1;  // segments 0 .. nseg-2 have summaries
  float h = 0.0f;
  // the summaries of kCarryBatch segments are loaded before any of them is composed, so their
  // loads overlap instead of costing one memory round trip per segment
  constexpr int kCarryBatch = 8;
  int s = 0;
  for (; s + kCarryBatch <= last; s += kCarryBatch) {
    float hs[kCarryBatch], ds[kCarryBatch];
#pragma unroll
    for (int u = 0; u < kCarryBatch; ++u) {
      hs[u] = p.seg_state[(s + u) * per_seg + i];
      ds[u] = p.seg_dsum[(s + u) * per_sum + bd];
    }
#pragma unroll
    for (int u = 0; u < kCarryBatch; ++u) {
      p.seg_state[(s + u) * per_seg + i] = h;
      h = fmaf(hw_exp2(a2 * ds[u]), h, hs[u]);
    }
  }
  for (; s < last; ++s) {
    const float hs = p.seg_state[s * per_seg + i];
    p.seg_state[s * per_seg + i] = h;
    h = fmaf(hw_exp2(a2 * p.seg_dsum[s * per_sum + bd]), h, hs);
  }
  p.seg_state[static_cast<int64_t>(last) * per_seg + i] = h;
}

}  // namespace ssm
