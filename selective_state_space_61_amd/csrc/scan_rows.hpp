// scan_rows.hpp -- the selective-scan forward with state rows: a scan wave holds 16 channels x all
// 16 state indices, and the per-(t, d) work runs on a SIMD of its own (gfx950, wave64).
//
// The recurrence is the one of scan_fwd.hpp ("Mamba 论文精读" sec. 2.2 and sec. 3.3;
// "mamba->jamba" sec. 2.3), computed in the same order of operations, so the two layouts give the
// same bits.  What differs is the work decomposition, chosen from two measured properties of
// MI355X:
//   * a workgroup's waves w, w+4, w+8, w+12 always share one SIMD (the SIMD the first wave lands
//     on rotates between workgroups, the grouping does not);
//   * v_exp_f32 occupies a SIMD for about 11 cycles and DPP operands keep other waves from
//     issuing beside it, so one scan wave per SIMD gets nearly all the issue a SIMD can give to
//     this instruction block; the per-(t, d) prologue and epilogue then only steal it.
// So a workgroup has 16 waves in four groups of one SIMD each: waves 3, 7, 11 (the prologue) and 15
// (the epilogue) share one SIMD, and the scan waves take the slots of the other three SIMDs
// (waves 0, 1, 2, then 4, 5, 6, ...); slots without work only take part in the barriers.
//
//   * scan wave s (S per workgroup) covers channels 16 s .. 16 s + 15 of the workgroup's 16 S:
//     lane = 16 r + k is channel k with state indices 4 r .. 4 r + 3 in VGPRs for the whole
//     sequence.  B_t and C_t of the row's four states are the same for its 16 lanes: lane k of row
//     r loads step k of each 16-step half, and each step takes them through DPP row broadcasts, as
//     in scan_fwd.hpp.  The partial read-out of each row goes to LDS, two steps per instruction.
//   * prologue waves load the x / delta / z tile two chunks ahead with 16-byte loads and write
//     (dt, dt x) for the scan waves and (x, silu(z)) for the epilogue into LDS.  They only load,
//     so their waits never cover a store.
//   * the epilogue wave sums the four row partials of a channel, adds D x, gates and stores y with
//     16-byte stores.  It only stores, so it never waits on memory.
// One barrier per chunk; (dt, dt x) and the partials are double-buffered, (x, silu(z)) lives two
// iterations and is triple-buffered.  Rows past the sequence and channels past dim carry
// dt = dt x = 0, B = C = 0: exact identity steps whose outputs are never stored.
#pragma once

#include "scan_fwd.hpp"
#include "scan_rows_table.hpp"

namespace ssm {

constexpr int kRowsPrologueWaves = 3;  // waves 3, 7, 11; wave 15 is the epilogue
constexpr int kRowsMaxS = 12;          // scan slots: waves with (w & 3) != 3

// float2 per LDS row of (dt, dt x): padded to a multiple of 64 so that rows are a multiple of 512
// bytes apart and a scan wave reads two steps with one ds_read2st64_b64
constexpr int rows_dw_stride(int S) { return 64 * ((S + 3) / 4); }

constexpr int rows_lds_bytes(int S, int ch) {
  return 2 * ch * rows_dw_stride(S) * 8  // (dt, dt x), double-buffered
         + 2 * S * ch * 64 * 4           // partial read-outs of the state rows, double-buffered
         + 3 * ch * 16 * S * 8;          // (x, silu z), triple-buffered
}

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, workgroups dealt round robin

// Logical workgroup index for hardware index i of n: the first n - n % 8 workgroups are regrouped
// so that the hardware indices i with i % 8 == x (one XCD) take logical indices x * (n / 8) ..
// (x + 1) * (n / 8) - 1; the last n % 8 keep their index.  A bijection on [0, n).
__device__ __forceinline__ int64_t xcd_local(int64_t i, int64_t n) {
  const int64_t per = n / kXcds;
  if (i >= per * kXcds) return i;
  return (i % kXcds) * per + i / kXcds;
}

template <bool BF16, int S, int CH>
__global__ __launch_bounds__(64 * kRowsWaves) void scan_rows_kernel(const ScanArgs p) {
  constexpr int N = 16, NPL = 4;
  constexpr int CW = 16 * S;                 // channels per workgroup
  constexpr int DWS = rows_dw_stride(S);
  static_assert(S >= 1 && S <= kRowsMaxS, "scan waves per workgroup");
  static_assert(CH == 16 || CH == 32, "chunks of 16 or 32 steps");
  static_assert(rows_lds_bytes(S, CH) <= kLdsBudget, "LDS tiles exceed a workgroup's share");
  constexpr int kHalves = CH / 16;
  constexpr int VEC = BF16 ? 8 : 4;          // 16-byte pieces of a tile row
  constexpr int PPR = CW / VEC;              // pieces per tile row
  static_assert(CW % VEC == 0, "whole pieces per row");
  constexpr int PIECES = CH * PPR;
  constexpr int PT = 64 * kRowsPrologueWaves;
  constexpr int ITEMS = (PIECES + PT - 1) / PT;  // pieces per prologue thread
  constexpr int EITEMS = (PIECES + 63) / 64;     // pieces per epilogue thread

  __shared__ float2 s_dw[2][CH][DWS];
  __shared__ float s_yp[2][S][CH][64];
  __shared__ float2 s_xz[3][CH][CW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Workgroups are dispatched to the 8 XCDs (each with its own L2) round robin.  A 16 S-channel
  // block's rows are not whole 128-byte lines, so neighbouring channel blocks share lines: the
  // logical index is permuted so that consecutive logical blocks (neighbours in a batch row)
  // land on the same XCD and share its L2 instead of fetching each line twice.
  const int64_t blk = xcd_local(blockIdx.x, gridDim.x);
  const int cb = static_cast<int>(blk % p.ncb);
  const int64_t b = blk / p.ncb;
  const int64_t t_end = p.seqlen;
  const int64_t nchunks = (t_end + CH - 1) / CH;
  const int64_t row_base = b * p.seqlen;
  const int64_t d_base = static_cast<int64_t>(cb) * CW;
  const bool vec_ok = p.vec_ok != 0;
  const bool full_cols = vec_ok && d_base + CW <= p.dim;
  auto chunk_full = [&](int64_t c) { return full_cols && (c + 1) * CH <= t_end; };

  const int group = wave & 3;
  if (group != 3) {
    const int s = (wave >> 2) * 3 + group;
    if (s >= S) {  // a slot without work: only the barriers
      for (int64_t j = -1; j <= nchunks; ++j) __syncthreads();
      return;
    }
    // =============================== scan role ===================================================
    const int r = lane >> 4, k = lane & 15;
    const int64_t d = d_base + 16 * s + k;
    const bool lane_ok = d < p.dim;
    const int n0 = 4 * r;
    float A2[NPL], h[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      A2[j] = lane_ok ? fmaxf(p.A[d * N + n0 + j] * kLog2e, -3.0e38f) : 0.0f;
      h[j] = 0.0f;
    }
    BcRow<BF16, NPL> nb[kHalves], nc[kHalves];
    auto load_bc = [&](int64_t c) {
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) {
        const int64_t t = c * CH + hf * 16 + k;
        const int64_t e = (row_base + t) * N + n0;
        nb[hf].load(p.B, e, t < t_end);
        nc[hf].load(p.C, e, t < t_end);
      }
    };
    if (nchunks > 0) load_bc(0);
    const int col = 16 * s + k;
    for (int64_t j = -1; j <= nchunks; ++j) {
      if (j >= 0 && j < nchunks) {
        const int sb = static_cast<int>(j & 1);
        float Bv[kHalves][NPL], Cv[kHalves][NPL];
#pragma unroll
        for (int hf = 0; hf < kHalves; ++hf)
#pragma unroll
          for (int jj = 0; jj < NPL; ++jj) {
            Bv[hf][jj] = nb[hf].get(jj);
            Cv[hf][jj] = nc[hf].get(jj);
          }
        if (j + 1 < nchunks) load_bc(j + 1);
        constexpr int kBatch = 8;
        float2 dwq[2][kBatch];
        float ypp = 0.0f;  // read-out of the even step, written with the odd one
        static_for<kBatch>([&](auto K) { dwq[0][decltype(K)::value] = s_dw[sb][decltype(K)::value][col]; });
        static_for<CH / kBatch>([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          if constexpr (q + 1 < CH / kBatch)
            static_for<kBatch>([&](auto K) {
              dwq[(q + 1) & 1][decltype(K)::value] = s_dw[sb][(q + 1) * kBatch + decltype(K)::value][col];
            });
          float2* dw = dwq[q & 1];
          static_for<kBatch>([&](auto K) {
            constexpr int kk = decltype(K)::value;
            constexpr int t = q * kBatch + kk;
            if constexpr (t > 0) {
              const float yp =
                  step_readout<NPL, t % 16, (t - 1) % 16>(dw[kk].x, dw[kk].y, A2, Bv[t / 16], Cv[(t - 1) / 16], h);
              if constexpr ((t - 1) % 2 == 0) {
                ypp = yp;
              } else {
                s_yp[sb][s][t - 2][lane] = ypp;
                s_yp[sb][s][t - 1][lane] = yp;
              }
            } else {
#pragma unroll
              for (int jj = 0; jj < NPL; ++jj)
                h[jj] = fmaf(hw_exp2(dw[kk].x * A2[jj]), h[jj], row_bcast<0>(Bv[0][jj]) * dw[kk].y);
            }
          });
        });
        float yp = row_bcast<15>(Cv[kHalves - 1][0]) * h[0];
#pragma unroll
        for (int jj = 1; jj < NPL; ++jj) yp = fmaf(row_bcast<15>(Cv[kHalves - 1][jj]), h[jj], yp);
        s_yp[sb][s][CH - 2][lane] = ypp;
        s_yp[sb][s][CH - 1][lane] = yp;
      }
      __syncthreads();
    }
    if (lane_ok && p.last_state) {
      float* dst = p.last_state + (b * p.dim + d) * N + n0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) dst[j] = h[j];
    }
    return;
  }

  const int io = wave >> 2;
  if (io < kRowsPrologueWaves) {
    // =============================== prologue role ===============================================
    const int pt = io * 64 + lane;
    int prow[ITEMS], pcol[ITEMS], pnv[ITEMS];
    bool pon[ITEMS];
    float bias[ITEMS][VEC];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int piece = pt + i * PT;
      pon[i] = piece < PIECES;
      prow[i] = pon[i] ? piece / PPR : 0;
      pcol[i] = pon[i] ? (piece % PPR) * VEC : 0;
      const int64_t dc = d_base + pcol[i];
      pnv[i] = (!pon[i] || dc >= p.dim) ? 0 : static_cast<int>((p.dim - dc) < VEC ? (p.dim - dc) : VEC);
#pragma unroll
      for (int v = 0; v < VEC; ++v) bias[i][v] = (p.delta_bias && v < pnv[i]) ? p.delta_bias[dc + v] : 0.0f;
    }
    const bool has_z = p.z != nullptr;
    RawVec<BF16, VEC> nx[2][ITEMS], nd[2][ITEMS], nz[2][ITEMS];
    auto load_tile = [&](int64_t c, auto SL) {
      constexpr int sl = decltype(SL)::value;
      const int64_t t0 = c * CH;
      const bool full = chunk_full(c);
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int64_t t = t0 + prow[i];
        const int nv = (t < t_end) ? pnv[i] : 0;
        const int64_t idx = (row_base + t) * p.dim + d_base + pcol[i];
        if (full && pon[i]) {
          nx[sl][i].load(p.x, idx, VEC, true);
          nd[sl][i].load(p.delta, idx, VEC, true);
          if (has_z) nz[sl][i].load(p.z, idx, VEC, true);
        } else {
          nx[sl][i].load(p.x, idx, nv, vec_ok);
          nd[sl][i].load(p.delta, idx, nv, vec_ok);
          if (has_z) nz[sl][i].load(p.z, idx, nv, vec_ok);
        }
      }
    };
    using Slot0 = std::integral_constant<int, 0>;
    using Slot1 = std::integral_constant<int, 1>;
    if (nchunks > 0) load_tile(0, Slot0{});
    if (nchunks > 1) load_tile(1, Slot1{});
    // iteration j: prologue of chunk j+1 from slot (j+1) & 1, then the tile of chunk j+3 into it
    auto iteration = [&](int64_t j, auto SL) {
      constexpr int sl = decltype(SL)::value;
      const int64_t c = j + 1;
      if (c < nchunks) {
        const int pb = static_cast<int>(c & 1);
        const int xb = static_cast<int>(c % 3);
        const bool full = chunk_full(c);
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
          if (!pon[i]) continue;
          const bool row_ok = full || (c * CH + prow[i] < t_end);
          float dts[VEC], xs[VEC], sz[VEC];
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            dts[v] = nd[sl][i].get(v) + bias[i][v];
            xs[v] = nx[sl][i].get(v);
          }
          if (p.softplus) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) dts[v] = softplus_f32(dts[v]);
          }
          if (has_z) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) sz[v] = silu_f32(nz[sl][i].get(v));
          } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) sz[v] = 1.0f;
          }
          if (!full) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              const bool ok = row_ok && v < pnv[i];
              dts[v] = ok ? dts[v] : 0.0f;
              xs[v] = ok ? xs[v] : 0.0f;
            }
          }
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            s_dw[pb][prow[i]][pcol[i] + v] = make_float2(dts[v], dts[v] * xs[v]);
            s_xz[xb][prow[i]][pcol[i] + v] = make_float2(xs[v], sz[v]);
          }
        }
      }
      if (c + 2 < nchunks) load_tile(c + 2, SL);
      __syncthreads();
    };
    for (int64_t j = -1; j <= nchunks; j += 2) {
      iteration(j, Slot0{});
      if (j + 1 <= nchunks) iteration(j + 1, Slot1{});
    }
    return;
  }

  // =============================== epilogue role =================================================
  int erow[EITEMS], ecol[EITEMS], env[EITEMS];
  bool eon[EITEMS];
  float dsk[EITEMS][VEC];
#pragma unroll
  for (int i = 0; i < EITEMS; ++i) {
    const int piece = lane + i * 64;
    eon[i] = piece < PIECES;
    erow[i] = eon[i] ? piece / PPR : 0;
    ecol[i] = eon[i] ? (piece % PPR) * VEC : 0;
    const int64_t dc = d_base + ecol[i];
    env[i] = (!eon[i] || dc >= p.dim) ? 0 : static_cast<int>((p.dim - dc) < VEC ? (p.dim - dc) : VEC);
#pragma unroll
    for (int v = 0; v < VEC; ++v) dsk[i][v] = (p.Dskip && v < env[i]) ? p.Dskip[dc + v] : 0.0f;
  }
  for (int64_t j = -1; j <= nchunks; ++j) {
    const int64_t e = j - 1;
    if (e >= 0) {
      const int yb = static_cast<int>(e & 1);
      const int xb = static_cast<int>(e % 3);
      const bool full = chunk_full(e);
#pragma unroll
      for (int i = 0; i < EITEMS; ++i) {
        if (!eon[i]) continue;
        const int sw = ecol[i] / 16, k0 = ecol[i] % 16;
        float out[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          float acc = s_yp[yb][sw][erow[i]][k0 + v];
#pragma unroll
          for (int rr = 1; rr < 4; ++rr) acc += s_yp[yb][sw][erow[i]][16 * rr + k0 + v];
          const float2 xz = s_xz[xb][erow[i]][ecol[i] + v];
          out[v] = fmaf(dsk[i][v], xz.x, acc) * xz.y;
        }
        const int64_t t = e * CH + erow[i];
        const int64_t idx = (row_base + t) * p.dim + d_base + ecol[i];
        if (full) {
          store_vec<BF16, VEC>(p.y, idx, out, VEC, true);
        } else {
          const int nv = (t < t_end) ? env[i] : 0;
          if (nv > 0) store_vec<BF16, VEC>(p.y, idx, out, nv, vec_ok);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace ssm
