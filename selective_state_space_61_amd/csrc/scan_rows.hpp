// scan_rows.hpp -- the selective-scan forward with state rows: a scan wave holds 16 channels x all
// 16 state indices, and the per-(t, d) work runs on a SIMD of its own (gfx950, wave64).
//
// The recurrence is the one of scan_fwd.hpp ("Mamba 论文精读" sec. 2.2 and sec. 3.3;
// "mamba->jamba" sec. 2.3), computed in the same order of operations, so the two layouts give the
// same bits.  What differs is the work decomposition, chosen from measured properties of MI355X:
//   * a workgroup's waves w, w+4, w+8, w+12 always share one SIMD (the SIMD the first wave lands
//     on rotates between workgroups, the grouping does not);
//   * v_exp_f32 occupies a SIMD for about 11 cycles and DPP operands keep other waves from
//     issuing beside it, so one scan wave per SIMD gets nearly all the issue a SIMD can give to
//     this instruction block; other waves on its SIMD only steal it.
// So a workgroup has 16 waves in four groups of one SIMD each.  Waves 3, 7, 11 (the prologue) and
// 15 (the epilogue) share one SIMD; the scan waves take the slots of the other three SIMDs (slot
// k = wave (k / 3) * 4 + k % 3: waves 0, 1, 2, then 4, 5, 6, ...); slot S holds the B / C
// stager (with three scan waves, slots 3 and 4: B on one, C on the other); the other slots only
// take part in the barriers.
//
//   * scan wave s (S per workgroup) covers channels 16 s .. 16 s + 15 of the workgroup's 16 S:
//     lane = 16 r + k is channel k with state indices 4 r .. 4 r + 3 in VGPRs for the whole
//     sequence.  B_t and C_t of the row's four states are the same for its 16 lanes: lane k of row
//     r reads step k of each 16-step half from LDS, and each step takes them through DPP row
//     broadcasts, as in scan_fwd.hpp.  The partial read-out of each row goes to LDS, two steps per
//     instruction.  The wave makes no global memory access inside the sequence loop.
//   * prologue waves load the x / delta / z tile of a chunk two iterations before they use it,
//     with 16-byte loads, and write (dt, dt x) for the scan waves and (x, silu(z)) for the
//     epilogue into LDS, two chunks ahead of the scan.  They only load.
//   * the stager loads the B and C rows of a chunk one iteration before it widens them to fp32
//     in LDS, two chunks ahead of the scan: a few instructions per chunk.
//   * the epilogue wave sums the four row partials of a channel, adds D x, gates and stores y with
//     16-byte stores.  It only stores, so it never waits on memory.
// Every loop issues the same loads on every path (rows past the sequence read the last row and
// are zeroed when used) and takes in the loaded registers on every path, so the compiler's waits
// before a use count only the loads that use needs: the tiles in flight stay in flight.
// One barrier per chunk.  Because the staging runs two chunks ahead, a scan wave reads the first
// (dt, dt x) batch and the first B / C rows of its next chunk during its last batch of steps, and
// after the barrier it goes straight into the steps.  (dt, dt x) and B / C live three iterations
// (triple-buffered), (x, silu(z)) four, the partials two.
// Rows past the sequence and channels past dim carry dt = dt x = 0, B = C = 0: exact identity
// steps whose outputs are never stored.
#pragma once

#include "scan_fwd.hpp"
#include "scan_rows_table.hpp"

namespace ssm {

constexpr int kRowsMaxS = 12;  // slots of scan and epilogue waves: waves with (w & 3) != 3

constexpr int kRowsPrologueWaves = 3;  // waves 3, 7, 11 (wave 15, on the same SIMD: the epilogue)


// float2 per LDS row of (dt, dt x): padded to a multiple of 64 so that rows are a multiple of 512
// bytes apart and a scan wave reads two steps with one ds_read2st64_b64
constexpr int rows_dw_stride(int S) { return 64 * ((S + 3) / 4); }

constexpr int kRowsDwBufs = 3;  // (dt, dt x), B, C: written in iteration c - 2, read in c - 1 and c
constexpr int kRowsXzBufs = 4;  // (x, silu z): written in iteration c - 2, read in c + 1

constexpr int rows_lds_bytes(int S, int ch) {
  return kRowsDwBufs * ch * rows_dw_stride(S) * 8  // (dt, dt x)
         + kRowsDwBufs * 2 * ch * 16 * 4           // B_t, C_t
         + 2 * S * ch * 64 * 4                     // partial read-outs of the state rows, double-buffered
         + kRowsXzBufs * ch * 16 * S * 8           // (x, silu z)
         + 16 * S * 4;                             // D
}

template <bool BF16, int S, int CH>
__global__ __launch_bounds__(64 * kRowsWaves) void scan_rows_kernel(const ScanArgs p) {
  constexpr int N = 16, NPL = 4;
  constexpr int CW = 16 * S;                 // channels per workgroup
  constexpr int DWS = rows_dw_stride(S);
  static_assert(S >= 1 && S < kRowsMaxS, "scan waves and the stager per workgroup");
  static_assert(CH * (BF16 ? 8 : 16) % 64 == 0, "whole B / C words per stager lane");
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

  __shared__ float2 s_dw[kRowsDwBufs][CH][DWS];
  __shared__ float s_bc[kRowsDwBufs][2][CH][16];  // B_t, C_t (fp32) of each step of a chunk
  __shared__ float s_yp[2][S][CH][64];
  __shared__ float2 s_xz[kRowsXzBufs][CH][CW];
  __shared__ float s_dsk[CW];

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
  if (t_end <= 0) return;  // (the host never launches an empty sequence; the loads below need a row)
  const int64_t nchunks = (t_end + CH - 1) / CH;
  const int64_t row_base = b * p.seqlen;
  const int64_t d_base = static_cast<int64_t>(cb) * CW;
  const bool vec_ok = p.vec_ok != 0;
  const bool full_cols = vec_ok && d_base + CW <= p.dim;
  auto chunk_full = [&](int64_t c) { return full_cols && (c + 1) * CH <= t_end; };

  const int group = wave & 3;
  const int slot = (wave >> 2) * 3 + group;  // slot of a wave with group != 3
  if (group != 3 && slot < S) {
    const int s = slot;
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
    const int col = 16 * s + k;
    constexpr int kBatch = 8;
    constexpr int kBatches = CH / kBatch;
    float Bv[kHalves][NPL], Cv[kHalves][NPL];
    float2 dwq[2][kBatch];
    // B_t and C_t of this lane's row for step hf * 16 + k of the chunk in buffer buf (the
    // epilogue wave widened them to fp32 and zeroed the steps past the sequence)
    auto read_bc = [&](int hf, int buf) {
      const float4 vb = *reinterpret_cast<const float4*>(&s_bc[buf][0][hf * 16 + k][n0]);
      const float4 vc = *reinterpret_cast<const float4*>(&s_bc[buf][1][hf * 16 + k][n0]);
      Bv[hf][0] = vb.x; Bv[hf][1] = vb.y; Bv[hf][2] = vb.z; Bv[hf][3] = vb.w;
      Cv[hf][0] = vc.x; Cv[hf][1] = vc.y; Cv[hf][2] = vc.z; Cv[hf][3] = vc.w;
    };
    auto read_first_batch = [&](int buf) {
      static_for<kBatch>([&](auto K) { dwq[0][decltype(K)::value] = s_dw[buf][decltype(K)::value][col]; });
    };
    // The loop body has no branch: what the next chunk needs first (its first (dt, dt x) batch and
    // the B / C rows of its first 16 steps) is read while the last batch of this chunk runs, and
    // the rows of steps 16 .. 31 right after the barrier, so that none of these reads waits at a
    // barrier and every register is written on every path (no copies).  Past the last chunk the
    // reads land on a buffer no chunk uses; their values go unused.
    __syncthreads();  // iteration -2: the prologue stages chunk 0
    read_first_batch(0);
    read_bc(0, 0);
    __syncthreads();  // iteration -1: the prologue stages chunk 1
    int sbuf = 0;     // (dt, dt x) and B / C buffer of chunk j
    int pbuf = 1;     // the same of chunk j + 1
    // the state entering every 32nd step, for a backward pass that starts from it: (batch,
    // ceil(L / 32), dim, 16) as last_state, so a lane's 4 states are one 16-byte store and a
    // wave's 16 channels 1 KB
    const int64_t nck = (t_end + 31) / 32;
    float* const ck = (p.ckpt && lane_ok) ? p.ckpt + (b * nck * p.dim + d) * N + n0 : nullptr;
    for (int64_t j = 0; j < nchunks; ++j) {
      if (ck != nullptr && (CH == 32 || (j & 1) == 0))
        *reinterpret_cast<float4*>(ck + ((j * CH) / 32) * p.dim * N) = make_float4(h[0], h[1], h[2], h[3]);
      if constexpr (kHalves == 2) read_bc(1, sbuf);
      const int yb = static_cast<int>(j & 1);
      float ypp = 0.0f;  // read-out of the even step, written with the odd one
      static_for<kBatches>([&](auto Q) {
        constexpr int q = decltype(Q)::value;
        if constexpr (q + 1 < kBatches) {
          static_for<kBatch>([&](auto K) {
            dwq[(q + 1) & 1][decltype(K)::value] = s_dw[sbuf][(q + 1) * kBatch + decltype(K)::value][col];
          });
        } else {
          static_assert(kBatches % 2 == 0, "the last batch sits in dwq[1]");
          read_first_batch(pbuf);
          if constexpr (kHalves == 2) read_bc(0, pbuf);  // rows 0 .. 15 are done with by now
        }
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
              s_yp[yb][s][t - 2][lane] = ypp;
              s_yp[yb][s][t - 1][lane] = yp;
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
      s_yp[yb][s][CH - 2][lane] = ypp;
      s_yp[yb][s][CH - 1][lane] = yp;
      if constexpr (kHalves == 1) read_bc(0, pbuf);
      __syncthreads();
      sbuf = pbuf;
      pbuf = pbuf == kRowsDwBufs - 1 ? 0 : pbuf + 1;
    }
    __syncthreads();  // iteration nchunks: the epilogue stores the last chunk
    if (lane_ok && p.last_state) {
      float* dst = p.last_state + (b * p.dim + d) * N + n0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) dst[j] = h[j];
    }
    return;
  }

  if (group == 3 && (wave >> 2) < kRowsPrologueWaves) {
    const int io = wave >> 2;
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
    // With 16-byte rows (vec_ok) every lane loads whole pieces on every path: steps past the
    // sequence read the last step's row, pieces past dim or past the tile read column 0, and both
    // are zeroed when used.  The loads are then the same in every iteration, so the compiler's
    // wait before a tile counts only the older slot's loads and each tile has two iterations to
    // arrive.  Otherwise pieces are read element by element (and the wait covers every load).
    // Without a gate the z tile is read from x and never used.
    const void* zsrc = has_z ? p.z : p.x;
    auto run = [&](auto VO) {
    constexpr bool kVec = decltype(VO)::value;
    RawVec<BF16, VEC> nx[2][ITEMS], nd[2][ITEMS], nz[2][ITEMS];
    auto load_tile = [&](int64_t c, auto SL) {
      constexpr int sl = decltype(SL)::value;
      const int64_t t0 = c * CH;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int64_t t = t0 + prow[i];
        if constexpr (kVec) {
          const int64_t tc = t < t_end ? t : t_end - 1;
          const int64_t idx = (row_base + tc) * p.dim + d_base + (pnv[i] > 0 ? pcol[i] : 0);
          nx[sl][i].load(p.x, idx, VEC, true);
          nd[sl][i].load(p.delta, idx, VEC, true);
          nz[sl][i].load(zsrc, idx, VEC, true);
        } else {
          if (c >= nchunks) continue;
          const int nv = (t < t_end) ? pnv[i] : 0;
          const int64_t idx = (row_base + t) * p.dim + d_base + pcol[i];
          nx[sl][i].load(p.x, idx, nv, false);
          nd[sl][i].load(p.delta, idx, nv, false);
          if (has_z) nz[sl][i].load(p.z, idx, nv, false);
        }
      }
    };
    using Slot0 = std::integral_constant<int, 0>;
    using Slot1 = std::integral_constant<int, 1>;
    load_tile(0, Slot0{});
    __builtin_amdgcn_sched_barrier(0);  // every slot-0 load before the slot-1 loads
    load_tile(1, Slot1{});
    // iteration j: prologue of chunk j+2 from slot j & 1, then the tile of chunk j+4 into it
    auto iteration = [&](int64_t j, auto SL) {
      constexpr int sl = decltype(SL)::value;
      const int64_t c = j + 2;
      if constexpr (kVec) {
        // the slot's registers are taken in on every path (also for pieces past the tile, past
        // the last chunk and without a gate), so that no path leaves their loads outstanding and
        // the new loads into them need no wait for the other slot's
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
          nx[sl][i].consume();
          nd[sl][i].consume();
          nz[sl][i].consume();
        }
      }
      if (c < nchunks) {
        const int pb = static_cast<int>(c % kRowsDwBufs);
        const int xb = static_cast<int>(c % kRowsXzBufs);
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
      load_tile(c + 2, SL);
      __syncthreads();
    };
    // both slots in every trip (the loads last issued at the loop head are always slot 1's), the
    // odd iteration after the loop
    int64_t j = -2;
    for (; j + 1 <= nchunks; j += 2) {
      iteration(j, Slot0{});
      iteration(j + 1, Slot1{});
    }
    if (j <= nchunks) iteration(j, Slot0{});
    };
    if (vec_ok) run(std::true_type{});
    else run(std::false_type{});
    return;
  }

  // With three scan waves (one per scan SIMD) B and C are staged by two waves, slots 3 and 4
  // (SIMDs 0 and 1), so that each scan wave loses less issue to the staging; otherwise one wave in
  // slot S stages both (on a SIMD with the fewest scan waves for S = 2, 4, 5).
  constexpr bool kSplitStager = S == 3;
  if (group != 3 && (slot == S || (kSplitStager && slot == S + 1))) {
    // =============================== B / C stager ================================================
    // B and C rows of a chunk, staged as fp32 for the scan waves two chunks ahead of them, from
    // 32-bit words loaded one iteration earlier: word w = lane + 64 i of a tile is step w / WPR,
    // word w % WPR of its row.  Every lane loads on every path (no register merges, so no wait
    // right after a load): steps past the sequence read the last step's row and are stored as
    // zeros.  A few instructions per chunk, in a slot of a scan SIMD.
    constexpr int WPR = BF16 ? 8 : 16;  // 32-bit words per row of 16 states
    constexpr int WPT = CH * WPR;       // words per tile
    constexpr int BI = WPT / 64;
    // NT tensors from tensor t0 (0 = B, 1 = C)
    auto run = [&](auto NT_, int t0) {
      constexpr int NT = decltype(NT_)::value;
      const uint32_t* src[NT];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) src[tt] = static_cast<const uint32_t*>(t0 + tt == 0 ? p.B : p.C);
      uint32_t nw[NT][BI];
      auto load_bc_tile = [&](int64_t c) {
        const int64_t lim = t_end - 1 - c * CH;  // last step of the sequence, relative to the chunk
#pragma unroll
        for (int i = 0; i < BI; ++i) {
          const int w = lane + 64 * i;
          const int row = w / WPR;
          const int64_t off = (row_base + c * CH + (row <= lim ? static_cast<int64_t>(row) : lim)) * WPR + w % WPR;
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) nw[tt][i] = src[tt][off];
        }
      };
      auto stage_bc = [&](int64_t c) {
        const int pb = static_cast<int>(c % kRowsDwBufs);
#pragma unroll
        for (int i = 0; i < BI; ++i) {
          const int w = lane + 64 * i;
          const int row = w / WPR, wc = w % WPR;
          const bool ok = c * CH + row < t_end;
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            const uint32_t word = ok ? nw[tt][i] : 0u;
            if constexpr (BF16)
              *reinterpret_cast<float2*>(&s_bc[pb][t0 + tt][row][2 * wc]) = make_float2(bf16_lo(word), bf16_hi(word));
            else
              s_bc[pb][t0 + tt][row][wc] = __builtin_bit_cast(float, word);
          }
        }
      };
      // iteration j: B / C of chunk j + 2, then the loads of chunk j + 3's rows (past the last
      // chunk: in-range loads whose values go unused)
      load_bc_tile(0);
      for (int64_t j = -2; j <= nchunks; ++j) {
        // the words are taken in on every path, so that no path leaves their loads outstanding
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int i = 0; i < BI; ++i) asm volatile("" ::"v"(nw[tt][i]));
        if (j + 2 < nchunks) stage_bc(j + 2);
        load_bc_tile(j + 3);
        __syncthreads();
      }
    };
    if constexpr (kSplitStager) run(std::integral_constant<int, 1>{}, slot - S);
    else run(std::integral_constant<int, 2>{}, 0);
    return;
  }

  if (group != 3) {  // a slot without work: only the barriers
    for (int64_t j = -2; j <= nchunks; ++j) __syncthreads();
    return;
  }
  // =============================== epilogue role (wave 15) =======================================
  // D of the workgroup's channels, in LDS (written and read by this wave only, so in order)
  for (int c = lane; c < CW; c += 64) {
    const int64_t dc = d_base + c;
    s_dsk[c] = (p.Dskip && dc < p.dim) ? p.Dskip[dc] : 0.0f;
  }
  // iteration j: the output of chunk j - 1.  The wave only stores, so it never waits on memory.
  for (int64_t j = -2; j <= nchunks; ++j) {
    const int64_t e = j - 1;
    if (e >= 0) {
      const int yb = static_cast<int>(e & 1);
      const int xb = static_cast<int>(e % kRowsXzBufs);
      const bool full = chunk_full(e);
      // 16-byte pieces (VEC channels of one step), lane + 64 i; the indices are recomputed and
      // D read from LDS, and at most three rounds overlap, which keeps the wave's registers few
#pragma unroll 3
      for (int i = 0; i < EITEMS; ++i) {
        const int piece = lane + 64 * i;
        if (piece >= PIECES) break;
        const int er = piece / PPR, ec = (piece % PPR) * VEC;
        const int sw = ec / 16, k0 = ec % 16;
        float out[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          float acc = s_yp[yb][sw][er][k0 + v];
#pragma unroll
          for (int rr = 1; rr < 4; ++rr) acc += s_yp[yb][sw][er][16 * rr + k0 + v];
          const float2 xz = s_xz[xb][er][ec + v];
          out[v] = fmaf(s_dsk[ec + v], xz.x, acc) * xz.y;
        }
        const int64_t t = e * CH + er;
        const int64_t idx = (row_base + t) * p.dim + d_base + ec;
        if (full) {
          store_vec<BF16, VEC>(p.y, idx, out, VEC, true);
        } else {
          const int64_t dc = d_base + ec;
          const int nv = (t >= t_end || dc >= p.dim) ? 0 : static_cast<int>((p.dim - dc) < VEC ? (p.dim - dc) : VEC);
          if (nv > 0) store_vec<BF16, VEC>(p.y, idx, out, nv, vec_ok);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace ssm
