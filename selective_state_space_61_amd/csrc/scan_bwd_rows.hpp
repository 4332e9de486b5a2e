// scan_bwd_rows.hpp -- backward of the selective scan with state rows (dstate 16, Delta B input
// term, bf16 I/O with 16-byte rows), gfx950.
//
// The gradients and the adjoint recurrence are those of scan_bwd.hpp (its header lists them),
// with the states recomputed rather than stored ("mamba->jamba" sec. 2.3); the work decomposition
// is the forward's state rows of scan_rows.hpp ("Mamba 论文精读" sec. 2.2 and 3.3):
//   * scan wave s (waves 0 .. S-1, one per SIMD) holds channels 16 s .. 16 s + 15 of the
//     workgroup's 16 S: lane 16 r + k is channel k with state indices 4 r .. 4 r + 3.  B_t and C_t
//     come from LDS through DPP row broadcasts.  A workgroup of 48 channels gives the 130M shape
//     (8 x 1536 channels) 256 workgroups, one per compute unit.
//   * wave 3 (the prologue) stages (dt, dt x), dy0 = dy silu(z) and the raw x, delta, z, dy of a
//     chunk; wave 7 (the epilogue) turns the row sums into dx, ddelta, dz and accumulates dD and
//     dbias; both sit on the fourth SIMD.  Wave 4 (the stager, on a scan SIMD: a few instructions
//     per chunk) stages B and C and adds the chunk's dB / dC sums into the global accumulator.
//     The other waves only take part in the barriers.
//   * 512 threads, so a wave has 256 VGPRs: the 33 states of a 32-step chunk stay in registers
//     between the recompute and the reverse sweep.
// Phase 0 runs the recurrence forward and stores the state at the start of every 32-step chunk
// (fp32, (batch, nc, dim, 16): each chunk's states in last_state's layout); when the forward pass stored these states (scan_rows.hpp, the
// same layout), every role skips phase 0.  Phase 1 walks the chunks backwards; per chunk a scan wave
//   1. recomputes the chunk's states from the stored one, with the read-outs C_t.h_t;
//   2. sweeps the chunk in reverse: g_t = dy0_t C_t + abar_{t+1} g_{t+1}, dA in registers, and per
//      step the row partials sum_j g B_j (for dx) and sum_j g A_j abar_j h_{t-1,j} (for ddelta);
//   3. hands the channel sums of dB_t = sum_d g dt x and dC_t = sum_d dy0 h_t over its 16
//      channels to LDS (a transpose through LDS, one output per lane every two steps, stored in
//      the wave's own slot; the stager adds the S slots).  LDS float atomics are avoided: on this
//      chip a ds_add_f32 keeps the LDS busy many times longer than a store, and the scan's own
//      LDS reads queue behind it.
// The four row partials of a channel (read-out, gB, pdt) are summed inside the scan wave, four
// steps at a time, with v_permlane16_swap / v_permlane32_swap (gfx950): after the swaps lane
// 16 q + k holds step q's sum for channel k, one LDS write per four steps.
// The dB / dC sums of a workgroup are added into an fp32 accumulator with global atomics, so
// their order (and the last bits of dB and dC) may vary from run to run; the reduce kernel of
// scan_bwd.hpp converts them to the storage type.  Everything else is summed in a fixed order.
// Rows past the sequence carry dt = dt x = dy0 = 0 (identity steps with no gradient); channels
// past dim carry A = 0, dt x = dy0 = 0; neither is stored.
#pragma once

#include "scan_bwd.hpp"
#include "scan_fwd.hpp"

namespace ssm {

constexpr int kBwdRowsT = 32;      // steps per chunk
constexpr int kBwdRowsWaves = 8;   // waves per workgroup
constexpr int kBwdRowsMaxS = 3;    // scan waves: waves 0 .. S-1
constexpr int kBwdRowsPrologue = 3, kBwdRowsStager = 4, kBwdRowsEpilogue = 7;

// float2 per LDS row of (dt, dt x): the workgroup's channels plus 4 (rows 8 bytes apart in banks)
constexpr int bwd_rows_dws(int S) { return 16 * S + 4; }

constexpr int bwd_rows_lds_bytes(int S) {
  return 2 * kBwdRowsT * bwd_rows_dws(S) * 8   // (dt, dt x), double-buffered
         + 2 * 2 * kBwdRowsT * 16 * 4         // B, C (fp32)
         + 2 * kBwdRowsT * 16 * S * 4         // dy0
         + 3 * kBwdRowsT * 16 * S * 8         // raw x, delta, z, dy (bf16), triple-buffered
         + 2 * 3 * (kBwdRowsT / 4) * S * 64 * 4  // row sums: read-out, gB, pdt
         + S * 16 * 68 * 4                    // per-wave dB / dC transposes
         + 2 * S * kBwdRowsT * 32 * 4;        // each scan wave's dB / dC sums
}

// v_permlane16_swap (gfx950) on two registers: afterwards a holds rows (a0, b0, a2, b2) and b rows
// (a1, b1, a3, b3) of the 16-lane rows before.  The results pass through an empty asm: this
// compiler, given the builtin's two results as floats, has added the first to itself.
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                                  false, false);
  uint32_t x = r[0], y = r[1];
  asm volatile("" : "+v"(x), "+v"(y));
  a = __builtin_bit_cast(float, x);
  b = __builtin_bit_cast(float, y);
}
// v_permlane32_swap: afterwards a holds the lower halves (a_lo, b_lo), b the upper (a_hi, b_hi)
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                                  false, false);
  uint32_t x = r[0], y = r[1];
  asm volatile("" : "+v"(x), "+v"(y));
  a = __builtin_bit_cast(float, x);
  b = __builtin_bit_cast(float, y);
}

// One step of the four state chains of a lane with separate input and output state registers
// (the recompute keeps all 33 states of a chunk): out_j = exp2(dt a2_j) in_j + B_j w with B
// broadcast from lane KB of each row, and the read-out of the input states, sum_j C_j in_j with C
// broadcast from lane KC (the previous step's read-out).  The instructions and their order are
// those of step_readout4 (the forward's block), so the states are the forward's bits.
#define SSM_BWD_DPP_KB "row_newbcast:%[kb] row_mask:0xf bank_mask:0xf"
#define SSM_BWD_DPP_KC "row_newbcast:%[kc] row_mask:0xf bank_mask:0xf"
template <int KB, int KC>
__device__ __forceinline__ float step_readout4_io(float dt, float w, const float* a2, const float* b, const float* c,
                                                  const float* hin, float* hout) {
  float t0, t1, t2, t3, u0, u1, u2, u3, yp, o0, o1, o2, o3;
  asm("v_mul_f32 %[t0], %[dt], %[a0]\n\t"
      "v_mul_f32 %[t1], %[dt], %[a1]\n\t"
      "v_mul_f32 %[t2], %[dt], %[a2]\n\t"
      "v_mul_f32 %[t3], %[dt], %[a3]\n\t"
      "v_exp_f32 %[t0], %[t0]\n\t"
      "v_exp_f32 %[t1], %[t1]\n\t"
      "v_exp_f32 %[t2], %[t2]\n\t"
      "v_exp_f32 %[t3], %[t3]\n\t"
      "v_mul_f32_dpp %[u0], %[b0], %[w] " SSM_BWD_DPP_KB "\n\t"
      "v_mul_f32_dpp %[yp], %[c0], %[i0] " SSM_BWD_DPP_KC "\n\t"
      "v_mul_f32_dpp %[u1], %[b1], %[w] " SSM_BWD_DPP_KB "\n\t"
      "v_fma_f32 %[o0], %[t0], %[i0], %[u0]\n\t"
      "v_fmac_f32_dpp %[yp], %[c1], %[i1] " SSM_BWD_DPP_KC "\n\t"
      "v_mul_f32_dpp %[u2], %[b2], %[w] " SSM_BWD_DPP_KB "\n\t"
      "v_fma_f32 %[o1], %[t1], %[i1], %[u1]\n\t"
      "v_fmac_f32_dpp %[yp], %[c2], %[i2] " SSM_BWD_DPP_KC "\n\t"
      "v_mul_f32_dpp %[u3], %[b3], %[w] " SSM_BWD_DPP_KB "\n\t"
      "v_fma_f32 %[o2], %[t2], %[i2], %[u2]\n\t"
      "v_fmac_f32_dpp %[yp], %[c3], %[i3] " SSM_BWD_DPP_KC "\n\t"
      "v_fma_f32 %[o3], %[t3], %[i3], %[u3]"
      : [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3), [u0] "=&v"(u0), [u1] "=&v"(u1),
        [u2] "=&v"(u2), [u3] "=&v"(u3), [yp] "=&v"(yp), [o0] "=&v"(o0), [o1] "=&v"(o1), [o2] "=&v"(o2),
        [o3] "=&v"(o3)
      : [dt] "v"(dt), [w] "v"(w), [a0] "v"(a2[0]), [a1] "v"(a2[1]), [a2] "v"(a2[2]), [a3] "v"(a2[3]),
        [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]), [c0] "v"(c[0]), [c1] "v"(c[1]),
        [c2] "v"(c[2]), [c3] "v"(c[3]), [i0] "v"(hin[0]), [i1] "v"(hin[1]), [i2] "v"(hin[2]), [i3] "v"(hin[3]),
        [kb] "i"(KB), [kc] "i"(KC));
  hout[0] = o0;
  hout[1] = o1;
  hout[2] = o2;
  hout[3] = o3;
  return yp;
}

// One reverse step of the four state chains of a lane, B_t and C_t broadcast from lane KB of each
// row.  With abar_{t+1} in an and the adjoint of the step after in g:
//   g  <- abar_{t+1} g + dy0 C_t               (the adjoint of h_t)
//   an <- abar_t = exp2(dt a2)
//   gB  = sum_j g_j B_t,j                       (this row's share of d/d(dt x))
//   pdt = sum_j a_j abar_t h_{t-1},j g_j        (this row's share of d/d(dt) through abar)
//   dA += dt abar_t h_{t-1} g
// The products and their rounding are those of the plain expressions: (abar h) g, fma chains.
template <int KB>
__device__ __forceinline__ void bwd_step4(float dt, float dy0, const float* a2, const float* araw, const float* b,
                                          const float* c, const float* hin, float* g, float* an, float* dA,
                                          float& gB, float& pdt) {
  float t0, t1, t2, t3, u0, u1, u2, u3, gb, pd;
  asm("v_mul_f32 %[t0], %[dt], %[a0]\n\t"
      "v_mul_f32 %[t1], %[dt], %[a1]\n\t"
      "v_mul_f32 %[t2], %[dt], %[a2]\n\t"
      "v_mul_f32 %[t3], %[dt], %[a3]\n\t"
      "v_mul_f32_dpp %[u0], %[c0], %[dy] " SSM_BWD_DPP_KB "\n\t"
      "v_mul_f32_dpp %[u1], %[c1], %[dy] " SSM_BWD_DPP_KB "\n\t"
      "v_mul_f32_dpp %[u2], %[c2], %[dy] " SSM_BWD_DPP_KB "\n\t"
      "v_mul_f32_dpp %[u3], %[c3], %[dy] " SSM_BWD_DPP_KB "\n\t"
      "v_fmac_f32 %[u0], %[n0], %[g0]\n\t"
      "v_fmac_f32 %[u1], %[n1], %[g1]\n\t"
      "v_fmac_f32 %[u2], %[n2], %[g2]\n\t"
      "v_fmac_f32 %[u3], %[n3], %[g3]\n\t"
      "v_exp_f32 %[n0], %[t0]\n\t"
      "v_exp_f32 %[n1], %[t1]\n\t"
      "v_exp_f32 %[n2], %[t2]\n\t"
      "v_exp_f32 %[n3], %[t3]\n\t"
      "v_mul_f32_dpp %[gb], %[b0], %[u0] " SSM_BWD_DPP_KB "\n\t"
      "v_fmac_f32_dpp %[gb], %[b1], %[u1] " SSM_BWD_DPP_KB "\n\t"
      "v_fmac_f32_dpp %[gb], %[b2], %[u2] " SSM_BWD_DPP_KB "\n\t"
      "v_fmac_f32_dpp %[gb], %[b3], %[u3] " SSM_BWD_DPP_KB "\n\t"
      "v_mul_f32 %[t0], %[n0], %[h0]\n\t"
      "v_mul_f32 %[t1], %[n1], %[h1]\n\t"
      "v_mul_f32 %[t2], %[n2], %[h2]\n\t"
      "v_mul_f32 %[t3], %[n3], %[h3]\n\t"
      "v_mul_f32 %[t0], %[t0], %[u0]\n\t"
      "v_mul_f32 %[t1], %[t1], %[u1]\n\t"
      "v_mul_f32 %[t2], %[t2], %[u2]\n\t"
      "v_mul_f32 %[t3], %[t3], %[u3]\n\t"
      "v_mul_f32 %[pd], %[t0], %[r0]\n\t"
      "v_fmac_f32 %[d0], %[t0], %[dt]\n\t"
      "v_fmac_f32 %[pd], %[t1], %[r1]\n\t"
      "v_fmac_f32 %[d1], %[t1], %[dt]\n\t"
      "v_fmac_f32 %[pd], %[t2], %[r2]\n\t"
      "v_fmac_f32 %[d2], %[t2], %[dt]\n\t"
      "v_fmac_f32 %[pd], %[t3], %[r3]\n\t"
      "v_fmac_f32 %[d3], %[t3], %[dt]"
      : [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3), [u0] "=&v"(u0), [u1] "=&v"(u1),
        [u2] "=&v"(u2), [u3] "=&v"(u3), [gb] "=&v"(gb), [pd] "=&v"(pd), [n0] "+v"(an[0]), [n1] "+v"(an[1]),
        [n2] "+v"(an[2]), [n3] "+v"(an[3]), [d0] "+v"(dA[0]), [d1] "+v"(dA[1]), [d2] "+v"(dA[2]), [d3] "+v"(dA[3])
      : [dt] "v"(dt), [dy] "v"(dy0), [a0] "v"(a2[0]), [a1] "v"(a2[1]), [a2] "v"(a2[2]), [a3] "v"(a2[3]),
        [r0] "v"(araw[0]), [r1] "v"(araw[1]), [r2] "v"(araw[2]), [r3] "v"(araw[3]), [b0] "v"(b[0]),
        [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]), [c0] "v"(c[0]), [c1] "v"(c[1]), [c2] "v"(c[2]),
        [c3] "v"(c[3]), [h0] "v"(hin[0]), [h1] "v"(hin[1]), [h2] "v"(hin[2]), [h3] "v"(hin[3]), [g0] "v"(g[0]),
        [g1] "v"(g[1]), [g2] "v"(g[2]), [g3] "v"(g[3]), [kb] "i"(KB));
  g[0] = u0;
  g[1] = u1;
  g[2] = u2;
  g[3] = u3;
  gB = gb;
  pdt = pd;
}
#undef SSM_BWD_DPP_KB
#undef SSM_BWD_DPP_KC

// sum_k p_k w_k over the 16 lanes k of a row, w_k taken from lane k of the lane's own row; two
// fma chains of eight.  (The leading wait covers a VALU write of w just before: a DPP source.)
__device__ __forceinline__ float dot16_row_bcast(const float4* p, float w) {
  float s0, s1;
#define SSM_BC(k) "row_newbcast:" #k " row_mask:0xf bank_mask:0xf"
  asm("s_nop 1\n\t"
      "v_mul_f32_dpp %[s0], %[w], %[p0] " SSM_BC(0) "\n\t"
      "v_mul_f32_dpp %[s1], %[w], %[p8] " SSM_BC(8) "\n\t"
      "v_fmac_f32_dpp %[s0], %[w], %[p1] " SSM_BC(1) "\n\t"
      "v_fmac_f32_dpp %[s1], %[w], %[p9] " SSM_BC(9) "\n\t"
      "v_fmac_f32_dpp %[s0], %[w], %[p2] " SSM_BC(2) "\n\t"
      "v_fmac_f32_dpp %[s1], %[w], %[p10] " SSM_BC(10) "\n\t"
      "v_fmac_f32_dpp %[s0], %[w], %[p3] " SSM_BC(3) "\n\t"
      "v_fmac_f32_dpp %[s1], %[w], %[p11] " SSM_BC(11) "\n\t"
      "v_fmac_f32_dpp %[s0], %[w], %[p4] " SSM_BC(4) "\n\t"
      "v_fmac_f32_dpp %[s1], %[w], %[p12] " SSM_BC(12) "\n\t"
      "v_fmac_f32_dpp %[s0], %[w], %[p5] " SSM_BC(5) "\n\t"
      "v_fmac_f32_dpp %[s1], %[w], %[p13] " SSM_BC(13) "\n\t"
      "v_fmac_f32_dpp %[s0], %[w], %[p6] " SSM_BC(6) "\n\t"
      "v_fmac_f32_dpp %[s1], %[w], %[p14] " SSM_BC(14) "\n\t"
      "v_fmac_f32_dpp %[s0], %[w], %[p7] " SSM_BC(7) "\n\t"
      "v_fmac_f32_dpp %[s1], %[w], %[p15] " SSM_BC(15)
      : [s0] "=&v"(s0), [s1] "=&v"(s1)
      : [w] "v"(w), [p0] "v"(p[0].x), [p1] "v"(p[0].y), [p2] "v"(p[0].z), [p3] "v"(p[0].w), [p4] "v"(p[1].x),
        [p5] "v"(p[1].y), [p6] "v"(p[1].z), [p7] "v"(p[1].w), [p8] "v"(p[2].x), [p9] "v"(p[2].y),
        [p10] "v"(p[2].z), [p11] "v"(p[2].w), [p12] "v"(p[3].x), [p13] "v"(p[3].y), [p14] "v"(p[3].z),
        [p15] "v"(p[3].w));
#undef SSM_BC
  return s0 + s1;
}

// The four 16-lane rows of y0 .. y3 summed per lane column: lane 16 q + k of the result holds
// (y_q[k] + y_q[16 + k]) + (y_q[32 + k] + y_q[48 + k]).
__device__ __forceinline__ float rows4_transpose_sum(float y0, float y1, float y2, float y3) {
  permlane16_swap(y0, y1);  // y0 = (y0 r0, y1 r0, y0 r2, y1 r2), y1 = (y0 r1, y1 r1, y0 r3, y1 r3)
  float u = y0 + y1;        // (y0 r01, y1 r01, y0 r23, y1 r23)
  permlane16_swap(y2, y3);
  float v = y2 + y3;        // (y2 r01, y3 r01, y2 r23, y3 r23)
  permlane32_swap(u, v);    // u = (y0 r01, y1 r01, y2 r01, y3 r01), v = the same of r23
  return u + v;
}

template <int S>
__global__ __launch_bounds__(64 * kBwdRowsWaves) void scan_bwd_rows_kernel(const BwdArgs p) {
  constexpr int N = 16, NPL = 4, T = kBwdRowsT;
  constexpr int CW = 16 * S;          // channels per workgroup
  constexpr int DWS = bwd_rows_dws(S);
  constexpr int VEC = 8;              // bf16 channels per 16-byte piece
  constexpr int PPR = CW / VEC;       // pieces per tile row
  constexpr int PIECES = T * PPR;
  constexpr int ITEMS = (PIECES + 63) / 64;  // pieces per prologue / epilogue lane
  static_assert(S >= 1 && S <= kBwdRowsMaxS, "scan waves per workgroup");
  static_assert(bwd_rows_lds_bytes(S) <= kLdsBudget, "LDS tiles exceed a workgroup's share");

  __shared__ float2 s_dw[2][T][DWS];
  __shared__ __align__(16) float s_bc[2][2][T][N];
  __shared__ float s_dy0[2][T][CW];
  __shared__ uint2 s_ep[3][T][CW];                 // {x | delta << 16, z | dy << 16}
  __shared__ float s_part[2][3][T / 4][S][64];     // row sums: read-out, gB, pdt
  __shared__ __align__(16) float s_red[S][16][68]; // dB / dC transpose rows of a scan wave
  __shared__ float s_bsum[2][S][T][2 * N];         // each scan wave's dB (0..15), dC (16..31)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t blk = xcd_local(blockIdx.x, gridDim.x);
  const int cb = static_cast<int>(blk % p.ncb);
  const int64_t b = blk / p.ncb;
  const int64_t L = p.seqlen;
  const int64_t nc = p.nc;  // chunks of T steps (L >= 1: the host does not launch an empty pass)
  const int64_t row_base = b * L;
  const int64_t d_base = static_cast<int64_t>(cb) * CW;

  // ===================================== scan role ==============================================
  if (wave < S) {
    const int s = wave;
    const int r = lane >> 4, k = lane & 15;
    const int64_t d = d_base + 16 * s + k;
    const bool lane_ok = d < p.dim;
    const int n0 = 4 * r;
    const int col = 16 * s + k;
    float A2[NPL], Araw[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      Araw[j] = lane_ok ? p.A[d * N + n0 + j] : 0.0f;
      A2[j] = fmaxf(Araw[j] * kLog2e, -3.0e38f);
    }
    // the state before chunk c, (batch, nc, dim, 16) as last_state: the lane's 4 states are 16
    // contiguous bytes, a wave's 16 channels 1 KB
    auto hstart = [&](int64_t c) -> float4* {
      return reinterpret_cast<float4*>(p.hstart + ((b * nc + c) * p.dim + d) * N + n0);
    };
    float Bv[2][NPL], Cv[2][NPL];
    auto read_b = [&](int buf) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float4 v = *reinterpret_cast<const float4*>(&s_bc[buf][0][hf * 16 + k][n0]);
        Bv[hf][0] = v.x; Bv[hf][1] = v.y; Bv[hf][2] = v.z; Bv[hf][3] = v.w;
      }
    };
    auto read_c = [&](int buf) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float4 v = *reinterpret_cast<const float4*>(&s_bc[buf][1][hf * 16 + k][n0]);
        Cv[hf][0] = v.x; Cv[hf][1] = v.y; Cv[hf][2] = v.z; Cv[hf][3] = v.w;
      }
    };

    // ---- phase 0: forward over chunk j - 1 in iteration j, storing its starting state ----------
    // (skipped by every role when the forward pass stored the states)
    if (!p.have_hstart) {
      float h[NPL] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int64_t j = 0; j <= nc; ++j) {
        if (j >= 1) {
          const int64_t c = j - 1;
          const int buf = static_cast<int>(c & 1);
          if (lane_ok) *hstart(c) = make_float4(h[0], h[1], h[2], h[3]);
          read_b(buf);
          // (dt, dt x) in batches of 8 steps, each read while the batch before it runs
          float2 rq[2][8];
          static_for<8>([&](auto J) { rq[0][decltype(J)::value] = s_dw[buf][decltype(J)::value][col]; });
          static_for<T>([&](auto K) {
            constexpr int t = decltype(K)::value;
            if constexpr (t % 8 == 0 && t + 8 < T)
              static_for<8>([&](auto J) {
                rq[(t / 8 + 1) & 1][decltype(J)::value] = s_dw[buf][t + 8 + decltype(J)::value][col];
              });
            const float2 dw = rq[(t / 8) & 1][t % 8];
#pragma unroll
            for (int q = 0; q < NPL; ++q)
              h[q] = fmaf(hw_exp2(dw.x * A2[q]), h[q], row_bcast<t % 16>(Bv[t / 16][q]) * dw.y);
          });
        }
        __syncthreads();
      }
    }

    // ---- phase 1: chunk cs = nc - 1 - i in iteration i -----------------------------------------
    float g[NPL], an[NPL], dA[NPL];  // adjoint (of the step after), abar of the step after, dA
#pragma unroll
    for (int q = 0; q < NPL; ++q) g[q] = an[q] = dA[q] = 0.0f;
    // the starting state of the next chunk to sweep, loaded one iteration ahead (always in range)
    float hn[NPL];
    auto load_hn = [&](int64_t c) {
      const int64_t cc = c < 0 ? 0 : c;
      const float4 v = lane_ok ? *hstart(cc) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      hn[0] = v.x; hn[1] = v.y; hn[2] = v.z; hn[3] = v.w;
    };
    load_hn(nc - 1);
    __syncthreads();  // iteration -1: the prologue stages chunk nc - 1
    float* const red = &s_red[s][0][0];
    for (int64_t cs = nc - 1; cs >= 0; --cs) {
      const int buf = static_cast<int>(cs & 1);
      float hs[T + 1][NPL];
#pragma unroll
      for (int q = 0; q < NPL; ++q) hs[0][q] = hn[q];
      load_hn(cs - 1);
      read_b(buf);
      read_c(buf);
      // recompute the states and the row read-outs C_t.h_t; (dt, dt x) in batches of 8 steps, each
      // read while the batch before it runs
      float yq[4];
      float2 rq[2][8];
      static_for<8>([&](auto J) { rq[0][decltype(J)::value] = s_dw[buf][decltype(J)::value][col]; });
      // step t's block also reads out step t - 1 (its input states); one more read-out after the
      // last step
      static_for<T + 1>([&](auto K) {
        constexpr int t = decltype(K)::value;
        float yp;
        if constexpr (t < T) {
          if constexpr (t % 8 == 0 && t + 8 < T)
            static_for<8>([&](auto J) {
              rq[(t / 8 + 1) & 1][decltype(J)::value] = s_dw[buf][t + 8 + decltype(J)::value][col];
            });
          const float2 dw = rq[(t / 8) & 1][t % 8];
          // (for t = 0 the read-out uses step 31's C and goes unused)
          yp = step_readout4_io<t % 16, (t + 15) % 16>(dw.x, dw.y, A2, Bv[t / 16], Cv[((t + T - 1) % T) / 16], hs[t],
                                                       hs[t + 1]);
        } else {
          yp = 0.0f;
#pragma unroll
          for (int q = 0; q < NPL; ++q) yp = fmaf(row_bcast<(T - 1) % 16>(Cv[(T - 1) / 16][q]), hs[T][q], yp);
        }
        if constexpr (t >= 1) {
          constexpr int tp = t - 1;  // the step this read-out belongs to
          yq[tp % 4] = yp;
          if constexpr (tp % 4 == 3)
            s_part[buf][0][tp / 4][s][lane] = rows4_transpose_sum(yq[0], yq[1], yq[2], yq[3]);
        }
      });
      // reverse sweep.  The compiler barrier makes the sweep read (dt, dt x) from LDS again and
      // recompute abar, and the opaque B / C registers make it broadcast them again: reusing the
      // recompute's values would keep 32 (dt, dt x) pairs, 128 exponentials and 256 broadcasts
      // alive next to the 132 states, more registers than a wave has.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int q = 0; q < NPL; ++q) asm volatile("" : "+v"(Bv[hf][q]), "+v"(Cv[hf][q]));
      // (dt, dt x) and dy0 in batches of 4 steps (reverse order), each read while the batch after
      // it runs
      float2 wq[2][4];
      float dq[2][4];
      auto read_batch = [&](auto M) {  // steps 4 m .. 4 m + 3 into slot m & 1
        constexpr int m = decltype(M)::value;
        static_for<4>([&](auto J) {
          constexpr int j = decltype(J)::value;
          wq[m & 1][j] = s_dw[buf][4 * m + j][col];
          dq[m & 1][j] = s_dy0[buf][4 * m + j][col];
        });
      };
      read_batch(std::integral_constant<int, T / 4 - 1>{});
      float gq[4], pq[4];
      // dB_t = sum over channels of g_t dt x, dC_t = sum over channels of dy0 h_t: a round (two
      // steps) writes g_t and h_t of its steps as rows of a transpose; at the end of the next
      // round lane (row, rr) takes the 16 channels of its row and state group, which arrived in
      // the meantime (a wave's LDS instructions run in order, so they return the round's values
      // although the next round rewrites the rows), and multiplies them by the channels' dt x or
      // dy0 broadcast from the lanes of its own 16-lane row (that row's (sub, kind) is fixed)
      const int row = lane >> 2, rr = lane & 3;
      const int sub = row >> 3, kind = (row >> 2) & 1, qrow = row & 3;
      const float4* const src = reinterpret_cast<const float4*>(red + row * 68 + 16 * rr);
      float4 pend[4];
      float wpend;  // lane 16 R + k: channel k's dt x (R even) or dy0 (R odd) of step t_even + R / 2
      auto add_round = [&](int t_even) {
        s_bsum[buf][s][t_even + sub][kind * N + 4 * rr + qrow] = dot16_row_bcast(pend, wpend);
      };
      static_for<T>([&](auto K) {
        constexpr int t = T - 1 - decltype(K)::value;
        constexpr int m = t / 4;
        if constexpr (t % 4 == 3 && m > 0) read_batch(std::integral_constant<int, m - 1>{});
        const float2 dw = wq[m & 1][t % 4];
        const float dy0 = dq[m & 1][t % 4];
        float gB, pdt;
        bwd_step4<t % 16>(dw.x, dy0, A2, Araw, Bv[t / 16], Cv[t / 16], hs[t], g, an, dA, gB, pdt);
        gq[t % 4] = gB;
        pq[t % 4] = pdt;
        if constexpr (t % 4 == 0) {
          s_part[buf][1][t / 4][s][lane] = rows4_transpose_sum(gq[0], gq[1], gq[2], gq[3]);
          s_part[buf][2][t / 4][s][lane] = rows4_transpose_sum(pq[0], pq[1], pq[2], pq[3]);
        }
        // row (sub, kind, q) of the transpose, sub = t % 2
        asm volatile("" ::: "memory");  // after the previous round's reads
#pragma unroll
        for (int q = 0; q < NPL; ++q) {
          red[((t % 2) * 8 + q) * 68 + lane] = g[q];
          red[((t % 2) * 8 + 4 + q) * 68 + lane] = hs[t + 1][q];
        }
        if constexpr (t % 2 == 0) {
          // steps t, t + 1 written
          if constexpr (t + 2 < T) add_round(t + 2);  // the previous round's reads have arrived
          asm volatile("" ::: "memory");
          pend[0] = src[0]; pend[1] = src[1]; pend[2] = src[2]; pend[3] = src[3];
          const float2 dw1 = wq[m & 1][t % 4 + 1];
          const float dy1 = dq[m & 1][t % 4 + 1];
          const float w0 = (r & 1) ? dy0 : dw.y, w1 = (r & 1) ? dy1 : dw1.y;
          wpend = (r & 2) ? w1 : w0;
        }
      });
      add_round(0);
      __syncthreads();
    }
    __syncthreads();  // iteration nc: the epilogue finishes chunk 0
    if (lane_ok) {
#pragma unroll
      for (int q = 0; q < NPL; ++q) p.part_a[(b * N + n0 + q) * p.dim + d] = dA[q];
    }
    return;
  }

  // ===================================== prologue (wave 3) ======================================
  if (wave == kBwdRowsPrologue) {
    int prow[ITEMS], pcol[ITEMS];
    bool pon[ITEMS];
    float bias[ITEMS][VEC];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int piece = lane + 64 * i;
      pon[i] = piece < PIECES;
      prow[i] = pon[i] ? piece / PPR : 0;
      pcol[i] = pon[i] ? (piece % PPR) * VEC : 0;
      const int64_t dc = d_base + pcol[i];
#pragma unroll
      for (int v = 0; v < VEC; ++v) bias[i][v] = (p.delta_bias && dc + v < p.dim) ? p.delta_bias[dc + v] : 0.0f;
    }
    const bool has_z = p.z != nullptr;
    const void* zsrc = has_z ? p.z : p.x;
    // piece i of chunk c: 16 bytes at row c T + prow (the last row past the sequence) and column
    // d_base + pcol (column 0 past dim): in range on every path
    auto tile_idx = [&](int64_t c, int i) {
      const int64_t t = c * T + prow[i];
      const int64_t tc = t < L ? t : L - 1;
      const int64_t dc = d_base + pcol[i];
      return (row_base + tc) * p.dim + (dc < p.dim ? dc : 0);
    };
    auto ok_at = [&](int64_t c, int i, int v) { return c * T + prow[i] < L && d_base + pcol[i] + v < p.dim; };
    using Slot0 = std::integral_constant<int, 0>;
    using Slot1 = std::integral_constant<int, 1>;

    // ---- phase 0: (dt, dt x) of chunk j in iteration j, tiles loaded two iterations ahead ------
    if (!p.have_hstart) {
      RawVec<true, VEC> nx[2][ITEMS], nd[2][ITEMS];
      auto load = [&](int64_t c, auto SL) {
        constexpr int sl = decltype(SL)::value;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
          const int64_t idx = tile_idx(c, i);
          nx[sl][i].load(p.x, idx, VEC, true);
          nd[sl][i].load(p.delta, idx, VEC, true);
        }
      };
      auto iteration = [&](int64_t j, auto SL) {
        constexpr int sl = decltype(SL)::value;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
          nx[sl][i].consume();
          nd[sl][i].consume();
        }
        if (j < nc) {
          const int buf = static_cast<int>(j & 1);
#pragma unroll
          for (int i = 0; i < ITEMS; ++i) {
            if (!pon[i]) continue;
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              const float vv = nd[sl][i].get(v) + bias[i][v];
              const float dtv = p.softplus ? softplus_f32(vv) : vv;
              const bool ok = ok_at(j, i, v);
              const float dt = ok ? dtv : 0.0f, xs = ok ? nx[sl][i].get(v) : 0.0f;
              s_dw[buf][prow[i]][pcol[i] + v] = make_float2(dt, dt * xs);
            }
          }
        }
        load(j + 2 < nc ? j + 2 : nc - 1, SL);
        __syncthreads();
      };
      load(0, Slot0{});
      __builtin_amdgcn_sched_barrier(0);
      load(nc > 1 ? 1 : 0, Slot1{});
      int64_t j = 0;
      for (; j + 1 <= nc; j += 2) {
        iteration(j, Slot0{});
        iteration(j + 1, Slot1{});
      }
      if (j <= nc) iteration(j, Slot0{});
    }

    // ---- phase 1: chunk cp = nc - 2 - i in iteration i, tiles loaded two iterations ahead -----
    RawVec<true, VEC> nx[2][ITEMS], nd[2][ITEMS], nz[2][ITEMS], ny[2][ITEMS];
    auto load = [&](int64_t c, auto SL) {
      constexpr int sl = decltype(SL)::value;
      const int64_t cc = c < 0 ? 0 : c;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int64_t idx = tile_idx(cc, i);
        nx[sl][i].load(p.x, idx, VEC, true);
        nd[sl][i].load(p.delta, idx, VEC, true);
        nz[sl][i].load(zsrc, idx, VEC, true);
        ny[sl][i].load(p.dy, idx, VEC, true);
      }
    };
    auto iteration = [&](int64_t i, auto SL) {
      constexpr int sl = decltype(SL)::value;
      const int64_t cp = nc - 2 - i;
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        nx[sl][it].consume();
        nd[sl][it].consume();
        nz[sl][it].consume();
        ny[sl][it].consume();
      }
      if (cp >= 0) {
        const int buf = static_cast<int>(cp & 1);
        const int eb = static_cast<int>(cp % 3);
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
          if (!pon[it]) continue;
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            const bool ok = ok_at(cp, it, v);
            const float vv = nd[sl][it].get(v) + bias[it][v];
            const float dtv = p.softplus ? softplus_f32(vv) : vv;
            const float xs = nx[sl][it].get(v), zs = nz[sl][it].get(v), dys = ny[sl][it].get(v);
            const float dy0 = has_z ? dys * silu_f32(zs) : dys;
            const float dt = ok ? dtv : 0.0f;
            s_dw[buf][prow[it]][pcol[it] + v] = make_float2(dt, dt * (ok ? xs : 0.0f));
            s_dy0[buf][prow[it]][pcol[it] + v] = ok ? dy0 : 0.0f;
          }
          // raw bf16 words: {x, delta} and {z, dy} per channel
          uint2 raw[VEC];
#pragma unroll
          for (int v = 0; v < VEC; v += 2) {
            const uint32_t xw = nx[sl][it].w[v / 2], dw = nd[sl][it].w[v / 2];
            const uint32_t zw = nz[sl][it].w[v / 2], yw = ny[sl][it].w[v / 2];
            raw[v] = make_uint2((xw & 0xffffu) | (dw << 16), (zw & 0xffffu) | (yw << 16));
            raw[v + 1] = make_uint2((xw >> 16) | (dw & 0xffff0000u), (zw >> 16) | (yw & 0xffff0000u));
          }
          uint4* dst = reinterpret_cast<uint4*>(&s_ep[eb][prow[it]][pcol[it]]);
#pragma unroll
          for (int v = 0; v < VEC; v += 2) dst[v / 2] = make_uint4(raw[v].x, raw[v].y, raw[v + 1].x, raw[v + 1].y);
        }
      }
      load(cp - 2, SL);
      __syncthreads();
    };
    load(nc - 1, Slot0{});
    __builtin_amdgcn_sched_barrier(0);
    load(nc - 2, Slot1{});
    // iterations -1 .. nc (the slot of iteration i is (i + 1) & 1)
    int64_t i = -1;
    for (; i + 1 <= nc; i += 2) {
      iteration(i, Slot0{});
      iteration(i + 1, Slot1{});
    }
    if (i <= nc) iteration(i, Slot0{});
    return;
  }

  // ===================================== stager (wave 4) ========================================
  if (wave == kBwdRowsStager) {
    // B and C rows of a chunk: 32 rows of 32 bytes each = 64 pieces of 16 bytes, one per lane;
    // loaded two iterations ahead (rows past the sequence read the last row), zero when staged
    const int srow = lane >> 1, shalf = lane & 1;
    auto piece_off = [&](int64_t c) {
      const int64_t t = c * T + srow;
      return (row_base + (t < L ? t : L - 1)) * N + 8 * shalf;
    };
    auto widen = [&](uint4 w, float* dst) {
      *reinterpret_cast<float4*>(dst) = make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
      *reinterpret_cast<float4*>(dst + 4) = make_float4(bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w));
    };
    const uint16_t* Bg = static_cast<const uint16_t*>(p.B);
    const uint16_t* Cg = static_cast<const uint16_t*>(p.C);
    const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
    using Slot0 = std::integral_constant<int, 0>;
    using Slot1 = std::integral_constant<int, 1>;
    // ---- phase 0: B of chunk j in iteration j ------------------------------------------------
    if (!p.have_hstart) {
      uint4 nb[2];
      auto load = [&](int64_t c, auto SL) {
        nb[decltype(SL)::value] = *reinterpret_cast<const uint4*>(Bg + piece_off(c));
      };
      auto iteration = [&](int64_t j, auto SL) {
        constexpr int sl = decltype(SL)::value;
        asm volatile("" ::"v"(nb[sl].x), "v"(nb[sl].y), "v"(nb[sl].z), "v"(nb[sl].w));
        if (j < nc) widen(j * T + srow < L ? nb[sl] : zero4, &s_bc[j & 1][0][srow][8 * shalf]);
        load(j + 2 < nc ? j + 2 : nc - 1, SL);
        __syncthreads();
      };
      load(0, Slot0{});
      __builtin_amdgcn_sched_barrier(0);
      load(nc > 1 ? 1 : 0, Slot1{});
      int64_t j = 0;
      for (; j + 1 <= nc; j += 2) {
        iteration(j, Slot0{});
        iteration(j + 1, Slot1{});
      }
      if (j <= nc) iteration(j, Slot0{});
    }
    // ---- phase 1: B, C of chunk cp = nc - 2 - i and the dB / dC sums of chunk ce = nc - i -----
    uint4 nb[2], ncr[2];
    auto load = [&](int64_t c, auto SL) {
      constexpr int sl = decltype(SL)::value;
      const int64_t off = piece_off(c < 0 ? 0 : c);
      nb[sl] = *reinterpret_cast<const uint4*>(Bg + off);
      ncr[sl] = *reinterpret_cast<const uint4*>(Cg + off);
    };
    float* const acc_b = p.part_bc;                            // (batch, L, N) fp32
    float* const acc_c = p.part_bc + p.batch * L * N;
    auto iteration = [&](int64_t i, auto SL) {
      constexpr int sl = decltype(SL)::value;
      const int64_t cp = nc - 2 - i, ce = nc - i;
      asm volatile("" ::"v"(nb[sl].x), "v"(nb[sl].y), "v"(nb[sl].z), "v"(nb[sl].w));
      asm volatile("" ::"v"(ncr[sl].x), "v"(ncr[sl].y), "v"(ncr[sl].z), "v"(ncr[sl].w));
      if (cp >= 0) {
        const bool ok = cp * T + srow < L;
        widen(ok ? nb[sl] : zero4, &s_bc[cp & 1][0][srow][8 * shalf]);
        widen(ok ? ncr[sl] : zero4, &s_bc[cp & 1][1][srow][8 * shalf]);
      }
      if (ce < nc) {
        const float* sums = &s_bsum[ce & 1][0][0][0];
#pragma unroll
        for (int e0 = 0; e0 < T * 2 * N; e0 += 64) {
          const int e = e0 + lane;
          const int tt = e / (2 * N), q = e % (2 * N);
          const int64_t t = ce * T + tt;
          float sum = sums[e];
#pragma unroll
          for (int sw = 1; sw < S; ++sw) sum += sums[sw * T * 2 * N + e];
          // every lane adds on every path (0 to the last row past the sequence): one wait count
          const int64_t tc = t < L ? t : L - 1;
          atomicAdd((q < N ? acc_b : acc_c) + (row_base + tc) * N + (q % N), t < L ? sum : 0.0f);
        }
      }
      load(cp - 2, SL);
      __syncthreads();
    };
    load(nc - 1, Slot0{});
    __builtin_amdgcn_sched_barrier(0);
    load(nc - 2, Slot1{});
    int64_t i = -1;
    for (; i + 1 <= nc; i += 2) {
      iteration(i, Slot0{});
      iteration(i + 1, Slot1{});
    }
    if (i <= nc) iteration(i, Slot0{});
    return;
  }

  // ===================================== epilogue (wave 7) ======================================
  if (wave == kBwdRowsEpilogue) {
    const bool has_z = p.z != nullptr;
    // per piece: D and the delta bias of its channels, and the dD / dbias accumulators.  The wave
    // makes no loads inside the loop, so it never waits on memory (its stores would sit ahead of
    // any load in the wait count)
    float accD[ITEMS][VEC], accBias[ITEMS][VEC], edsk[ITEMS][VEC], ebias[ITEMS][VEC];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int piece = lane + 64 * i;
      const int64_t dc = d_base + (piece < PIECES ? (piece % PPR) * VEC : 0);
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        accD[i][v] = accBias[i][v] = 0.0f;
        const bool ok = piece < PIECES && dc + v < p.dim;
        edsk[i][v] = (ok && p.Dskip) ? p.Dskip[dc + v] : 0.0f;
        ebias[i][v] = (ok && p.delta_bias) ? p.delta_bias[dc + v] : 0.0f;
      }
    }
    if (!p.have_hstart)
      for (int64_t j = 0; j <= nc; ++j) __syncthreads();  // phase 0
    for (int64_t i = -1; i <= nc; ++i) {
      const int64_t ce = nc - i;
      if (ce < nc) {
        const int pb = static_cast<int>(ce & 1), eb = static_cast<int>(ce % 3);
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
          const int piece = lane + 64 * it;
          if (piece >= PIECES) break;
          const int er = piece / PPR, ec = (piece % PPR) * VEC;
          const int sw = ec / 16, k0 = ec % 16;
          const int64_t t = ce * T + er;
          const int64_t dc = d_base + ec;
          float dxo[VEC], ddo[VEC], dzo[VEC];
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            const uint2 raw = s_ep[eb][er][ec + v];
            const float xs = bf16_lo(raw.x), vv = bf16_hi(raw.x) + ebias[it][v];
            const float zs = bf16_lo(raw.y), dys = bf16_hi(raw.y);
            const int lq = 16 * (er % 4) + k0 + v;
            const float yp = s_part[pb][0][er / 4][sw][lq];
            const float gB = s_part[pb][1][er / 4][sw][lq];
            const float pdt = s_part[pb][2][er / 4][sw][lq];
            const float dsk = edsk[it][v];
            const float dt = p.softplus ? softplus_f32(vv) : vv;
            float dy0 = dys, dz = 0.0f;
            const float y0 = fmaf(dsk, xs, yp);
            if (has_z) {
              const float sg = hw_rcp(1.0f + hw_exp2(-zs * kLog2e));
              dy0 = dys * (zs * sg);
              dz = dys * y0 * fmaf(zs * sg, 1.0f - sg, sg);
            }
            dxo[v] = fmaf(dy0, dsk, dt * gB);
            const float ddt = fmaf(gB, xs, pdt);
            ddo[v] = p.softplus ? ddt * hw_rcp(1.0f + hw_exp2(-vv * kLog2e)) : ddt;
            dzo[v] = dz;
            const bool ok = t < L && dc + v < p.dim;
            accD[it][v] = ok ? fmaf(dy0, xs, accD[it][v]) : accD[it][v];
            accBias[it][v] += ok ? ddo[v] : 0.0f;
          }
          if (t < L) {
            const int64_t idx = (row_base + t) * p.dim + dc;
            const int nv = dc >= p.dim ? 0 : static_cast<int>((p.dim - dc) < VEC ? (p.dim - dc) : VEC);
            if (nv > 0) {
              store_vec<true, VEC>(p.dx, idx, dxo, nv, true);
              store_vec<true, VEC>(p.ddelta, idx, ddo, nv, true);
              if (has_z) store_vec<true, VEC>(p.dz, idx, dzo, nv, true);
            }
          }
        }
      }
      __syncthreads();
    }
    // per-(batch row, tile row) partials of dD and dbias, summed by the reduce kernel
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int piece = lane + 64 * it;
      if (piece >= PIECES) break;
      const int er = piece / PPR, ec = (piece % PPR) * VEC;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const int64_t dc = d_base + ec + v;
        if (dc < p.dim) {
          p.part_d[(b * T + er) * p.dim + dc] = accD[it][v];
          p.part_bias[(b * T + er) * p.dim + dc] = accBias[it][v];
        }
      }
    }
    return;
  }

  // ===================================== the other waves: barriers only =========================
  if (!p.have_hstart)
    for (int64_t j = 0; j <= nc; ++j) __syncthreads();
  for (int64_t i = -1; i <= nc; ++i) __syncthreads();
}

using BwdRowsKernel = void (*)(const BwdArgs);
// The state-row backward with S scan waves per workgroup (1 .. kBwdRowsMaxS), else NULL.
BwdRowsKernel bwd_rows_kernel(int S);

}  // namespace ssm
