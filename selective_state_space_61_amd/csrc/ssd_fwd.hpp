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
// Sequence split (for grids too small to fill the chip): the chunks are cut into segments.  The
// recurrence is linear, so a segment's true end state is e^{sum dt A over it} S_in + S_end, with
// S_end its end state from zero.  Pass 1 (MODE kSsdStateOnly) runs segments 0..k-2 from zero
// through the state update only and records S_end and sum dt A; ssd_carry_kernel composes the
// entering states in order (with few segments each workgroup of pass 2 composes its own instead);
// pass 2 (kSsdOutputs) runs every segment from its entering state.
//
// Work split: one workgroup per (batch row, head, slice of PS = 16*NW head channels).  Wave w
// owns channels [16w, 16w+16) of the slice, so the columns of S it updates are exactly the ones
// it reads out: S never leaves the wave's accumulators.  The twelve 16 x 16 tiles of C B^T a
// chunk needs are split over the waves and exchanged through LDS as the masked matrix M.
//
// Operand layouts of the 16x16x32 product D = A B (lane l, q = l / 16, i = 0..7, r = 0..3):
//   A: lane l holds A[l % 16][8q + i];  B: lane l holds B[8q + i][l % 16];
//   D: lane l holds D[4q + r][l % 16].
// Every tile of the chunk (B, C, X, the weighted X, M) sits in LDS row-major, as it comes from
// memory, written with 16-byte stores.  Operands whose K index is the row (B^T and X^T over the
// steps) are read with the transposing LDS read ds_read_b64_tr_b16: in each 16-lane group,
// output lane i receives, for e = 0..3, element i % 4 of the 8 bytes that lane 4e + i/4
// addresses.  So when lane s of the group addresses row k0 + s/4 at column c(s % 4), lane i gets
// rows k0..k0+3 of column c(i/4) + i%4: four consecutive K values of one M/N index, from any four
// 4-column groups.  Two such reads make a K = 32 fragment.
//
// The S tiles (16 dstate rows x 16 channels each) interleave the dstate index in pairs: row
// 4j + r of tile nb is dstate 32 (nb / 2) + 8 j + 4 (nb % 2) + r.  A lane holds rows 4q .. 4q+3
// of a tile, so tiles 2ks and 2ks+1 give lane l the eight consecutive dstate indices
// 32 ks + 8q .. +7: exactly the K values a K = 32 step asks of lane l.  The accumulators pack
// straight into the A operand of the read-out, C is read with one 16-byte load per fragment, and
// the state update's transposing reads of B address those rows (column group 8 (s % 4) + 4 (nb % 2)
// of the 32-column block for source lane s).
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
  const float* init_state;  // (batch, nheads, headdim, dstate) state entering the sequence, or NULL (zero)
  const float* seg_init;  // (nseg-1, batch, nheads, headdim, dstate): state entering segment s >= 1 at
                          // [s-1], or NULL (every segment starts from zero)
  float* seg_state;       // same layout: end state of segment s from zero at [s] (state-only pass)
  float* seg_dsum;        // (nseg, batch, nheads): sum over segment s of dt A log2(e) (state-only pass)
  const float* gram;      // (batch, ngroups, chunks, 12, 64, 4): the tiles of C B^T per chunk, as
                          // ssd_gram_kernel leaves them (the precomputed-Gram outputs pass), or NULL
  float* gram_out;        // the same buffer, written by ssd_gram_kernel
  int64_t batch;
  int64_t seqlen;
  int32_t nheads;
  int32_t headdim;
  int32_t ngroups;
  int32_t nslices;  // headdim / PS
  int32_t softplus;
  int32_t nseg;        // segments the chunks are cut into
  int32_t seg_chunks;  // chunks per segment (the last may hold fewer)
  int32_t compose;     // 1: a later segment composes its entering state itself from seg_state and
                       // seg_dsum (few segments; no carry kernel); 0: it reads seg_init
};

constexpr int kSsdOutputs = 0;    // full chunk work: y, and the final state from the last segment
constexpr int kSsdStateOnly = 1;  // state update only: the segment's end state and summed decay
constexpr int kSsdOutputsGram = 2;  // kSsdOutputs with the tiles of C B^T read from SsdArgs::gram

constexpr int kSsdChunk = 64;  // steps per chunk: one per lane of a wave

typedef __bf16 ssd_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float ssd_f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t ssd_u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t ssd_u32x2_t __attribute__((ext_vector_type(2)));
typedef short ssd_i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ ssd_f32x4_t mfma16x16x32(ssd_u32x4_t a, ssd_u32x4_t b, ssd_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(ssd_bf16x8_t, a),
                                                 __builtin_bit_cast(ssd_bf16x8_t, b), c, 0, 0, 0);
}

// ds_read_b64_tr_b16 at an LDS address, as two 32-bit words.
__device__ __forceinline__ ssd_u32x2_t lds_read_tr(const uint16_t* p) {
  const ssd_i16x4_t v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ssd_i16x4_t*)(p));
  return __builtin_bit_cast(ssd_u32x2_t, v);
}

// A K = 32 fragment over rows k0 .. k0+31 of a row-major LDS tile with row stride ld: this lane
// (group q, local index s16) addresses rows k0 + 8q + s16/4 and +4 at column col, which the
// caller chooses as the column group for local source lane s16 % 4.  The receiving lane i of the
// group gets rows k0 + 8q .. +7 of column col(i / 4) + i % 4.
__device__ __forceinline__ ssd_u32x4_t lds_frag_tr(const uint16_t* tile, int ld, int k0, int q, int s16, int col) {
  const uint16_t* ptr = tile + (k0 + 8 * q + s16 / 4) * ld + col;
  const ssd_u32x2_t lo = lds_read_tr(ptr), hi = lds_read_tr(ptr + 4 * ld);
  return ssd_u32x4_t{lo.x, lo.y, hi.x, hi.y};
}

// The chunk's B rows in LDS.  The state update reads them transposed (ds_read_b64_tr_b16: 16 lanes
// address rows k0 .. k0+3 at four column groups 8 elements apart), which with rows padded to
// N + 8 elements puts up to four lanes on one bank.  With SWZ a row is stored unpadded, its
// 16-byte pieces permuted by the row: piece p of row j sits at p ^ h(j), h(j) = 4 (j % 4) +
// (j / 4) % 4.  Then those reads hit each bank at most twice (the least for 8-byte reads of one
// half of each piece), the staging stores meet no conflict, and the tile is 2 KB smaller.  The
// chunk kernel takes it from dstate 128 when it does not compute C B^T itself (whose register
// budget the swizzled addressing of its B reads would exceed).
template <int N, bool SWZ>
struct SsdBLayout {
  static constexpr bool kSwizzle = SWZ && N >= 128;
  static constexpr int LD = kSwizzle ? N : N + 8;  // row stride (elements)
  // element offset of (row, col); col % 8 is kept, so 8- and 16-byte accesses stay in one piece
  __device__ static __forceinline__ int off(int row, int col) {
    if constexpr (kSwizzle)
      return row * LD + 8 * ((col >> 3) ^ (((row & 3) << 2) | ((row >> 2) & 3))) + (col & 7);
    else
      return row * LD + col;
  }
};

// lds_frag_tr for the B tile in its SsdBLayout BL.
template <class BL>
__device__ __forceinline__ ssd_u32x4_t lds_frag_tr_b(const uint16_t* s_b, int k0, int q, int s16, int col) {
  const int r = k0 + 8 * q + s16 / 4;
  const ssd_u32x2_t lo = lds_read_tr(s_b + BL::off(r, col));
  const ssd_u32x2_t hi = lds_read_tr(s_b + BL::off(r + 4, col));
  return ssd_u32x4_t{lo.x, lo.y, hi.x, hi.y};
}

template <int E>
__device__ __forceinline__ float bf16_elem(ssd_u32x4_t v) {
  return (E & 1) ? bf16_hi(v[E / 2]) : bf16_lo(v[E / 2]);
}

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

// The twelve 16 x 16 tiles (i-block ib, j-block jb) of C B^T a chunk needs: the ten with
// jb <= ib and the two just past the diagonal, (0, 1) and (2, 3), that a K = 32 step of the
// masked product reads (the mask zeroes them).  Tile k is (k/2, k%2) for k < 4, else
// (k/4 + 1, k%4).
__device__ __forceinline__ int gram_tile_i(int k) { return k < 4 ? k / 2 : k / 4 + 1; }
__device__ __forceinline__ int gram_tile_j(int k) { return k < 4 ? k % 2 : k % 4; }

// The three 16 x 16 tiles of G^T = B C^T (over dstate) that wave w of four computes:
// (w / 2, w % 2), (2, w) and (3, w) in (i-block, j-block) terms, i.e. tiles k = w, w + 4, w + 8.
// The last two share their B rows, and for w < 2 the first does too, so a K step reads 4 or 5
// fragments instead of 6.  frag_b(r, col) / frag_c(r, col) return 16 bytes (8 bf16) of row r of the
// chunk's B / C at dstate column col, wherever the caller keeps them.  gt must hold zeros.
template <int N, class FragB, class FragC>
__device__ __forceinline__ void gram_tiles_nw4(FragB frag_b, FragC frag_c, int wave, int l16, int q,
                                               ssd_f32x4_t* gt) {
  constexpr int NKS = N / 32;
  const bool b0_shared = wave < 2;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int col = 32 * ks + 8 * q;
    const ssd_u32x4_t bw = frag_b(16 * wave + l16, col);
    const ssd_u32x4_t c2 = frag_c(32 + l16, col);
    const ssd_u32x4_t c3 = frag_c(48 + l16, col);
    const ssd_u32x4_t c0 = frag_c(16 * (wave >> 1) + l16, col);
    const ssd_u32x4_t b0 = b0_shared ? bw : frag_b(16 * (wave & 1) + l16, col);
    gt[0] = mfma16x16x32(b0, c0, gt[0]);
    gt[1] = mfma16x16x32(bw, c2, gt[1]);
    gt[2] = mfma16x16x32(bw, c3, gt[2]);
  }
}

// Workgroups of 4 waves (dstate <= 128) keep two workgroups per compute unit: their LDS fits
// twice in 160 KB and the registers are held to 256 per lane.
template <int N, int NW>
constexpr int kSsdWavesPerEu = (NW == 4 && N <= 128) ? 2 : 1;

template <int N, int NW, int MODE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(kSsdWavesPerEu<N, NW>)))
void ssd_chunk_kernel(const SsdArgs p) {
  constexpr bool OUT = MODE != kSsdStateOnly;
  constexpr bool PRE = MODE == kSsdOutputsGram;  // C B^T tiles from the buffer, not computed here
  constexpr int Q = kSsdChunk;
  constexpr int PS = 16 * NW;         // head channels per workgroup
  constexpr int T = 64 * NW;          // threads
  constexpr int LDB = N + 8;          // row stride (elements) of the C tile (B: SsdBLayout)
  constexpr int LDX = PS + 8;         // row stride of the X and weighted-X tiles
  constexpr int LDM = Q + 8;          // row stride of M
  constexpr int LDY = PS + 4;         // row stride of the fp32 output tile
  constexpr int kDtPer = Q / NW;      // raw dt values each wave loads
  constexpr int NKS = N / 32;         // K = 32 steps over dstate
  constexpr int NT = N / 16;          // 16-row tiles of S per wave
  constexpr int kBCPer = 8 * N / T;   // 16-byte pieces of B (and of C) per thread
  constexpr int kXPer = 8 * PS / T;   // 16-byte pieces of X per thread
  constexpr int kTiles = 12 / NW;     // tiles of C B^T per wave
  static_assert(N % 32 == 0 && (8 * N) % T == 0, "dstate is a multiple of 32");
  static_assert(kXPer == 2, "two 16-byte pieces of X per thread");
  static_assert(!PRE || NW == 4, "the precomputed C B^T tiles are laid out for four waves");

  using BL = SsdBLayout<N, MODE != kSsdOutputs>;  // swizzled unless this kernel computes C B^T
  __shared__ __align__(16) uint16_t s_b[Q * BL::LD];  // B[j][n] at BL::off(j, n)
  __shared__ __align__(16) uint16_t s_c[Q * LDB];   // C[i][n]
  __shared__ __align__(16) uint16_t s_x[Q * LDX];   // X[j][p]
  __shared__ __align__(16) uint16_t s_xw[Q * LDX];  // X[j][p] * exp(cum_last - cum_j) dt_j
  __shared__ __align__(16) uint16_t s_m[Q * LDM];   // M[i][j] = (C_i . B_j) exp(cum_i - cum_j) dt_j, j <= i
  __shared__ __align__(16) float s_cum[Q];          // cum_j in log2 units
  __shared__ __align__(16) float s_dt[Q];           // dt_j (0 past the end of the sequence)
  __shared__ __align__(16) float s_y[Q * LDY];      // Y[i][p] of the previous chunk, for the epilogue
  __shared__ __align__(16) uint16_t s_dtraw[Q];     // raw dt of the chunk being staged

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  // The heads of a group read the same B and C rows: the logical index is permuted so that
  // consecutive heads (and slices) share an XCD and its L2, which then fetches those rows once.
  const int64_t blk = xcd_local(blockIdx.x, gridDim.x);
  const int slice = static_cast<int>(blk % p.nslices);
  const int64_t bhs = blk / p.nslices;
  const int64_t nbh = p.batch * p.nheads;
  const int64_t bh = bhs % nbh;
  const int seg = static_cast<int>(bhs / nbh);
  const int h = static_cast<int>(bh % p.nheads);
  const int64_t b = bh / p.nheads;
  const int g = h / (p.nheads / p.ngroups);
  const int64_t L = p.seqlen, H = p.nheads, P = p.headdim, G = p.ngroups;
  const int p0 = slice * PS;
  const float A2 = p.A[h] * kLog2e;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const float Dh = p.D ? p.D[h] : 0.0f;
  const int pw = 16 * wave + l16;            // this lane's S column (and output channel of its D rows)
  const int pe = 16 * wave + 4 * q;          // first of the 4 output channels this lane's Y tiles hold
  const int cx = 16 * wave + 4 * (l16 & 3);  // column group this lane addresses in transposing reads of X

  const uint16_t* xg = p.x + (b * L * H + h) * P + p0;  // step t at xg + t * H * P
  const uint16_t* zg = p.z ? p.z + (b * L * H + h) * P + p0 : nullptr;
  uint16_t* yg = p.y + (b * L * H + h) * P + p0;
  const uint16_t* bg = p.B + (b * L * G + g) * N;  // step t at bg + t * G * N
  const uint16_t* cg = p.C + (b * L * G + g) * N;
  const uint16_t* dtg = p.dt + b * L * H + h;       // step t at dtg + t * H
  const int64_t xs = H * P, bs = G * N;

  // Registers that carry the next chunk's inputs while the current one is computed.  A piece is
  // 16 bytes of one row; consecutive threads take consecutive pieces of a row (coalesced).  x and
  // z come in two register sets, alternating between chunks: the set of the chunk whose epilogue
  // is pending takes the next chunk's loads once that epilogue has run (no copies between sets).
  ssd_u32x4_t rb[kBCPer], rc[kBCPer], rx[2][kXPer], rz[2][kXPer];
  uint32_t rdt = 0u;
#pragma unroll
  for (int u = 0; u < kXPer; ++u) rz[0][u] = rz[1][u] = rx[1][u] = ssd_u32x4_t{0u, 0u, 0u, 0u};
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;

  float dsum = 0.0f;  // sum of dt A log2(e) over the chunks run

  // Steps past the end of the sequence load the last step's rows (always in range, so every
  // lane loads on every path and no register merge makes the compiler wait right after a load):
  // their dt is staged as 0, which zeroes their weighted X, their columns of M and their share of
  // the state, and their output rows are not stored.  Without a gate the z pieces are x's.
  const uint16_t* zsrc = zg ? zg : xg;
  auto load_chunk = [&](int64_t t0, auto SET) {
    constexpr int st = decltype(SET)::value;
#pragma unroll
    for (int u = 0; u < kBCPer; ++u) {
      const int k = tid + u * T;
      const int c8 = k % (N / 8), j = k / (N / 8);
      const int64_t t = t0 + j < L ? t0 + j : L - 1;
      rb[u] = *reinterpret_cast<const ssd_u32x4_t*>(bg + t * bs + 8 * c8);
      if constexpr (OUT) rc[u] = *reinterpret_cast<const ssd_u32x4_t*>(cg + t * bs + 8 * c8);
    }
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      const int k = tid + u * T;
      const int p8 = k % (PS / 8), j = k / (PS / 8);
      const int64_t t = t0 + j < L ? t0 + j : L - 1;
      rx[st][u] = *reinterpret_cast<const ssd_u32x4_t*>(xg + t * xs + 8 * p8);
      if constexpr (OUT) rz[st][u] = *reinterpret_cast<const ssd_u32x4_t*>(zsrc + t * xs + 8 * p8);
    }
    // wave w loads the raw dt of steps kDtPer w .. +kDtPer-1 (lanes below kDtPer)
    const int64_t td = t0 + kDtPer * wave + lane;
    rdt = lane < kDtPer ? dtg[(td < L ? td : L - 1) * H] : 0u;
  };
  // The raw dt just loaded goes to LDS once it has arrived (read by every wave at the next stage).
  auto publish_dt = [&]() {
    if (lane < kDtPer) s_dtraw[kDtPer * wave + lane] = static_cast<uint16_t>(rdt);
  };

  // Skip term, gate and store of the chunk at step te0 whose Y sits in s_y: each thread takes the
  // same 16-byte pieces it loaded (x and z in register set SET), 8 channels of one step.  FULL:
  // all 64 steps of the chunk are inside the sequence (no bounds checks).
  auto epilogue = [&](int64_t te0, auto full, auto SET) {
    constexpr bool FULL = decltype(full)::value;
    constexpr int st = decltype(SET)::value;
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      const int k = tid + u * T;
      const int p8 = k % (PS / 8), j = k / (PS / 8);
      const int64_t t = te0 + j;
      if (FULL || t < L) {
        const ssd_f32x4_t y0 = *reinterpret_cast<const ssd_f32x4_t*>(&s_y[j * LDY + 8 * p8]);
        const ssd_f32x4_t y1 = *reinterpret_cast<const ssd_f32x4_t*>(&s_y[j * LDY + 8 * p8 + 4]);
        float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xr = (e & 1) ? bf16_hi(rx[st][u][e / 2]) : bf16_lo(rx[st][u][e / 2]);
          const float zr = (e & 1) ? bf16_hi(rz[st][u][e / 2]) : bf16_lo(rz[st][u][e / 2]);
          yv[e] = fmaf(Dh, xr, yv[e]) * (zg ? silu_f32(zr) : 1.0f);
        }
        // y is written once and read by the next layer, not here: a non-temporal store keeps the
        // caches for the B and C rows that every head of the group reads
        __builtin_nontemporal_store(
            ssd_u32x4_t{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]), pack_bf16x2(yv[4], yv[5]),
                        pack_bf16x2(yv[6], yv[7])},
            reinterpret_cast<ssd_u32x4_t*>(yg + t * xs + 8 * p8));
      }
    }
  };

  // Writes the chunk held in registers to LDS.
  auto stage_chunk = [&](int64_t t0, auto SET) {
    constexpr int st = decltype(SET)::value;
    // dt and the cumulative decay: lane l of every wave holds step l of the chunk
    const float v = bf16_lo(s_dtraw[lane]) + bias;
    const float dtv = t0 + lane < L ? (p.softplus ? softplus_f32(v) : v) : 0.0f;
    const float cum = wave_inclusive_sum(dtv * A2);
    const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cum), 63));
    const float wgt = hw_exp2(last - cum) * dtv;
    dsum += last;
    if (wave == 0) {
      s_cum[lane] = cum;
      s_dt[lane] = dtv;
    }
#pragma unroll
    for (int u = 0; u < kBCPer; ++u) {
      const int k = tid + u * T;
      const int c8 = k % (N / 8), j = k / (N / 8);
      *reinterpret_cast<ssd_u32x4_t*>(&s_b[BL::off(j, 8 * c8)]) = rb[u];
      if constexpr (OUT) *reinterpret_cast<ssd_u32x4_t*>(&s_c[j * LDB + 8 * c8]) = rc[u];
    }
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      const int k = tid + u * T;
      const int p8 = k % (PS / 8), j = k / (PS / 8);
      const float w = __shfl(wgt, j);
      if constexpr (OUT) {
        *reinterpret_cast<ssd_u32x4_t*>(&s_x[j * LDX + 8 * p8]) = rx[st][u];
      }
      *reinterpret_cast<ssd_u32x4_t*>(&s_xw[j * LDX + 8 * p8]) =
          ssd_u32x4_t{pack_bf16x2(bf16_elem<0>(rx[st][u]) * w, bf16_elem<1>(rx[st][u]) * w),
                      pack_bf16x2(bf16_elem<2>(rx[st][u]) * w, bf16_elem<3>(rx[st][u]) * w),
                      pack_bf16x2(bf16_elem<4>(rx[st][u]) * w, bf16_elem<5>(rx[st][u]) * w),
                      pack_bf16x2(bf16_elem<6>(rx[st][u]) * w, bf16_elem<7>(rx[st][u]) * w)};
    }
  };

  // S tile nb, lane (q, r): dstate index 32 (nb / 2) + 8q + 4 (nb % 2) + r of channel pw (the
  // final-state layout), at state_off + toff(nb) + r
  const int64_t state_off = ((b * H + h) * P + p0 + pw) * N + 8 * q;
  auto toff = [](int nb) { return 32 * (nb >> 1) + 4 * (nb & 1); };
  const int64_t state_seg = nbh * P * N;  // elements per segment in the segment buffers
  ssd_f32x4_t S[NT];
  // the entering state: the carried one for a later segment, the caller's for the first (the
  // state-only pass starts every segment from zero; the carry adds the caller's state)
  if (OUT && p.compose && seg > 0) {
    // composed here, with the carry kernel's arithmetic in its order: from the caller's state
    // (zero without one), S <- e^{sum dt A of segment r} S + S_end(r) for r = 0 .. seg-1
#pragma unroll
    for (int nb = 0; nb < NT; ++nb)
      S[nb] = p.init_state ? *reinterpret_cast<const ssd_f32x4_t*>(p.init_state + state_off + toff(nb))
                           : ssd_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int r = 0; r < seg; ++r) {
      const float decay = hw_exp2(p.seg_dsum[r * nbh + bh]);
      const float* sr = p.seg_state + r * state_seg + state_off;
#pragma unroll
      for (int nb = 0; nb < NT; ++nb) {
        const ssd_f32x4_t e = *reinterpret_cast<const ssd_f32x4_t*>(sr + toff(nb));
#pragma unroll
        for (int i = 0; i < 4; ++i) S[nb][i] = fmaf(decay, S[nb][i], e[i]);
      }
    }
  } else {
    const float* si = (p.seg_init && seg > 0) ? p.seg_init + (seg - 1) * state_seg + state_off
                      : (OUT && p.init_state && seg == 0) ? p.init_state + state_off
                                                          : nullptr;
    if (si) {
#pragma unroll
      for (int nb = 0; nb < NT; ++nb) S[nb] = *reinterpret_cast<const ssd_f32x4_t*>(si + toff(nb));
    } else {
#pragma unroll
      for (int nb = 0; nb < NT; ++nb) S[nb] = ssd_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  const int64_t nch = (L + Q - 1) / Q;
  const int64_t cbeg = static_cast<int64_t>(seg) * p.seg_chunks;
  const int64_t cend = cbeg + p.seg_chunks < nch ? cbeg + p.seg_chunks : nch;
  using Full = std::integral_constant<bool, true>;
  using Ragged = std::integral_constant<bool, false>;
  if (cbeg < cend) {
    load_chunk(cbeg * Q, Set0{});
    publish_dt();
  }
  // chunk c, whose x and z sit in register set SET (chunk cbeg in set 0, then alternating)
  auto chunk = [&](int64_t c, auto SET) {
    using Prev = std::integral_constant<int, 1 - decltype(SET)::value>;
    const int64_t t0 = c * Q;
    // this wave's three tiles of C B^T (k = wave, wave + 4, wave + 8), issued here so that they
    // arrive during the epilogue and the staging
    ssd_f32x4_t gpre[3];
    if constexpr (PRE) {
      const float* gsrc = p.gram + (((b * G + g) * nch + c) * 12 + wave) * 256 + 4 * lane;
#pragma unroll
      for (int s = 0; s < 3; ++s) gpre[s] = *reinterpret_cast<const ssd_f32x4_t*>(gsrc + 4 * 256 * s);
    }
    __syncthreads();  // every wave is done with the previous chunk's tiles
    if (OUT && c > cbeg) epilogue(t0 - Q, Full{}, Prev{});  // the chunk before this one is whole
    stage_chunk(t0, SET);
    __syncthreads();
    // the next chunk; after the segment's last one the loads still run (one path, no merge) but
    // read this chunk's rows again, which its L2 holds, and their values go unused
    load_chunk(c + 1 < cend ? t0 + Q : t0, Prev{});

    if constexpr (OUT) {
      // M, split over the waves: G^T tile (j-block jb, i-block ib) = B_j . C_i (both rows are
      // dstate-contiguous: plain 16-byte reads), masked to j <= i, decayed and stored as M[i][j]
      {
        ssd_f32x4_t gt[kTiles];
#pragma unroll
        for (int s = 0; s < kTiles; ++s) gt[s] = ssd_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (PRE) {
#pragma unroll
          for (int s = 0; s < kTiles; ++s) gt[s] = gpre[s];
        } else if constexpr (NW == 4) {
          gram_tiles_nw4<N>([&](int r, int col) { return *reinterpret_cast<const ssd_u32x4_t*>(&s_b[BL::off(r, col)]); },
                            [&](int r, int col) { return *reinterpret_cast<const ssd_u32x4_t*>(&s_c[r * LDB + col]); },
                            wave, l16, q, gt);
        } else {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int s = 0; s < kTiles; ++s) {
              const int k = wave + NW * s;
              const int ib = gram_tile_i(k), jb = gram_tile_j(k);
              gt[s] = mfma16x16x32(*reinterpret_cast<const ssd_u32x4_t*>(&s_b[BL::off(16 * jb + l16, 32 * ks + 8 * q)]),
                                   *reinterpret_cast<const ssd_u32x4_t*>(&s_c[(16 * ib + l16) * LDB + 32 * ks + 8 * q]),
                                   gt[s]);
            }
        }
#pragma unroll
        for (int s = 0; s < kTiles; ++s) {
          const int k = wave + NW * s;
          const int ib = gram_tile_i(k), jb = gram_tile_j(k);
          const int irow = 16 * ib + l16;
          const float cum_i = s_cum[irow];
          const ssd_f32x4_t cj = *reinterpret_cast<const ssd_f32x4_t*>(&s_cum[16 * jb + 4 * q]);
          const ssd_f32x4_t dj = *reinterpret_cast<const ssd_f32x4_t*>(&s_dt[16 * jb + 4 * q]);
          float m[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            m[r] = (16 * jb + 4 * q + r <= irow) ? gt[s][r] * hw_exp2(cum_i - cj[r]) * dj[r] : 0.0f;
          *reinterpret_cast<ssd_u32x2_t*>(&s_m[irow * LDM + 16 * jb + 4 * q]) =
              ssd_u32x2_t{pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3])};
        }
      }

      // S entering the chunk as bf16 A operands of the read-out: S^T[pw][n], n permuted as the
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
      for (int ib = 0; ib < 4; ++ib) acc[ib] = ssd_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
          acc[ib] = mfma16x16x32(sf[ks], *reinterpret_cast<const ssd_u32x4_t*>(&s_c[(16 * ib + l16) * LDB + 32 * ks + 8 * q]),
                                 acc[ib]);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) acc[ib] *= hw_exp2(s_cum[16 * ib + l16]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const ssd_u32x4_t xa = lds_frag_tr(s_x, LDX, 32 * ks, q, l16, cx);  // X^T[pw][32 ks + 8q ..]
#pragma unroll
        for (int ib = 2 * ks; ib < 4; ++ib)
          acc[ib] = mfma16x16x32(xa, *reinterpret_cast<const ssd_u32x4_t*>(&s_m[(16 * ib + l16) * LDM + 32 * ks + 8 * q]),
                                 acc[ib]);
      }
      // Y^T tiles to LDS as Y[i][p] for the epilogue (run at the next chunk's staging)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) *reinterpret_cast<ssd_f32x4_t*>(&s_y[(16 * ib + l16) * LDY + pe]) = acc[ib];
    }

    // state update: S = exp(cum_last) S + B^T (weighted X); the B^T operand of tile nb is its 16
    // dstate rows of B^T, read transposed from B (this lane addresses column
    // 32 (nb / 2) + 8 (l16 % 4) + 4 (nb % 2))
    const float decay = hw_exp2(s_cum[Q - 1]);
#pragma unroll
    for (int nb = 0; nb < NT; ++nb) S[nb] *= decay;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const ssd_u32x4_t xw = lds_frag_tr(s_xw, LDX, 32 * ks, q, l16, cx);  // weighted X[32 ks + 8q ..][pw]
#pragma unroll
      for (int nb = 0; nb < NT; ++nb)
        S[nb] = mfma16x16x32(lds_frag_tr_b<BL>(s_b, 32 * ks, q, l16, 32 * (nb >> 1) + 8 * (l16 & 3) + 4 * (nb & 1)),
                             xw, S[nb]);
    }
    publish_dt();
  };
  int64_t c = cbeg;
  for (; c + 1 < cend; c += 2) {
    chunk(c, Set0{});
    chunk(c + 1, Set1{});
  }
  if (c < cend) chunk(c, Set0{});
  if (OUT && cbeg < cend) {
    __syncthreads();
    if ((cend - cbeg) & 1) epilogue((cend - 1) * Q, Ragged{}, Set0{});
    else epilogue((cend - 1) * Q, Ragged{}, Set1{});
  }
  if constexpr (!OUT) {
    float* so = p.seg_state + seg * state_seg + state_off;
#pragma unroll
    for (int nb = 0; nb < NT; ++nb) *reinterpret_cast<ssd_f32x4_t*>(so + toff(nb)) = S[nb];
    if (slice == 0 && tid == 0) p.seg_dsum[seg * nbh + bh] = dsum;
    return;
  }

  if (p.final_state && seg == p.nseg - 1) {
    float* fs = p.final_state + state_off;
#pragma unroll
    for (int nb = 0; nb < NT; ++nb) *reinterpret_cast<ssd_f32x4_t*>(fs + toff(nb)) = S[nb];
  }
}

// The tiles of C B^T of one 64-step chunk of one (batch row, group), computed once for every head
// of the group and every slice of its channels (the twelve tiles gram_tile_i / gram_tile_j name,
// "Mamba 论文精读" sec. 4.2: the heads of a group share B and C).  Workgroup (b, g, c) of 4
// waves stages the chunk's B and C rows as the chunk kernel does (steps past the sequence take the
// last step's rows) and runs the same product, gram_tiles_nw4, so each tile holds the bits the
// chunk kernel would compute; tile k goes to gram[((b G + g) nch + c) 12 + k] as 64 lanes x 4 fp32
// in the product's output layout.
template <int N>
__global__ __launch_bounds__(256) void ssd_gram_kernel(const SsdArgs p) {
  constexpr int Q = kSsdChunk, LDB = N + 8, T = 256, kBCPer = 8 * N / T;
  static_assert(N % 32 == 0 && (8 * N) % T == 0, "dstate is a multiple of 32");
  __shared__ __align__(16) uint16_t s_b[Q * LDB];
  __shared__ __align__(16) uint16_t s_c[Q * LDB];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t L = p.seqlen, G = p.ngroups;
  const int64_t nch = (L + Q - 1) / Q;
  const int64_t blk = blockIdx.x;  // (batch row, group, chunk)
  const int64_t c = blk % nch, bg_i = blk / nch;
  const int64_t g = bg_i % G, b = bg_i / G;
  const uint16_t* bg = p.B + (b * L * G + g) * N;
  const uint16_t* cg = p.C + (b * L * G + g) * N;
  const int64_t bs = G * N, t0 = c * Q;
  ssd_u32x4_t rb[kBCPer], rc[kBCPer];
#pragma unroll
  for (int u = 0; u < kBCPer; ++u) {
    const int k = tid + u * T;
    const int c8 = k % (N / 8), j = k / (N / 8);
    const int64_t t = t0 + j < L ? t0 + j : L - 1;
    rb[u] = *reinterpret_cast<const ssd_u32x4_t*>(bg + t * bs + 8 * c8);
    rc[u] = *reinterpret_cast<const ssd_u32x4_t*>(cg + t * bs + 8 * c8);
  }
#pragma unroll
  for (int u = 0; u < kBCPer; ++u) {
    const int k = tid + u * T;
    const int c8 = k % (N / 8), j = k / (N / 8);
    *reinterpret_cast<ssd_u32x4_t*>(&s_b[j * LDB + 8 * c8]) = rb[u];
    *reinterpret_cast<ssd_u32x4_t*>(&s_c[j * LDB + 8 * c8]) = rc[u];
  }
  __syncthreads();
  ssd_f32x4_t gt[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) gt[s] = ssd_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  gram_tiles_nw4<N>([&](int r, int col) { return *reinterpret_cast<const ssd_u32x4_t*>(&s_b[r * LDB + col]); },
                    [&](int r, int col) { return *reinterpret_cast<const ssd_u32x4_t*>(&s_c[r * LDB + col]); },
                    wave, l16, q, gt);
  float* dst = p.gram_out + (blk * 12 + wave) * 256 + 4 * lane;
#pragma unroll
  for (int s = 0; s < 3; ++s) *reinterpret_cast<ssd_f32x4_t*>(dst + 4 * 256 * s) = gt[s];
}

// Composes the segment states in order, one thread per (batch row, head, channel, dstate index):
// from the caller's entering state (zero without one), S <- e^{sum dt A of segment s} S + S_end(s)
// for s = 0 .. nseg-2, leaving in seg_state[s] the state that enters segment s + 1.
template <int UNUSED = 0>
__global__ __launch_bounds__(256) void ssd_carry_kernel(const SsdArgs p, int32_t dstate) {
  const int64_t per_seg = p.batch * p.nheads * p.headdim * dstate;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= per_seg) return;
  const int64_t bh = e / (static_cast<int64_t>(p.headdim) * dstate);
  const int64_t nbh = p.batch * p.nheads;
  float st = p.init_state ? p.init_state[e] : 0.0f;
  for (int s = 0; s + 1 < p.nseg; ++s) {
    st = fmaf(hw_exp2(p.seg_dsum[s * nbh + bh]), st, p.seg_state[s * per_seg + e]);
    p.seg_state[s * per_seg + e] = st;
  }
}

// ---------------------------------------------------------------------------------------------
// One token of the layer, the recurrent view of "Mamba 论文精读" sec. 4.1 (O(1) work per token):
// for each (batch row b, head h, channel p) and its group g,
//   dt = softplus(dt[b,h] + dt_bias[h]);  S[b,h,p,:] = exp(dt A[h]) S[b,h,p,:] + dt x[b,h,p] B[b,g,:]
//   y[b,h,p] = (C[b,g,:] . S[b,h,p,:] + D[h] x[b,h,p]) * silu(z[b,h,p])
// The state is read and written once: a streaming kernel, with non-temporal state accesses.  A
// thread owns 4 consecutive dstate entries of one channel (16-byte state access, 8-byte B and C); the N/4 lanes of a channel add
// their partial read-outs with cross-lane shuffles.  The decay is one exp per channel.
// ---------------------------------------------------------------------------------------------
struct SsdUpdateArgs {
  float* state;          // (batch, nheads, headdim, dstate) fp32, in place
  const uint16_t* x;     // (batch, nheads, headdim) bf16
  const uint16_t* dt;    // (batch, nheads) bf16
  const float* A;        // (nheads)
  const uint16_t* B;     // (batch, ngroups, dstate) bf16
  const uint16_t* C;
  const float* D;        // (nheads) or NULL
  const uint16_t* z;     // like x, or NULL
  const float* dt_bias;  // (nheads) or NULL
  uint16_t* y;           // like x
  int64_t batch;
  int32_t nheads;
  int32_t headdim;
  int32_t ngroups;
  int32_t softplus;
};

constexpr int kSsdUpdateThreads = 256;

template <int N>
__global__ __launch_bounds__(kSsdUpdateThreads) void ssd_state_update_kernel(const SsdUpdateArgs p) {
  constexpr int TPC = N / 4;  // lanes per channel
  static_assert(N % 4 == 0 && TPC <= 64 && 64 % TPC == 0, "a channel's lanes share one wave");
  const int64_t H = p.nheads, P = p.headdim, G = p.ngroups;
  const int64_t nquads = p.batch * H * P * TPC;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * kSsdUpdateThreads + threadIdx.x;
  const bool ok = q < nquads;
  // a thread past the end works on quad 0 (in bounds) and stores nothing, so every lane of a
  // channel takes part in the shuffles
  const int64_t qq = ok ? q : 0;
  const int64_t ch = qq / TPC;  // (b * H + h) * P + p
  const int n0 = static_cast<int>(qq % TPC) * 4;
  const int64_t bh = ch / P;
  const int64_t h = bh % H, b = bh / H;
  const int64_t g = h / (H / G);
  const float xv = bf16_lo(p.x[ch]);
  const float v = bf16_lo(p.dt[bh]) + (p.dt_bias ? p.dt_bias[h] : 0.0f);
  const float dtv = p.softplus ? softplus_f32(v) : v;
  const float a = hw_exp2(dtv * (p.A[h] * kLog2e));
  const float w = dtv * xv;
  float* st = p.state + ch * N + n0;
  float4 s4 = load_stream(st);
  const uint2 b2 = *reinterpret_cast<const uint2*>(p.B + (b * G + g) * N + n0);
  const uint2 c2 = *reinterpret_cast<const uint2*>(p.C + (b * G + g) * N + n0);
  s4.x = fmaf(a, s4.x, w * bf16_lo(b2.x));
  s4.y = fmaf(a, s4.y, w * bf16_hi(b2.x));
  s4.z = fmaf(a, s4.z, w * bf16_lo(b2.y));
  s4.w = fmaf(a, s4.w, w * bf16_hi(b2.y));
  float yp = bf16_lo(c2.x) * s4.x;
  yp = fmaf(bf16_hi(c2.x), s4.y, yp);
  yp = fmaf(bf16_lo(c2.y), s4.z, yp);
  yp = fmaf(bf16_hi(c2.y), s4.w, yp);
  if (ok) store_stream(st, s4);
#pragma unroll
  for (int off = 1; off < TPC; off <<= 1) yp += __shfl_xor(yp, off, 64);
  if (ok && n0 == 0) {
    float yv = fmaf(p.D ? p.D[h] : 0.0f, xv, yp);
    if (p.z) yv *= silu_f32(bf16_lo(p.z[ch]));
    p.y[ch] = to_bf16(yv);
  }
}

using SsdUpdateKernel = void (*)(const SsdUpdateArgs);
SsdUpdateKernel ssd_update_kernel(int64_t dstate);

using SsdKernel = void (*)(const SsdArgs);
// The C B^T tile kernel for dstate (256 threads per workgroup, one workgroup per (batch row,
// group, chunk)), or NULL when dstate is not instantiated.
SsdKernel ssd_gram_kernel_for(int64_t dstate);
// The chunk kernel for (dstate, waves per workgroup, MODE), or NULL when that pair is not
// instantiated.
SsdKernel ssd_kernel(int64_t dstate, int waves, int mode);

}  // namespace ssm
