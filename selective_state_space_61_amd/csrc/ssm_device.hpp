// ssm_device.hpp -- device-side helpers shared by the scan and decode kernels
// (gfx950 / CDNA4, wave64).  Storage types: fp32, or bf16 held as raw 16-bit
// patterns.  All arithmetic is fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even: one v_cvt_pk_bf16_f32 per pair on gfx950.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// Hardware transcendentals: v_exp_f32 = 2^x, v_log_f32 = log2(x), v_rcp_f32 = 1/x.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// 16-byte state accesses marked non-temporal: a decode step reads and writes each state once, and
// the next touch of that state is a whole model step later (every other layer's state in
// between), so keeping it in the caches only displaces other lines.
typedef float StreamF4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float* p) {
  const StreamF4 v = __builtin_nontemporal_load(reinterpret_cast<const StreamF4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(float* p, float4 v) {
  const StreamF4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<StreamF4*>(p));
}

// softplus(v) = log(1 + e^v).  Above 20 the correction log1p(e^-v) < 2.1e-9 is below the fp32
// resolution of v and v is returned.  Otherwise u = e^v, w = fl(1 + u) and
//   log1p(u) = log(w) + log(1 + e / w),  e = u - (w - 1)  (the exact rounding error of 1 + u;
// w - 1 is exact),  and log(1 + e/w) is replaced by e: |e| <= 2^-24 w, so the dropped terms are
// below 2^-24 * u * |e| + e^2, far under one ulp of the result.  For u < 2^-24, w = 1 and the
// result is u exactly.  Small steps (delta ~ 1e-4) stay accurate to about an ulp.
__device__ __forceinline__ float softplus_f32(float v) {
  const float u = hw_exp2(v * kLog2e);
  const float w = 1.0f + u;
  const float e = u - (w - 1.0f);
  const float r = fmaf(hw_log2(w), kLn2, e);
  return v > 20.0f ? v : r;
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z).
__device__ __forceinline__ float silu_f32(float z) { return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e)); }

// ---------------------------------------------------------------------------------------------
// VEC consecutive elements of a (bf16 | fp32) tensor kept as raw 32-bit words between the
// load and the conversion, so the load can be issued a chunk ahead.
// ---------------------------------------------------------------------------------------------
template <bool BF16, int VEC>
struct RawVec {
  static constexpr int kBytes = VEC * (BF16 ? 2 : 4);
  static constexpr int kWords = kBytes < 4 ? 1 : kBytes / 4;
  uint32_t w[kWords];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = 0u;
  }

  // Loads elements [idx, idx + VEC) of `base`; only the first `nvalid` are read (the rest are
  // zero).  `vec_ok` says that a single aligned vector load is allowed.
  __device__ __forceinline__ void load(const void* __restrict__ base, int64_t idx, int nvalid, bool vec_ok) {
    if (vec_ok && nvalid == VEC) {
      if constexpr (kBytes == 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + idx * (BF16 ? 2 : 4));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      } else if constexpr (kBytes == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const char*>(base) + idx * (BF16 ? 2 : 4));
        w[0] = v.x; w[1] = v.y;
      } else if constexpr (kBytes == 4) {
        w[0] = *reinterpret_cast<const uint32_t*>(static_cast<const char*>(base) + idx * (BF16 ? 2 : 4));
      } else {
        w[0] = static_cast<const uint16_t*>(base)[idx];
      }
      return;
    }
    zero();
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      if (v < nvalid) {
        uint32_t e;
        if constexpr (BF16) e = static_cast<const uint16_t*>(base)[idx + v];
        else e = static_cast<const uint32_t*>(base)[idx + v];
        if constexpr (BF16) w[v >> 1] |= (v & 1) ? (e << 16) : e;
        else w[v] = e;
      }
    }
  }

  __device__ __forceinline__ float get(int v) const {
    if constexpr (BF16) return (v & 1) ? bf16_hi(w[v >> 1]) : bf16_lo(w[v >> 1]);
    else return __builtin_bit_cast(float, w[v]);
  }

  // an (empty) use of the words: the compiler waits for their load here, on every path through it
  __device__ __forceinline__ void consume() const {
#pragma unroll
    for (int i = 0; i < kWords; ++i) asm volatile("" ::"v"(w[i]));
  }
};

// Stores VEC fp32 values as (bf16 | fp32) at base[idx ...]; only the first `nvalid` when the
// vector store is not allowed.
template <bool BF16, int VEC>
__device__ __forceinline__ void store_vec(void* __restrict__ base, int64_t idx, const float (&val)[VEC], int nvalid,
                                          bool vec_ok) {
  constexpr int kBytes = VEC * (BF16 ? 2 : 4);
  char* p = static_cast<char*>(base) + idx * (BF16 ? 2 : 4);
  if (vec_ok && nvalid == VEC) {
    if constexpr (BF16) {
      if constexpr (kBytes == 16) {
        *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3]),
                                                  pack_bf16x2(val[4], val[5]), pack_bf16x2(val[6], val[7]));
      } else if constexpr (kBytes == 8) {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3]));
      } else if constexpr (kBytes == 4) {
        *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(val[0], val[1]);
      } else {
        *reinterpret_cast<uint16_t*>(p) = to_bf16(val[0]);
      }
    } else {
      if constexpr (kBytes == 16) {
        *reinterpret_cast<float4*>(p) = make_float4(val[0], val[1], val[2], val[3]);
      } else if constexpr (kBytes == 8) {
        *reinterpret_cast<float2*>(p) = make_float2(val[0], val[1]);
      } else {
        *reinterpret_cast<float*>(p) = val[0];
      }
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    if (v < nvalid) {
      if constexpr (BF16) reinterpret_cast<uint16_t*>(p)[v] = to_bf16(val[v]);
      else reinterpret_cast<float*>(p)[v] = val[v];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Row broadcasts (DPP row_newbcast:K, gfx90a and later): every lane of a 16-lane row reads lane K
// of that row.  A register whose lane (row r, k) holds the value for step k (the same in every
// row) hands step K's value to all 64 lanes without a memory access.
// ---------------------------------------------------------------------------------------------
// (Every lane has a source in its row, so bound_ctrl changes nothing; it spares the compiler a
// register for the unused "old" value, one v_mov per broadcast that it cannot fold.)
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  static_assert(K >= 0 && K < 16, "row_newbcast selects one of 16 lanes");
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + K, 0xF, 0xF, true));
}

// ---------------------------------------------------------------------------------------------
// One step of the recurrence for a lane's chains, fused with the read-out of the PREVIOUS step:
//   read-out (step t-1):  yp = sum_j C_{t-1}[j] * h[j]           (h still holds h_{t-1})
//   update   (step t):    h[j] = exp2(dt * a2[j]) * h[j] + B_t[j] * w
// B_t and C_{t-1} come from DPP row broadcasts (lanes KB and KC of each 16-lane row).  The
// compiler does not fold a broadcast into a multiply-accumulate, so the step is written as one
// instruction sequence.  Its order obeys the gfx9 VALU hazards, which the compiler cannot enforce
// inside an asm statement:
//   * a DPP instruction reads each VGPR operand (the broadcast source, the other source and a
//     multiply-accumulate's accumulator) at least two instructions after the VALU write of it
//     (inside the block), and its first DPP instruction comes late enough that any write made
//     just before the block is two or more instructions old;
//   * no instruction reads a v_exp_f32 result sooner than two instructions after it;
//   * a chain's h is read by its read-out before the update overwrites it.
// The block has only VALU instructions: no memory access, no EXEC change.
// ---------------------------------------------------------------------------------------------
#define SSM_DPP_KB "row_newbcast:%[kb] row_mask:0xf bank_mask:0xf"
#define SSM_DPP_KC "row_newbcast:%[kc] row_mask:0xf bank_mask:0xf"

template <int KB, int KC>
__device__ __forceinline__ float step_readout1(float dt, float w, float a2, float b, float c, float& h) {
  float t0, u0, yp;
  asm("v_mul_f32 %[t0], %[dt], %[a0]\n\t"
      "v_exp_f32 %[t0], %[t0]\n\t"
      "v_mul_f32_dpp %[u0], %[b0], %[w] " SSM_DPP_KB "\n\t"
      "v_mul_f32_dpp %[yp], %[c0], %[h0] " SSM_DPP_KC "\n\t"
      "v_fma_f32 %[h0], %[t0], %[h0], %[u0]"
      : [t0] "=&v"(t0), [u0] "=&v"(u0), [yp] "=&v"(yp), [h0] "+v"(h)
      : [dt] "v"(dt), [w] "v"(w), [a0] "v"(a2), [b0] "v"(b), [c0] "v"(c), [kb] "i"(KB), [kc] "i"(KC));
  return yp;
}

template <int KB, int KC>
__device__ __forceinline__ float step_readout2(float dt, float w, const float* a2, const float* b, const float* c,
                                               float* h) {
  float t0, t1, u0, u1, ya;
  asm("v_mul_f32 %[t0], %[dt], %[a0]\n\t"
      "v_mul_f32 %[t1], %[dt], %[a1]\n\t"
      "v_exp_f32 %[t0], %[t0]\n\t"
      "v_exp_f32 %[t1], %[t1]\n\t"
      "v_mul_f32_dpp %[u0], %[b0], %[w] " SSM_DPP_KB "\n\t"
      "v_mul_f32_dpp %[ya], %[c0], %[h0] " SSM_DPP_KC "\n\t"
      "v_mul_f32_dpp %[u1], %[b1], %[w] " SSM_DPP_KB "\n\t"
      "v_fma_f32 %[h0], %[t0], %[h0], %[u0]\n\t"
      "v_fmac_f32_dpp %[ya], %[c1], %[h1] " SSM_DPP_KC "\n\t"
      "v_fma_f32 %[h1], %[t1], %[h1], %[u1]"
      : [t0] "=&v"(t0), [t1] "=&v"(t1), [u0] "=&v"(u0), [u1] "=&v"(u1), [ya] "=&v"(ya), [h0] "+v"(h[0]),
        [h1] "+v"(h[1])
      : [dt] "v"(dt), [w] "v"(w), [a0] "v"(a2[0]), [a1] "v"(a2[1]), [b0] "v"(b[0]), [b1] "v"(b[1]),
        [c0] "v"(c[0]), [c1] "v"(c[1]), [kb] "i"(KB), [kc] "i"(KC));
  return ya;
}

template <int KB, int KC>
__device__ __forceinline__ float step_readout4(float dt, float w, const float* a2, const float* b, const float* c,
                                               float* h) {
  float t0, t1, t2, t3, u0, u1, u2, u3, yp;
  asm("v_mul_f32 %[t0], %[dt], %[a0]\n\t"
      "v_mul_f32 %[t1], %[dt], %[a1]\n\t"
      "v_mul_f32 %[t2], %[dt], %[a2]\n\t"
      "v_mul_f32 %[t3], %[dt], %[a3]\n\t"
      "v_exp_f32 %[t0], %[t0]\n\t"
      "v_exp_f32 %[t1], %[t1]\n\t"
      "v_exp_f32 %[t2], %[t2]\n\t"
      "v_exp_f32 %[t3], %[t3]\n\t"
      "v_mul_f32_dpp %[u0], %[b0], %[w] " SSM_DPP_KB "\n\t"
      "v_mul_f32_dpp %[yp], %[c0], %[h0] " SSM_DPP_KC "\n\t"
      "v_mul_f32_dpp %[u1], %[b1], %[w] " SSM_DPP_KB "\n\t"
      "v_fma_f32 %[h0], %[t0], %[h0], %[u0]\n\t"
      "v_fmac_f32_dpp %[yp], %[c1], %[h1] " SSM_DPP_KC "\n\t"
      "v_mul_f32_dpp %[u2], %[b2], %[w] " SSM_DPP_KB "\n\t"
      "v_fma_f32 %[h1], %[t1], %[h1], %[u1]\n\t"
      "v_fmac_f32_dpp %[yp], %[c2], %[h2] " SSM_DPP_KC "\n\t"
      "v_mul_f32_dpp %[u3], %[b3], %[w] " SSM_DPP_KB "\n\t"
      "v_fma_f32 %[h2], %[t2], %[h2], %[u2]\n\t"
      "v_fmac_f32_dpp %[yp], %[c3], %[h3] " SSM_DPP_KC "\n\t"
      "v_fma_f32 %[h3], %[t3], %[h3], %[u3]"
      : [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3), [u0] "=&v"(u0), [u1] "=&v"(u1),
        [u2] "=&v"(u2), [u3] "=&v"(u3), [yp] "=&v"(yp), [h0] "+v"(h[0]), [h1] "+v"(h[1]), [h2] "+v"(h[2]),
        [h3] "+v"(h[3])
      : [dt] "v"(dt), [w] "v"(w), [a0] "v"(a2[0]), [a1] "v"(a2[1]), [a2] "v"(a2[2]), [a3] "v"(a2[3]),
        [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]), [c0] "v"(c[0]), [c1] "v"(c[1]),
        [c2] "v"(c[2]), [c3] "v"(c[3]), [kb] "i"(KB), [kc] "i"(KC));
  return yp;
}

// NPL chains: blocks of 4 (or the 1 / 2 forms); each block is hazard-safe on its own, so blocks
// can follow one another in any order.
template <int NPL, int KB, int KC>
__device__ __forceinline__ float step_readout(float dt, float w, const float* a2, const float* b, const float* c,
                                              float* h) {
  if constexpr (NPL == 1) {
    return step_readout1<KB, KC>(dt, w, a2[0], b[0], c[0], h[0]);
  } else if constexpr (NPL == 2) {
    return step_readout2<KB, KC>(dt, w, a2, b, c, h);
  } else {
    static_assert(NPL % 4 == 0, "chains per lane: 1, 2 or a multiple of 4");
    float yp = step_readout4<KB, KC>(dt, w, a2, b, c, h);
#pragma unroll
    for (int g = 1; g < NPL / 4; ++g) yp += step_readout4<KB, KC>(dt, w, a2 + 4 * g, b + 4 * g, c + 4 * g, h + 4 * g);
    return yp;
  }
}

#undef SSM_DPP_KB
#undef SSM_DPP_KC

// NPL consecutive elements of one B or C row (state indices n0 .. n0+NPL-1 of step t), loaded by
// one lane as raw words and widened to fp32.  For bf16 with even NPL the elements come in
// 4-byte-aligned pairs (the host requires 4-byte aligned B and C for an even dstate).
template <bool BF16, int NPL>
struct BcRow {
  static constexpr int kWords = BF16 ? (NPL + 1) / 2 : NPL;
  uint32_t w[kWords];

  __device__ __forceinline__ void load(const void* __restrict__ tensor, int64_t e, bool valid) {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = 0u;
    if (!valid) return;
    if constexpr (BF16 && NPL == 1) {
      w[0] = static_cast<const uint16_t*>(tensor)[e];
    } else if constexpr (BF16) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(tensor) + e);
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = p[i];
    } else {
      const uint32_t* p = static_cast<const uint32_t*>(tensor) + e;
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = p[i];
    }
  }

  // the same words loaded on every path (e must be in range): no merge with a zero fill, so the
  // compiler never copies the destination registers, which would wait for the load at once
  __device__ __forceinline__ void load_in_range(const void* __restrict__ tensor, int64_t e) {
    if constexpr (BF16 && NPL == 1) {
      w[0] = static_cast<const uint16_t*>(tensor)[e];
    } else if constexpr (BF16) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(tensor) + e);
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = p[i];
    } else {
      const uint32_t* p = static_cast<const uint32_t*>(tensor) + e;
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = p[i];
    }
  }

  __device__ __forceinline__ float get(int j) const {
    if constexpr (BF16) return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
    else return __builtin_bit_cast(float, w[j]);
  }
};

// Factor of the exact zero-order-hold input term.  With tt = Delta A log2(e) and a = 2^tt =
// e^(Delta A), the ZOH input matrix is Bbar = (e^(Delta A) - 1) / A B = Delta B phi(Delta A),
// phi(z) = (e^z - 1) / z ("Mamba 论文精读" sec. 2.2).  This returns m = (a - 1) / tt = ln2 phi, so
// that Bbar x = B (Delta x log2 e) m.  For |tt| < 1 the division uses log2(a) in place of tt
// (Kahan's expm1 device: the rounding of a cancels between numerator and denominator, so no
// precision is lost to a - 1 when a is near 1); elsewhere a - 1 does not cancel, and tt itself is
// used, which stays right when a underflows.  a == 1 gives the limit ln2.
__device__ __forceinline__ float zoh_factor(float tt, float a) {
  const float l = fabsf(tt) < 1.0f ? hw_log2(a) : tt;
  return a == 1.0f ? kLn2 : (a - 1.0f) * hw_rcp(l);
}

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, workgroups dealt round robin

// Logical workgroup index for hardware index i of n: the first n - n % 8 workgroups are regrouped
// so that the hardware indices i with i % 8 == x (one XCD, with its own L2) take logical indices
// x * (n / 8) .. (x + 1) * (n / 8) - 1; the last n % 8 keep their index.  A bijection on [0, n):
// workgroups with neighbouring logical indices share an XCD and its L2.
__device__ __forceinline__ int64_t xcd_local(int64_t i, int64_t n) {
  const int64_t per = n / kXcds;
  if (i >= per * kXcds) return i;
  return (i % kXcds) * per + i / kXcds;
}

// compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace ssm
