// ssm_device.hpp -- device-side helpers shared by the scan and decode kernels
// (gfx950 / CDNA4, wave64).  Storage types: fp32, or bf16 held as raw 16-bit
// patterns.  All arithmetic is fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// Scalar-cache loads: a pointer in the constant address space whose address is
// wave-uniform is read with s_load into SGPRs.
typedef __attribute__((address_space(4))) const uint32_t* const_u32_ptr;
typedef __attribute__((address_space(4))) const float* const_f32_ptr;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}
__device__ __forceinline__ uint16_t to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// Hardware transcendentals: v_exp_f32 = 2^x, v_log_f32 = log2(x), v_rcp_f32 = 1/x.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(v) = log(1 + e^v).  Above 20 the correction log1p(e^-v) < 2.1e-9 is
// below fp32 resolution of v and v is returned.  Otherwise, with u = e^v and
// w = fl(1 + u), log1p(u) = log(w) * u / (w - 1) (Goldberg's correction for
// the rounding of 1 + u; exact when w == 1, where the result is u), which
// keeps small steps (delta ~ 1e-4) accurate to a few ulp.
__device__ __forceinline__ float softplus_f32(float v) {
  const float u = hw_exp2(v * kLog2e);
  const float w = 1.0f + u;
  const float wm1 = w - 1.0f;
  const float lg = hw_log2(w) * kLn2;
  const float r = (wm1 == 0.0f) ? u : lg * (u * hw_rcp(wm1));
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

// Element `idx` of a B or C row read through the scalar cache (wave-uniform idx).  A bf16
// element is taken from the aligned dword that holds it (that dword never leaves the memory
// page of the element itself).  Generic path; the scan kernels use BcChunk below when they can.
template <bool BF16>
__device__ __forceinline__ float load_uniform(const void* base, int64_t idx) {
  if constexpr (BF16) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(base) + static_cast<uintptr_t>(idx) * 2u;
    const uint32_t w = *reinterpret_cast<const_u32_ptr>(addr & ~static_cast<uintptr_t>(3));
    return (addr & 2u) ? bf16_hi(w) : bf16_lo(w);
  } else {
    return *reinterpret_cast<const_f32_ptr>(reinterpret_cast<uintptr_t>(base) + static_cast<uintptr_t>(idx) * 4u);
  }
}

// B_t[n0 + j] and C_t[n0 + j] for the steps t = 0.. of one chunk, read through the scalar cache
// from a per-chunk base pointer so that every load has a compile-time offset.  `e0` is the
// element index of (b, t0, n0).  For bf16 with even N the host guarantees 4-byte aligned B and
// C, so element e0 + t*N + j lies in dword (e0 + t*N + j) / 2 of the tensor, in the high half
// when that index is odd; with NPL even (so e0 even) the half is known at compile time.
template <bool BF16, int N, int NPL>
struct BcChunk {
  static constexpr bool kPairs = BF16 && (N % 2 == 0);
  const void* base;
  int64_t e0;
  int par;  // (e0 & 1) for the bf16 pair path

  __device__ __forceinline__ BcChunk(const void* tensor, int64_t elem0) : base(tensor), e0(elem0) {
    par = static_cast<int>(elem0 & 1);
    if constexpr (kPairs) base = static_cast<const uint32_t*>(tensor) + (elem0 >> 1);
    else if constexpr (!BF16) base = static_cast<const float*>(tensor) + elem0;
  }

  __device__ __forceinline__ float get(int t, int j) const {
    if constexpr (kPairs) {
      const const_u32_ptr w = reinterpret_cast<const_u32_ptr>(reinterpret_cast<uintptr_t>(base));
      if constexpr (NPL % 2 == 0) {
        const uint32_t v = w[(t * N + j) >> 1];
        return (j & 1) ? bf16_hi(v) : bf16_lo(v);
      } else {
        const uint32_t v = w[(t * N + j + par) >> 1];
        return ((j + par) & 1) ? bf16_hi(v) : bf16_lo(v);
      }
    } else if constexpr (!BF16) {
      return reinterpret_cast<const_f32_ptr>(reinterpret_cast<uintptr_t>(base))[t * N + j];
    } else {
      return load_uniform<true>(base, e0 + static_cast<int64_t>(t) * N + j);
    }
  }
};

}  // namespace ssm
