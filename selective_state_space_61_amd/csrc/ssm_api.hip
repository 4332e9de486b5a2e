// ssm_api.hip -- the C ABI declared in include/ssm.h: host-side validation, launch-shape choice
// and kernel launches on the caller's stream.  No torch types, no exceptions across the ABI.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/ssm.h"
#include "scan_table.hpp"
#include "scan_rows_table.hpp"
#include "scan_time_table.hpp"
#include "state_update.hpp"
#include "conv1d.hpp"
#include "scan_bwd.hpp"
#include "ssd_fwd.hpp"
#include "scan_bwd_rows.hpp"

namespace {

thread_local char g_err[512] = "";

ssm_status_t fail(ssm_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

struct Range {
  const void* p;
  int64_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Arg {
  const void* p;
  int64_t align;
  const char* name;
};

// first non-NULL argument not aligned to its element size, or NULL
const Arg* misaligned(const Arg* args, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (args[i].p && !aligned(args[i].p, static_cast<uintptr_t>(args[i].align))) return &args[i];
  return nullptr;
}

bool dstate_supported(int64_t n) {
  return n == 1 || n == 2 || n == 4 || n == 8 || n == 16 || n == 32 || n == 64;
}

// chains per lane the scan kernels are instantiated for, given N: at most 8 scan waves per
// workgroup (next to the IO waves, within 1024 threads)
bool npl_supported(int64_t n, int npl) {
  if (npl != 1 && npl != 2 && npl != 4 && npl != 8 && npl != 16) return false;
  if (npl > n || (n % npl) != 0) return false;
  return n / npl <= 8;
}

// Measured on MI355X (dstate 16): 4 chains per lane (4 scan waves next to the 4 IO waves) is
// fastest for both the 130M- and 2.8B-shaped workloads.
int default_npl(int64_t n, int64_t workgroups) {
  (void)workgroups;
  int npl = n >= 4 ? 4 : static_cast<int>(n);
  while (n / npl > 8) npl *= 2;  // at most 8 scan waves per workgroup
  return npl;
}

// compute units of the current device, cached per device
int device_cus() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    __atomic_store_n(&cache[dev], cus, __ATOMIC_RELAXED);
  }
  return cus;
}

// ---- kernel tables -----------------------------------------------------------------------------
using CarryKernel = void (*)(const ssm::ScanArgs);
using UpdateKernel = void (*)(const ssm::UpdateArgs);

CarryKernel carry_kernel(int64_t n) {
  switch (n) {
    case 1: return ssm::scan_carry_kernel<1>;
    case 2: return ssm::scan_carry_kernel<2>;
    case 4: return ssm::scan_carry_kernel<4>;
    case 8: return ssm::scan_carry_kernel<8>;
    case 16: return ssm::scan_carry_kernel<16>;
    case 32: return ssm::scan_carry_kernel<32>;
    case 64: return ssm::scan_carry_kernel<64>;
    default: return nullptr;
  }
}

using BwdKernel = void (*)(const ssm::BwdArgs);
using BwdReduceKernel = void (*)(const ssm::BwdReduceArgs);

// backward instantiations: chains per lane min(N, 4) up to N 16, so at most 4 scan waves
// (measured on MI355X: 2 chains per lane with 8 scan waves was 13% slower on the 130M shape);
// N 32 and 64 keep 4 scan waves with 8 and 16 chains per lane on 8- and 4-step chunks
template <bool BF16, bool ZOH>
BwdKernel bwd_kernel(int64_t n) {
  switch (n) {
    case 1: return ssm::scan_bwd_kernel<BF16, 1, 1, ZOH>;
    case 2: return ssm::scan_bwd_kernel<BF16, 2, 2, ZOH>;
    case 4: return ssm::scan_bwd_kernel<BF16, 4, 4, ZOH>;
    case 8: return ssm::scan_bwd_kernel<BF16, 8, 4, ZOH>;
    case 16: return ssm::scan_bwd_kernel<BF16, 16, 4, ZOH>;
    case 32: return ssm::scan_bwd_kernel<BF16, 32, 8, ZOH>;
    case 64: return ssm::scan_bwd_kernel<BF16, 64, 16, ZOH>;
    default: return nullptr;
  }
}

int bwd_npl(int64_t n) { return n <= 4 ? static_cast<int>(n) : (n <= 16 ? 4 : static_cast<int>(n / 4)); }

using ConvKernel = void (*)(const ssm::ConvArgs);
using ConvUpdateKernel = void (*)(const ssm::ConvUpdateArgs);

template <bool BF16>
ConvKernel conv_kernel(int64_t width) {
  switch (width) {
    case 1: return ssm::causal_conv1d_kernel<BF16, 1>;
    case 2: return ssm::causal_conv1d_kernel<BF16, 2>;
    case 3: return ssm::causal_conv1d_kernel<BF16, 3>;
    case 4: return ssm::causal_conv1d_kernel<BF16, 4>;
    default: return nullptr;
  }
}

template <bool BF16>
ConvUpdateKernel conv_update_kernel(int64_t width) {
  switch (width) {
    case 1: return ssm::conv1d_update_kernel<BF16, 1>;
    case 2: return ssm::conv1d_update_kernel<BF16, 2>;
    case 3: return ssm::conv1d_update_kernel<BF16, 3>;
    case 4: return ssm::conv1d_update_kernel<BF16, 4>;
    default: return nullptr;
  }
}

template <bool BF16, bool ZOH>
UpdateKernel update_kernel(int64_t n) {
  switch (n) {
    case 1: return ssm::state_update_kernel<BF16, 1, ZOH>;
    case 2: return ssm::state_update_kernel<BF16, 2, ZOH>;
    case 4: return ssm::state_update_kernel<BF16, 4, ZOH>;
    case 8: return ssm::state_update_kernel<BF16, 8, ZOH>;
    case 16: return ssm::state_update_kernel<BF16, 16, ZOH>;
    case 32: return ssm::state_update_kernel<BF16, 32, ZOH>;
    case 64: return ssm::state_update_kernel<BF16, 64, ZOH>;
    default: return nullptr;
  }
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// ---- segment scratch: one growable device buffer per (device, stream) ----------------------------
// A buffer that a larger call outgrows is retired, never freed: work already enqueued, or a graph
// captured earlier on that stream, may still hold its address, so freeing it could let a later
// replay write to memory that belongs to someone else.  Retired buffers live until the process
// ends (each is at most the size of the largest call before it).
struct Scratch {
  float* ptr = nullptr;
  int64_t floats = 0;
};
std::mutex g_scratch_mu;
std::map<std::pair<int, uintptr_t>, Scratch> g_scratch;
std::vector<void*> g_retired;

ssm_status_t get_scratch(hipStream_t stream, int64_t floats, float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  Scratch& s = g_scratch[{dev, reinterpret_cast<uintptr_t>(stream)}];
  if (s.floats < floats) {
    void* p = nullptr;
    e = hipMalloc(&p, static_cast<size_t>(floats) * sizeof(float));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "hipMalloc(%lld floats): %s", (long long)floats, hipGetErrorString(e));
    if (s.ptr) g_retired.push_back(s.ptr);
    s.ptr = static_cast<float*>(p);
    s.floats = floats;
  }
  *out = s.ptr;
  return SSM_OK;
}

ssm_status_t check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return SSM_OK;
}

}  // namespace

extern "C" {

const char* ssm_status_string(ssm_status_t s) {
  switch (s) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_INVALID_ARG: return "SSM_ERR_INVALID_ARG";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED";
    case SSM_ERR_MISALIGNED: return "SSM_ERR_MISALIGNED";
    case SSM_ERR_HIP: return "SSM_ERR_HIP";
  }
  return "SSM_ERR_UNKNOWN";
}

const char* ssm_last_error(void) { return g_err; }

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

}  // extern "C"

namespace {

// Where the split-sequence scan's segment summaries go: the per-(device, stream) buffer of
// get_scratch (fixed == nullptr), or a caller-provided buffer of fixed_floats fp32 (the
// allocation-free entry point), in which case nothing is allocated and a call needing more is
// rejected before any launch.
struct ScratchSource {
  float* fixed;
  int64_t fixed_floats;
};

ssm_status_t scan_fwd_impl(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                           const void* x, const void* delta, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* delta_bias, int delta_softplus, void* y,
                           float* last_state, void* stream, const ssm_scan_opts_t* opts, ScratchSource src,
                           float* ckpt = nullptr) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 0)
    return fail(SSM_ERR_INVALID_ARG, "negative size (batch=%lld seqlen=%lld dim=%lld dstate=%lld)",
                (long long)batch, (long long)seqlen, (long long)dim, (long long)dstate);
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (!dstate_supported(dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not in {1,2,4,8,16,32,64}", (long long)dstate);
  const int64_t es = dtype == SSM_BF16 ? 2 : 4;
  int64_t n_bld, n_bln, n_bdn, n_dn;
  if (!mul_ok(batch, seqlen, &n_bld) || !mul_ok(n_bld, dim, &n_bld) || !mul_ok(n_bld, es, &n_bld) ||
      !mul_ok(batch, seqlen, &n_bln) || !mul_ok(n_bln, dstate, &n_bln) || !mul_ok(n_bln, es, &n_bln) ||
      !mul_ok(batch, dim, &n_bdn) || !mul_ok(n_bdn, dstate * 4, &n_bdn) || !mul_ok(dim, dstate * 4, &n_dn))
    return fail(SSM_ERR_INVALID_ARG, "tensor size overflows int64");
  const int64_t nch = batch * dim;
  if (nch == 0) return SSM_OK;  // nothing to compute, nothing to write
  if (seqlen > 0) {
    if (!x || !delta || !A || !B || !C || !y)
      return fail(SSM_ERR_INVALID_ARG, "NULL required pointer (x, delta, A, B, C and y are required)");
  }
  const Arg args[] = {{x, es, "x"}, {delta, es, "delta"}, {A, 4, "A"}, {B, es, "B"}, {C, es, "C"},
                      {D, 4, "D"}, {z, es, "z"}, {delta_bias, 4, "delta_bias"}, {y, es, "y"},
                      {last_state, 4, "last_state"}, {ckpt, 4, "checkpoints"}};
  if (const Arg* bad = misaligned(args, sizeof args / sizeof args[0]))
    return fail(SSM_ERR_MISALIGNED, "%s (%p) is not aligned to its element size", bad->name, bad->p);
  if (dtype == SSM_BF16 && (dstate % 2) == 0 && seqlen > 0 && !(aligned(B, 4) && aligned(C, 4)))
    return fail(SSM_ERR_MISALIGNED, "bf16 B and C must be 4-byte aligned when dstate is even");
  if (!aligned(ckpt, 16)) return fail(SSM_ERR_MISALIGNED, "checkpoints (%p) is not 16-byte aligned", ckpt);
  // checkpoints: (batch, ceil(seqlen / 32), dim, dstate) fp32
  int64_t n_ck = 0;
  if (ckpt && (!mul_ok(batch, (seqlen + 31) / 32, &n_ck) || !mul_ok(n_ck, dstate * 4, &n_ck) ||
               !mul_ok(n_ck, dim, &n_ck)))
    return fail(SSM_ERR_INVALID_ARG, "tensor size overflows int64");
  const Range rx{x, n_bld}, rd{delta, n_bld}, rz{z, n_bld}, rB{B, n_bln}, rC{C, n_bln}, rA{A, n_dn},
      rD{D, dim * 4}, rb{delta_bias, dim * 4}, ry{seqlen > 0 ? y : nullptr, n_bld}, rs{last_state, n_bdn},
      rk{seqlen > 0 ? ckpt : nullptr, n_ck};
  for (Range in : {rx, rd, rz, rB, rC, rA, rD, rb})
    if (overlap(ry, in) || overlap(rs, in) || overlap(rk, in))
      return fail(SSM_ERR_INVALID_ARG, "an output overlaps an input");
  if (overlap(ry, rs)) return fail(SSM_ERR_INVALID_ARG, "y overlaps last_state");
  if (overlap(rk, ry) || overlap(rk, rs)) return fail(SSM_ERR_INVALID_ARG, "checkpoints overlap y or last_state");

  if (ckpt && (dstate != 16 || (opts && (opts->bbar_mode != SSM_BBAR_DELTA_B || opts->segments > 1 ||
                                          (opts->layout != SSM_LAYOUT_AUTO && opts->layout != SSM_LAYOUT_STATE_ROWS) ||
                                          (opts->chains_per_lane != 0 && opts->chains_per_lane != 4)))))
    return fail(SSM_ERR_UNSUPPORTED,
                "checkpoints need the state-row layout: dstate 16, SSM_BBAR_DELTA_B, one segment");

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (seqlen == 0) {
    if (last_state) {
      const int64_t n = nch * dstate;
      hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                         last_state, n);
      return check_launch("fill_zero_kernel");
    }
    return SSM_OK;
  }

  // launch shape
  const int64_t ncb = (dim + 63) / 64;
  const int64_t base_wgs = ncb * batch;
  if (opts) {
    if (opts->segments < 0 || opts->chains_per_lane < 0)
      return fail(SSM_ERR_INVALID_ARG, "negative launch-shape override");
    if (opts->bbar_mode != SSM_BBAR_DELTA_B && opts->bbar_mode != SSM_BBAR_ZOH)
      return fail(SSM_ERR_UNSUPPORTED, "bbar_mode %d is not SSM_BBAR_DELTA_B or SSM_BBAR_ZOH", (int)opts->bbar_mode);
    for (int32_t r : opts->reserved)
      if (r != 0) return fail(SSM_ERR_INVALID_ARG, "ssm_scan_opts_t.reserved must be zero");
    if (opts->layout != SSM_LAYOUT_AUTO && opts->layout != SSM_LAYOUT_CHANNEL_LANES &&
        opts->layout != SSM_LAYOUT_STATE_ROWS && opts->layout != SSM_LAYOUT_TIME_SCAN)
      return fail(SSM_ERR_UNSUPPORTED, "layout %d is not an ssm_scan_layout_t", (int)opts->layout);
    if (opts->channel_groups < 0 || opts->channel_groups > ssm::kRowsMaxScanWaves)
      return fail(SSM_ERR_UNSUPPORTED, "channel_groups %d not in 0..%d", (int)opts->channel_groups,
                  ssm::kRowsMaxScanWaves);
  }
  const bool split_auto = !(opts && opts->segments > 0) && base_wgs < 160;

  // The time-parallel layout (on request only: measured slower than the split sequence on the
  // genomics shape, which is the case it targets).
  if (opts && opts->layout == SSM_LAYOUT_TIME_SCAN) {
    if (dstate != 16 || opts->bbar_mode != SSM_BBAR_DELTA_B || opts->segments > 1 || opts->channel_groups != 0 ||
        (opts->chains_per_lane != 0 && opts->chains_per_lane != 4))
      return fail(SSM_ERR_UNSUPPORTED,
                  "SSM_LAYOUT_TIME_SCAN needs dstate 16, SSM_BBAR_DELTA_B, one segment and no channel groups");
    if (opts->chunk_steps != 0 && opts->chunk_steps != 256 && opts->chunk_steps != 512)
      return fail(SSM_ERR_UNSUPPORTED, "chunk_steps %d is not 256 or 512 for SSM_LAYOUT_TIME_SCAN",
                  (int)opts->chunk_steps);
    if (nch > 0x7fffffff) return fail(SSM_ERR_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)nch);
    const ssm::TimeKernel tk = ssm::time_kernel(dtype == SSM_BF16, opts->chunk_steps == 256 ? 4 : 8);
    ssm::ScanArgs a{};
    a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.Dskip = D; a.z = z; a.delta_bias = delta_bias;
    a.y = y; a.last_state = last_state;
    a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.seg_len = seqlen;
    a.nseg = 1;
    a.softplus = delta_softplus ? 1 : 0;
    hipLaunchKernelGGL(tk, dim3(static_cast<unsigned>(nch)), dim3(ssm::kTimeThreads), 0, st, a);
    return check_launch("scan (time parallel)");
  }

  // The state-row layout: dstate 16, Delta B, whole sequences (no split).  The automatic choice
  // takes it whenever it applies.
  {
    const int layout = opts ? opts->layout : SSM_LAYOUT_AUTO;
    const bool zoh_mode = opts && opts->bbar_mode == SSM_BBAR_ZOH;
    const bool rows_fit = dstate == 16 && !zoh_mode && !(opts && opts->segments > 1) &&
                          !(opts && opts->chains_per_lane != 0 && opts->chains_per_lane != 4);
    if (layout == SSM_LAYOUT_STATE_ROWS && !rows_fit)
      return fail(SSM_ERR_UNSUPPORTED,
                  "SSM_LAYOUT_STATE_ROWS needs dstate 16, SSM_BBAR_DELTA_B, one segment and 4 chains per lane");
    if (layout == SSM_LAYOUT_CHANNEL_LANES && opts && opts->channel_groups != 0)
      return fail(SSM_ERR_UNSUPPORTED, "channel_groups applies to SSM_LAYOUT_STATE_ROWS only");
    const bool use_rows =
        rows_fit && (layout == SSM_LAYOUT_STATE_ROWS || (layout == SSM_LAYOUT_AUTO && (!split_auto || ckpt)));
    if (use_rows) {
      const int cus = device_cus();
      int S = opts ? opts->channel_groups : 0;
      if (S == 0) {
        // cost = rounds of one workgroup per CU x scan waves on the busiest SIMD (three SIMDs take
        // scan waves); among equal costs, the one whose rounds leave the fewest CUs idle, then
        // the larger workgroup.  Measured on MI355X: 3 groups (256 workgroups) for the 130M
        // shape, 5 groups (256 workgroups) for the 2.8B shape.
        int64_t best = -1, best_idle = 0;
        for (int c = 1; c <= ssm::kRowsMaxScanWaves; ++c) {
          const int64_t wgs = batch * ((dim + 16 * c - 1) / (16 * c));
          const int64_t rounds = (wgs + cus - 1) / cus;
          const int64_t cost = rounds * ((c + 2) / 3);
          const int64_t idle = rounds * cus - wgs;
          if (best < 0 || cost < best || (cost == best && idle <= best_idle)) {
            best = cost;
            best_idle = idle;
            S = c;
          }
        }
      }
      const int64_t rncb = (dim + 16 * S - 1) / (16 * S);
      int64_t rgrid;
      if (!mul_ok(rncb, batch, &rgrid) || rgrid > 0x7fffffff)
        return fail(SSM_ERR_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)rncb * batch);
      const ssm::RowsVariants& rv = ssm::rows_table(dtype == SSM_BF16).v[S];
      const int chunk_opt = opts ? opts->chunk_steps : 0;
      if (chunk_opt != 0 && chunk_opt != 16 && chunk_opt != 32)
        return fail(SSM_ERR_UNSUPPORTED, "chunk_steps %d is not 16 or 32", chunk_opt);
      if (chunk_opt == 32 && !rv.k[1])
        return fail(SSM_ERR_UNSUPPORTED, "chunk_steps 32 does not fit LDS with %d channel groups", S);
      const bool ch32 = chunk_opt == 32 || (chunk_opt == 0 && rv.k[1] && rgrid <= cus);
      ssm::ScanArgs a{};
      a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.Dskip = D; a.z = z; a.delta_bias = delta_bias;
      a.y = y; a.last_state = last_state; a.ckpt = ckpt;
      a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.seg_len = seqlen;
      a.nseg = 1;
      a.ncb = static_cast<int32_t>(rncb);
      a.softplus = delta_softplus ? 1 : 0;
      const int64_t vmax = 16 / es;
      a.vec_ok = (dim % vmax == 0) && aligned(x, 16) && aligned(delta, 16) && aligned(y, 16) && (!z || aligned(z, 16));
      hipLaunchKernelGGL(rv.k[ch32 ? 1 : 0], dim3(static_cast<unsigned>(rgrid)), dim3(64 * ssm::kRowsWaves), 0, st, a);
      return check_launch("scan (state rows)");
    }
  }
  if (ckpt) return fail(SSM_ERR_UNSUPPORTED, "checkpoints need the state-row layout");
  int npl = default_npl(dstate, split_auto ? 1024 : base_wgs);
  if (opts && opts->chains_per_lane) {
    if (!npl_supported(dstate, opts->chains_per_lane))
      return fail(SSM_ERR_UNSUPPORTED, "chains_per_lane %d not available for dstate %lld",
                  (int)opts->chains_per_lane, (long long)dstate);
    npl = opts->chains_per_lane;
  }
  const int G = static_cast<int>(dstate / npl);
  const int64_t max_seg = (seqlen + 4 * ssm::kChunk - 1) / (4 * ssm::kChunk);  // >= 128 steps per segment
  int64_t nseg = 1;
  if (opts && opts->segments > 0) {
    nseg = opts->segments;
  } else if (split_auto) {
    const int64_t target_waves = 4096;
    nseg = (target_waves + base_wgs * G - 1) / (base_wgs * G);
  }
  if (nseg > max_seg) nseg = max_seg;
  if (nseg < 1) nseg = 1;
  int64_t seg_len = seqlen;
  if (nseg > 1) {
    seg_len = (seqlen + nseg - 1) / nseg;
    seg_len = (seg_len + ssm::kChunk - 1) / ssm::kChunk * ssm::kChunk;
    nseg = (seqlen + seg_len - 1) / seg_len;
  }
  int64_t grid;
  if (!mul_ok(base_wgs, nseg, &grid) || grid > 0x7fffffff)
    return fail(SSM_ERR_UNSUPPORTED, "grid of %lld x %lld workgroups is too large", (long long)base_wgs,
                (long long)nseg);

  const bool bf16 = dtype == SSM_BF16;
  const bool zoh = opts && opts->bbar_mode == SSM_BBAR_ZOH;
  const ssm::ScanTable& table = zoh ? (bf16 ? ssm::scan_table_zoh_bf16() : ssm::scan_table_zoh_f32())
                                    : (bf16 ? ssm::scan_table_bf16() : ssm::scan_table_f32());
  const auto it = table.find({static_cast<int>(dstate), npl});
  if (it == table.end()) return fail(SSM_ERR_UNSUPPORTED, "no kernel for dstate %lld chains %d", (long long)dstate, npl);
  // Chunk length: 32-step tiles halve the barriers per step but take twice the LDS, which with
  // 4 scan waves leaves room for one workgroup per CU; measured on MI355X they win while the
  // grid fits in one workgroup per CU, and 16-step tiles (several workgroups per CU) win beyond.
  const int chunk_opt = opts ? opts->chunk_steps : 0;
  if (chunk_opt != 0 && chunk_opt != 16 && chunk_opt != 32)
    return fail(SSM_ERR_UNSUPPORTED, "chunk_steps %d is not 16 or 32", chunk_opt);
  ssm::ScanKernel k_full, k_agg;
  if (chunk_opt == 32) {
    k_full = it->second.full[1];
    k_agg = it->second.agg[1];
    if (!k_full || !k_agg)
      return fail(SSM_ERR_UNSUPPORTED, "chunk_steps 32 not available for dstate %lld chains %d%s", (long long)dstate,
                  npl, zoh ? " with SSM_BBAR_ZOH" : "");
  } else if (chunk_opt == 16) {
    k_full = it->second.full[0];
    k_agg = it->second.agg[0];
  } else {
    const bool one_round = grid <= device_cus();
    k_full = (one_round && it->second.full[1]) ? it->second.full[1] : it->second.full[0];
    k_agg = it->second.agg[0];
  }
  if (!k_full || !k_agg) return fail(SSM_ERR_UNSUPPORTED, "no kernel for this chunk length and bbar_mode");

  ssm::ScanArgs a{};
  a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.Dskip = D; a.z = z; a.delta_bias = delta_bias;
  a.y = y; a.last_state = last_state;
  a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.seg_len = seg_len;
  a.nseg = static_cast<int32_t>(nseg);
  a.ncb = static_cast<int32_t>(ncb);
  a.softplus = delta_softplus ? 1 : 0;
  const int64_t vmax = 16 / es;
  a.vec_ok = (dim % vmax == 0) && aligned(x, 16) && aligned(delta, 16) && aligned(y, 16) && (!z || aligned(z, 16));

  const unsigned threads = static_cast<unsigned>(64 * (G + ssm::kIoWaves));
  if (nseg > 1) {
    float* scratch = nullptr;
    const int64_t floats = nseg * nch * (dstate + 1);
    ssm_status_t s;
    if (src.fixed) {
      if (floats > src.fixed_floats)
        return fail(SSM_ERR_UNSUPPORTED,
                    "the split scan needs %lld fp32 of scratch (%lld segments x %lld channels x (dstate + 1)); "
                    "the allocation-free entry point has %lld",
                    (long long)floats, (long long)nseg, (long long)nch, (long long)src.fixed_floats);
      scratch = src.fixed;
    } else if ((s = get_scratch(st, floats, &scratch)) != SSM_OK) {
      return s;
    }
    a.seg_state = scratch;
    a.seg_dsum = scratch + nseg * nch * dstate;
    hipLaunchKernelGGL(k_agg, dim3(static_cast<unsigned>(base_wgs * (nseg - 1))), dim3(threads), 0, st, a);
    if ((s = check_launch("scan aggregate")) != SSM_OK) return s;
    const int64_t per_seg = nch * dstate;
    hipLaunchKernelGGL(carry_kernel(dstate), dim3(static_cast<unsigned>((per_seg + 255) / 256)), dim3(256), 0, st, a);
    if ((s = check_launch("scan carry")) != SSM_OK) return s;
  }
  hipLaunchKernelGGL(k_full, dim3(static_cast<unsigned>(grid)), dim3(threads), 0, st, a);
  return check_launch("scan");
}

}  // namespace

// ---- the allocation-free scan: scratch in a file-scope device array ------------------------------
// Each GPU the library runs on holds its own copy for the life of the process.  Host code must not
// use the array's name as an address (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kNoAllocScratchFloats = int64_t{1} << 22;  // 16 MiB
static __device__ __align__(256) float scratch[kNoAllocScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
float* g_noalloc_ptr[kMaxDevices] = {};

ssm_status_t noalloc_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SSM_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SSM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_noalloc_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_noalloc_ptr[dev];
  return SSM_OK;
}

}  // namespace

extern "C" {

ssm_status_t ssm_scan_fwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                             const void* x, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int delta_softplus,
                             void* y, float* last_state, void* stream, const ssm_scan_opts_t* opts) {
  g_err[0] = '\0';
  return scan_fwd_impl(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, delta_bias, delta_softplus, y,
                       last_state, stream, opts, ScratchSource{nullptr, 0});
}

ssm_status_t ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                                  const void* x, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* delta_bias, int delta_softplus,
                                  void* y, float* last_state, void* stream, const ssm_scan_opts_t* opts) {
  g_err[0] = '\0';
  float* ptr = nullptr;
  const ssm_status_t s = noalloc_scratch(&ptr);
  if (s != SSM_OK) return s;
  return scan_fwd_impl(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, delta_bias, delta_softplus, y,
                       last_state, stream, opts, ScratchSource{ptr, kNoAllocScratchFloats});
}

ssm_status_t ssm_scan_fwd_ckpt(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                               const void* x, const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias, int delta_softplus, void* y,
                               float* last_state, float* checkpoints, void* stream) {
  g_err[0] = '\0';
  if (!checkpoints && batch > 0 && seqlen > 0 && dim > 0 && dstate > 0)
    return fail(SSM_ERR_INVALID_ARG, "NULL checkpoints");
  return scan_fwd_impl(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, delta_bias, delta_softplus, y,
                       last_state, stream, nullptr, ScratchSource{nullptr, 0}, checkpoints);
}

ssm_status_t ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                          const void* x, const void* delta, const float* A, const void* B, const void* C,
                          const float* D, const void* z, const float* delta_bias, int delta_softplus, void* y,
                          float* last_state, void* stream) {
  return ssm_scan_fwd_ex(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, delta_bias, delta_softplus,
                         y, last_state, stream, nullptr);
}

ssm_status_t ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, ssm_dtype_t dtype, float* state,
                              const void* x, const void* delta, const float* A, const void* B, const void* C,
                              const float* D, const void* z, const float* delta_bias, int delta_softplus, void* y,
                              void* stream) {
  return ssm_state_update_ex(batch, dim, dstate, dtype, state, x, delta, A, B, C, D, z, delta_bias, delta_softplus,
                             y, stream, nullptr);
}

ssm_status_t ssm_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, ssm_dtype_t dtype, float* state,
                                 const void* x, const void* delta, const float* A, const void* B, const void* C,
                                 const float* D, const void* z, const float* delta_bias, int delta_softplus, void* y,
                                 void* stream, const ssm_update_opts_t* opts) {
  g_err[0] = '\0';
  if (opts) {
    if (opts->bbar_mode != SSM_BBAR_DELTA_B && opts->bbar_mode != SSM_BBAR_ZOH)
      return fail(SSM_ERR_UNSUPPORTED, "bbar_mode %d is not SSM_BBAR_DELTA_B or SSM_BBAR_ZOH", (int)opts->bbar_mode);
    for (int32_t r : opts->reserved)
      if (r != 0) return fail(SSM_ERR_INVALID_ARG, "ssm_update_opts_t.reserved must be zero");
  }
  const bool zoh = opts && opts->bbar_mode == SSM_BBAR_ZOH;
  if (batch < 0 || dim < 0 || dstate < 0)
    return fail(SSM_ERR_INVALID_ARG, "negative size (batch=%lld dim=%lld dstate=%lld)", (long long)batch,
                (long long)dim, (long long)dstate);
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (!dstate_supported(dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not in {1,2,4,8,16,32,64}", (long long)dstate);
  const int64_t es = dtype == SSM_BF16 ? 2 : 4;
  int64_t nch, n_bd, n_bn, n_state;
  if (!mul_ok(batch, dim, &nch) || !mul_ok(nch, es, &n_bd) || !mul_ok(batch, dstate * es, &n_bn) ||
      !mul_ok(nch, dstate * 4, &n_state))
    return fail(SSM_ERR_INVALID_ARG, "tensor size overflows int64");
  if (nch == 0) return SSM_OK;
  if (!state || !x || !delta || !A || !B || !C || !y)
    return fail(SSM_ERR_INVALID_ARG, "NULL required pointer (state, x, delta, A, B, C and y are required)");
  const Arg args[] = {{state, 4, "state"}, {x, es, "x"}, {delta, es, "delta"}, {A, 4, "A"}, {B, es, "B"},
                      {C, es, "C"}, {D, 4, "D"}, {z, es, "z"}, {delta_bias, 4, "delta_bias"}, {y, es, "y"}};
  if (const Arg* bad = misaligned(args, sizeof args / sizeof args[0]))
    return fail(SSM_ERR_MISALIGNED, "%s (%p) is not aligned to its element size", bad->name, bad->p);
  const Range rs{state, n_state}, rx{x, n_bd}, rd{delta, n_bd}, rz{z, n_bd}, rB{B, n_bn}, rC{C, n_bn},
      rA{A, dim * dstate * 4}, rD{D, dim * 4}, rb{delta_bias, dim * 4}, ry{y, n_bd};
  for (Range in : {rx, rd, rz, rB, rC, rA, rD, rb})
    if (overlap(ry, in) || overlap(rs, in)) return fail(SSM_ERR_INVALID_ARG, "an output overlaps an input");
  if (overlap(ry, rs)) return fail(SSM_ERR_INVALID_ARG, "y overlaps state");

  const int64_t spt = dstate < 4 ? dstate : 4;
  const int64_t quads = nch * (dstate / spt);
  const int64_t per_block = static_cast<int64_t>(ssm::kUpdateThreads) * ssm::kQuadsPerThread;
  const int64_t blocks = (quads + per_block - 1) / per_block;
  if (blocks > 0x7fffffff) return fail(SSM_ERR_UNSUPPORTED, "grid too large");
  ssm::UpdateArgs a{};
  a.state = state; a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.Dskip = D; a.z = z;
  a.delta_bias = delta_bias; a.y = y; a.batch = batch; a.dim = dim;
  a.softplus = delta_softplus ? 1 : 0;
  a.state_vec_ok = aligned(state, 16) ? 1 : 0;
  a.a_vec_ok = aligned(A, 16) ? 1 : 0;
  const UpdateKernel k = dtype == SSM_BF16 ? (zoh ? update_kernel<true, true>(dstate) : update_kernel<true, false>(dstate))
                                            : (zoh ? update_kernel<false, true>(dstate) : update_kernel<false, false>(dstate));
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(blocks)), dim3(ssm::kUpdateThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return check_launch("state update");
}

ssm_status_t ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                          const void* x, const void* delta, const float* A, const void* B, const void* C,
                          const float* D, const void* z, const float* delta_bias, int delta_softplus,
                          const void* dy, void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                          void* dz, float* ddelta_bias, void* stream) {
  return ssm_scan_bwd_ex(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, delta_bias, delta_softplus, dy,
                         dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, stream, nullptr);
}

}  // extern "C"

namespace {

// The backward; ckpt (batch, ceil(seqlen / 32), dim, 16) fp32, when given, holds the forward's
// chunk-start states and replaces the state-row kernel's phase 0.
ssm_status_t scan_bwd_impl(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                           const void* x, const void* delta, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* delta_bias, int delta_softplus,
                           const void* dy, void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                           void* dz, float* ddelta_bias, void* stream, const ssm_bwd_opts_t* opts,
                           const float* ckpt) {
  if (opts) {
    if (opts->bbar_mode != SSM_BBAR_DELTA_B && opts->bbar_mode != SSM_BBAR_ZOH)
      return fail(SSM_ERR_UNSUPPORTED, "bbar_mode %d is not SSM_BBAR_DELTA_B or SSM_BBAR_ZOH", (int)opts->bbar_mode);
    for (int32_t r : opts->reserved)
      if (r != 0) return fail(SSM_ERR_INVALID_ARG, "ssm_bwd_opts_t.reserved must be zero");
    if (opts->layout < SSM_LAYOUT_AUTO || opts->layout > SSM_LAYOUT_TIME_SCAN)
      return fail(SSM_ERR_INVALID_ARG, "unknown layout %d", (int)opts->layout);
    if (opts->layout == SSM_LAYOUT_TIME_SCAN)
      return fail(SSM_ERR_UNSUPPORTED, "SSM_LAYOUT_TIME_SCAN is a forward layout");
  }
  const bool zoh = opts && opts->bbar_mode == SSM_BBAR_ZOH;
  const int layout = opts ? opts->layout : SSM_LAYOUT_AUTO;
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 0)
    return fail(SSM_ERR_INVALID_ARG, "negative size (batch=%lld seqlen=%lld dim=%lld dstate=%lld)",
                (long long)batch, (long long)seqlen, (long long)dim, (long long)dstate);
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (!dstate_supported(dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not in {1,2,4,8,16,32,64}", (long long)dstate);
  const int64_t es = dtype == SSM_BF16 ? 2 : 4;
  int64_t nch, n_bl, n_bld, n_bln;
  if (!mul_ok(batch, dim, &nch) || !mul_ok(batch, seqlen, &n_bl) || !mul_ok(n_bl, dim * es, &n_bld) ||
      !mul_ok(n_bl, dstate * es, &n_bln) || n_bld > (int64_t{1} << 46))
    return fail(SSM_ERR_INVALID_ARG, "tensor size overflows int64");
  if (dim == 0 || dstate == 0) return SSM_OK;
  if (!dA || (D && !dD) || (delta_bias && !ddelta_bias))
    return fail(SSM_ERR_INVALID_ARG, "NULL gradient for a given parameter (dA; dD when D; ddelta_bias when delta_bias)");
  const bool empty = batch == 0 || seqlen == 0;
  if (!empty && (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dB || !dC || (z && !dz)))
    return fail(SSM_ERR_INVALID_ARG, "NULL required pointer (x, delta, A, B, C, dy, dx, ddelta, dB, dC; dz when z)");
  const Arg args[] = {{x, es, "x"}, {delta, es, "delta"}, {A, 4, "A"}, {B, es, "B"}, {C, es, "C"}, {D, 4, "D"},
                      {z, es, "z"}, {delta_bias, 4, "delta_bias"}, {dy, es, "dy"}, {dx, es, "dx"},
                      {ddelta, es, "ddelta"}, {dA, 4, "dA"}, {dB, es, "dB"}, {dC, es, "dC"}, {dD, 4, "dD"},
                      {dz, es, "dz"}, {ddelta_bias, 4, "ddelta_bias"}};
  if (const Arg* bad = misaligned(args, sizeof args / sizeof args[0]))
    return fail(SSM_ERR_MISALIGNED, "%s (%p) is not aligned to its element size", bad->name, bad->p);
  if (dtype == SSM_BF16 && !empty && !(aligned(B, 4) && aligned(C, 4)))
    return fail(SSM_ERR_MISALIGNED, "bf16 B and C must be 4-byte aligned");
  int64_t n_ck = 0;
  if (ckpt && (!mul_ok(batch, (seqlen + 31) / 32, &n_ck) || !mul_ok(n_ck, dstate * 4, &n_ck) ||
               !mul_ok(n_ck, dim, &n_ck)))
    return fail(SSM_ERR_INVALID_ARG, "tensor size overflows int64");
  if (!aligned(ckpt, 16)) return fail(SSM_ERR_MISALIGNED, "checkpoints (%p) is not 16-byte aligned", ckpt);
  const Range ins[] = {{x, n_bld}, {delta, n_bld}, {z, n_bld}, {dy, n_bld}, {B, n_bln}, {C, n_bln},
                       {A, dim * dstate * 4}, {D, dim * 4}, {delta_bias, dim * 4},
                       {empty ? nullptr : ckpt, n_ck}};
  const Range outs[] = {{dx, n_bld}, {ddelta, n_bld}, {dz, n_bld}, {dB, n_bln}, {dC, n_bln},
                        {dA, dim * dstate * 4}, {dD, dim * 4}, {ddelta_bias, dim * 4}};
  for (const Range& o : outs) {
    for (const Range& i : ins)
      if (overlap(o, i)) return fail(SSM_ERR_INVALID_ARG, "an output overlaps an input");
    for (const Range& o2 : outs)
      if (&o2 != &o && overlap(o, o2)) return fail(SSM_ERR_INVALID_ARG, "two outputs overlap");
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  // state rows: bf16, dstate 16, Delta B, 16-byte rows of every per-step tensor
  const bool rows_fit = !empty && dtype == SSM_BF16 && dstate == 16 && !zoh && dim % 8 == 0 && aligned(x, 16) &&
                        aligned(delta, 16) && aligned(dy, 16) && aligned(dx, 16) && aligned(ddelta, 16) &&
                        (!z || (aligned(z, 16) && aligned(dz, 16))) && aligned(B, 16) && aligned(C, 16);
  if (layout == SSM_LAYOUT_STATE_ROWS && !rows_fit)
    return fail(SSM_ERR_UNSUPPORTED,
                "SSM_LAYOUT_STATE_ROWS backward needs bf16, dstate 16, SSM_BBAR_DELTA_B, dim a multiple of 8 and "
                "16-byte aligned x, delta, z, dy, dx, ddelta, dz, B, C");
  if (ckpt && !empty && (!rows_fit || layout == SSM_LAYOUT_CHANNEL_LANES))
    return fail(SSM_ERR_UNSUPPORTED,
                "a backward from checkpoints needs the state-row layout: bf16, dstate 16, SSM_BBAR_DELTA_B, dim a "
                "multiple of 8 and 16-byte aligned x, delta, z, dy, dx, ddelta, dz, B, C");
  if (rows_fit && layout != SSM_LAYOUT_CHANNEL_LANES) {
    // scan waves per workgroup: the fewest rounds of one workgroup per CU, then the larger
    // workgroup (a workgroup's time does not depend on its scan waves, one per SIMD)
    const int cus = device_cus();
    int S = 1;
    int64_t best = -1;
    for (int c = 1; c <= ssm::kBwdRowsMaxS; ++c) {
      const int64_t rounds = (batch * ((dim + 16 * c - 1) / (16 * c)) + cus - 1) / cus;
      if (best < 0 || rounds <= best) {
        best = rounds;
        S = c;
      }
    }
    constexpr int64_t T = ssm::kBwdRowsT;
    const int64_t nc = (seqlen + T - 1) / T;
    const int64_t ncb = (dim + 16 * S - 1) / (16 * S);
    int64_t grid;
    if (!mul_ok(batch, ncb, &grid) || grid > 0x7fffffff) return fail(SSM_ERR_UNSUPPORTED, "grid too large");
    // scratch: chunk-start states, the dB / dC accumulator, dA / dD / dbias batch partials
    const int64_t n_h = ckpt ? 0 : batch * nc * 16 * dim;
    const int64_t n_bc = 2 * batch * seqlen * 16;
    const int64_t n_a = batch * 16 * dim;
    const int64_t n_d = batch * T * dim;
    float* scratch = nullptr;
    ssm_status_t s = get_scratch(st, n_h + n_bc + n_a + 2 * n_d + 1, &scratch);
    if (s != SSM_OK) return s;
    ssm::BwdArgs a{};
    a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.Dskip = D; a.z = z; a.delta_bias = delta_bias; a.dy = dy;
    a.dx = dx; a.ddelta = ddelta; a.dz = dz;
    a.hstart = ckpt ? const_cast<float*>(ckpt) : scratch;  // read only when given
    a.have_hstart = ckpt ? 1 : 0;
    a.part_bc = scratch + n_h;
    a.part_a = a.part_bc + n_bc;
    a.part_d = a.part_a + n_a;
    a.part_bias = a.part_d + n_d;
    a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.nc = nc;
    a.ncb = static_cast<int32_t>(ncb);
    a.softplus = delta_softplus ? 1 : 0;
    a.vec_ok = 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((n_bc + 255) / 256)), dim3(256), 0, st,
                       a.part_bc, n_bc);
    if ((s = check_launch("fill_zero_kernel")) != SSM_OK) return s;
    hipLaunchKernelGGL(ssm::bwd_rows_kernel(S), dim3(static_cast<unsigned>(grid)), dim3(64 * ssm::kBwdRowsWaves), 0,
                       st, a);
    if ((s = check_launch("scan backward (state rows)")) != SSM_OK) return s;
    ssm::BwdReduceArgs r{};
    r.part_bc = a.part_bc; r.part_a = a.part_a; r.part_d = a.part_d; r.part_bias = a.part_bias;
    r.dB = dB; r.dC = dC; r.dA = dA; r.dD = dD; r.dbias = ddelta_bias;
    r.batch = batch; r.seqlen = seqlen; r.dim = dim; r.N = 16;
    r.ncb = 1;  // the accumulator already holds the channel sums
    r.T = static_cast<int32_t>(T);
    const int64_t nred = 2 * batch * seqlen * 16 + dim * 16 + dim;
    hipLaunchKernelGGL(ssm::scan_bwd_reduce_kernel<true>, dim3(static_cast<unsigned>((nred + 255) / 256)), dim3(256),
                       0, st, r);
    return check_launch("scan backward reduce");
  }
  const int npl = bwd_npl(dstate);
  const int64_t T = ssm::bwd_chunk(npl, zoh);
  const int64_t nc = empty ? 0 : (seqlen + T - 1) / T;
  const int64_t ncb = (dim + 63) / 64;
  // scratch: chunk-start states, dB/dC channel-block partials, dA / dD / dbias batch partials
  const int64_t n_h = batch * nc * dstate * dim;
  const int64_t n_bc = 2 * ncb * batch * seqlen * dstate;
  const int64_t n_a = batch * dstate * dim;
  const int64_t n_d = batch * T * dim;
  float* scratch = nullptr;
  ssm_status_t s = get_scratch(st, n_h + n_bc + n_a + 2 * n_d + 1, &scratch);
  if (s != SSM_OK) return s;
  ssm::BwdArgs a{};
  a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.Dskip = D; a.z = z; a.delta_bias = delta_bias; a.dy = dy;
  a.dx = dx; a.ddelta = ddelta; a.dz = dz;
  a.hstart = scratch;
  a.part_bc = scratch + n_h;
  a.part_a = a.part_bc + n_bc;
  a.part_d = a.part_a + n_a;
  a.part_bias = a.part_d + n_d;
  a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.nc = nc;
  a.ncb = static_cast<int32_t>(ncb);
  a.softplus = delta_softplus ? 1 : 0;
  const int64_t vbytes = 4 * es;  // the IO waves move 4 channels per access
  a.vec_ok = (dim % 4 == 0) && aligned(x, vbytes) && aligned(delta, vbytes) && aligned(dy, vbytes) &&
             aligned(dx, vbytes) && aligned(ddelta, vbytes) && (!z || (aligned(z, vbytes) && aligned(dz, vbytes)));
  const unsigned threads = static_cast<unsigned>(64 * (dstate / npl + ssm::kBwdIoWaves));
  if (!empty) {
    if (batch * ncb > 0x7fffffff) return fail(SSM_ERR_UNSUPPORTED, "grid too large");
    const BwdKernel k = dtype == SSM_BF16 ? (zoh ? bwd_kernel<true, true>(dstate) : bwd_kernel<true, false>(dstate))
                                          : (zoh ? bwd_kernel<false, true>(dstate) : bwd_kernel<false, false>(dstate));
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(batch * ncb)), dim3(threads), 0, st, a);
    if ((s = check_launch("scan backward")) != SSM_OK) return s;
  } else if (n_a + 2 * n_d > 0) {
    // nothing flows back: the parameter gradients are zero
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((n_a + 2 * n_d + 255) / 256)), dim3(256), 0,
                       st, a.part_a, n_a + 2 * n_d);
    if ((s = check_launch("fill_zero_kernel")) != SSM_OK) return s;
  }
  ssm::BwdReduceArgs r{};
  r.part_bc = a.part_bc; r.part_a = a.part_a; r.part_d = a.part_d; r.part_bias = a.part_bias;
  r.dB = dB; r.dC = dC; r.dA = dA; r.dD = dD; r.dbias = ddelta_bias;
  r.batch = batch; r.seqlen = seqlen; r.dim = dim; r.N = static_cast<int32_t>(dstate);
  r.ncb = static_cast<int32_t>(ncb);
  r.T = static_cast<int32_t>(T);
  const int64_t nred = 2 * batch * seqlen * dstate + dim * dstate + dim;
  const BwdReduceKernel rk =
      dtype == SSM_BF16 ? ssm::scan_bwd_reduce_kernel<true> : ssm::scan_bwd_reduce_kernel<false>;
  hipLaunchKernelGGL(rk, dim3(static_cast<unsigned>((nred + 255) / 256)), dim3(256), 0, st, r);
  return check_launch("scan backward reduce");
}

}  // namespace

extern "C" {

ssm_status_t ssm_scan_bwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                             const void* x, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int delta_softplus,
                             const void* dy, void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                             void* dz, float* ddelta_bias, void* stream, const ssm_bwd_opts_t* opts) {
  g_err[0] = '\0';
  return scan_bwd_impl(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, delta_bias, delta_softplus, dy,
                       dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, stream, opts, nullptr);
}

ssm_status_t ssm_scan_bwd_ckpt(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, ssm_dtype_t dtype,
                               const void* x, const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias, int delta_softplus,
                               const void* dy, void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                               void* dz, float* ddelta_bias, const float* checkpoints, void* stream) {
  g_err[0] = '\0';
  if (!checkpoints && batch > 0 && seqlen > 0 && dim > 0 && dstate > 0)
    return fail(SSM_ERR_INVALID_ARG, "NULL checkpoints");
  return scan_bwd_impl(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, delta_bias, delta_softplus, dy,
                       dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, stream, nullptr, checkpoints);
}

ssm_status_t ssm_causal_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, ssm_dtype_t dtype,
                                   const void* x, const float* weight, const float* bias, const void* initial_state,
                                   int silu, void* y, void* final_state, void* stream) {
  g_err[0] = '\0';
  if (batch < 0 || seqlen < 0 || dim < 0 || width < 0)
    return fail(SSM_ERR_INVALID_ARG, "negative size (batch=%lld seqlen=%lld dim=%lld width=%lld)", (long long)batch,
                (long long)seqlen, (long long)dim, (long long)width);
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (width < 1 || width > 4) return fail(SSM_ERR_UNSUPPORTED, "width %lld not in 1..4", (long long)width);
  const int64_t es = dtype == SSM_BF16 ? 2 : 4;
  int64_t nch, n_bl, n_bld, n_st, n_w;
  if (!mul_ok(batch, dim, &nch) || !mul_ok(batch, seqlen, &n_bl) || !mul_ok(n_bl, dim * es, &n_bld) ||
      !mul_ok(nch, (width - 1) * es, &n_st) || !mul_ok(dim, width * 4, &n_w))
    return fail(SSM_ERR_INVALID_ARG, "tensor size overflows int64");
  if (nch == 0) return SSM_OK;
  if (seqlen == 0 && !final_state) return SSM_OK;
  if (!weight || (seqlen > 0 && (!x || !y)))
    return fail(SSM_ERR_INVALID_ARG, "NULL required pointer (weight, and x and y when seqlen > 0)");
  const Arg args[] = {{x, es, "x"}, {weight, 4, "weight"}, {bias, 4, "bias"}, {initial_state, es, "initial_state"},
                      {y, es, "y"}, {final_state, es, "final_state"}};
  if (const Arg* bad = misaligned(args, sizeof args / sizeof args[0]))
    return fail(SSM_ERR_MISALIGNED, "%s (%p) is not aligned to its element size", bad->name, bad->p);
  const Range rx{x, n_bld}, rw{weight, n_w}, rb{bias, dim * 4}, ri{initial_state, n_st},
      ry{seqlen > 0 ? y : nullptr, n_bld}, rf{final_state, n_st};
  for (Range in : {rx, rw, rb, ri})
    if (overlap(ry, in) || overlap(rf, in)) return fail(SSM_ERR_INVALID_ARG, "an output overlaps an input");
  if (overlap(ry, rf)) return fail(SSM_ERR_INVALID_ARG, "y overlaps final_state");

  const int64_t vec = dtype == SSM_BF16 ? ssm::kConvVec<true> : ssm::kConvVec<false>;
  ssm::ConvArgs a{};
  a.x = x; a.weight = weight; a.bias = bias; a.init = initial_state; a.y = y; a.final_state = final_state;
  a.batch = batch; a.seqlen = seqlen; a.dim = dim;
  a.ncv = (dim + vec - 1) / vec;
  a.ntiles = seqlen > 0 ? (seqlen + ssm::kConvTile - 1) / ssm::kConvTile : 1;
  a.silu = silu ? 1 : 0;
  a.vec_ok = (dim % vec == 0) && aligned(x, ssm::kConvVecBytes) && aligned(y, ssm::kConvVecBytes);
  int64_t threads;
  if (!mul_ok(a.ncv * a.ntiles, batch, &threads)) return fail(SSM_ERR_INVALID_ARG, "tensor size overflows int64");
  const int64_t blocks = (threads + ssm::kConvThreads - 1) / ssm::kConvThreads;
  if (blocks > 0x7fffffff) return fail(SSM_ERR_UNSUPPORTED, "grid too large");
  const ConvKernel k = dtype == SSM_BF16 ? conv_kernel<true>(width) : conv_kernel<false>(width);
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(blocks)), dim3(ssm::kConvThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return check_launch("causal conv1d");
}

ssm_status_t ssm_causal_conv1d_update(int64_t batch, int64_t dim, int64_t width, ssm_dtype_t dtype, void* conv_state,
                                      const void* x, const float* weight, const float* bias, int silu, void* y,
                                      void* stream) {
  g_err[0] = '\0';
  if (batch < 0 || dim < 0 || width < 0)
    return fail(SSM_ERR_INVALID_ARG, "negative size (batch=%lld dim=%lld width=%lld)", (long long)batch,
                (long long)dim, (long long)width);
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (width < 1 || width > 4) return fail(SSM_ERR_UNSUPPORTED, "width %lld not in 1..4", (long long)width);
  const int64_t es = dtype == SSM_BF16 ? 2 : 4;
  int64_t nch, n_bd, n_st, n_w;
  if (!mul_ok(batch, dim, &nch) || !mul_ok(nch, es, &n_bd) || !mul_ok(nch, (width - 1) * es, &n_st) ||
      !mul_ok(dim, width * 4, &n_w))
    return fail(SSM_ERR_INVALID_ARG, "tensor size overflows int64");
  if (nch == 0) return SSM_OK;
  if (!x || !weight || !y || (width > 1 && !conv_state))
    return fail(SSM_ERR_INVALID_ARG, "NULL required pointer (x, weight, y, and conv_state when width > 1)");
  const Arg args[] = {{conv_state, es, "conv_state"}, {x, es, "x"}, {weight, 4, "weight"}, {bias, 4, "bias"},
                      {y, es, "y"}};
  if (const Arg* bad = misaligned(args, sizeof args / sizeof args[0]))
    return fail(SSM_ERR_MISALIGNED, "%s (%p) is not aligned to its element size", bad->name, bad->p);
  const Range rs{width > 1 ? conv_state : nullptr, n_st}, rx{x, n_bd}, rw{weight, n_w}, rb{bias, dim * 4},
      ry{y, n_bd};
  for (Range in : {rx, rw, rb})
    if (overlap(ry, in) || overlap(rs, in)) return fail(SSM_ERR_INVALID_ARG, "an output overlaps an input");
  if (overlap(ry, rs)) return fail(SSM_ERR_INVALID_ARG, "y overlaps conv_state");

  ssm::ConvUpdateArgs a{};
  a.state = conv_state; a.x = x; a.weight = weight; a.bias = bias; a.y = y;
  a.batch = batch; a.dim = dim; a.silu = silu ? 1 : 0;
  const int64_t blocks = (nch + ssm::kConvThreads - 1) / ssm::kConvThreads;
  if (blocks > 0x7fffffff) return fail(SSM_ERR_UNSUPPORTED, "grid too large");
  const ConvUpdateKernel k = dtype == SSM_BF16 ? conv_update_kernel<true>(width) : conv_update_kernel<false>(width);
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(blocks)), dim3(ssm::kConvThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return check_launch("causal conv1d update");
}


ssm_status_t ssm_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                         int64_t ngroups, ssm_dtype_t dtype, const void* x, const void* dt, const float* A,
                         const void* B, const void* C, const float* D, const void* z, const float* dt_bias,
                         int dt_softplus, const float* initial_state, void* y, float* final_state, void* stream,
                         const ssm_ssd_opts_t* opts) {
  g_err[0] = '\0';
  if (batch < 0 || seqlen < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1)
    return fail(SSM_ERR_INVALID_ARG, "bad size (batch=%lld seqlen=%lld nheads=%lld headdim=%lld dstate=%lld "
                "ngroups=%lld)", (long long)batch, (long long)seqlen, (long long)nheads, (long long)headdim,
                (long long)dstate, (long long)ngroups);
  if (nheads % ngroups != 0)
    return fail(SSM_ERR_INVALID_ARG, "ngroups %lld does not divide nheads %lld", (long long)ngroups,
                (long long)nheads);
  if (nheads > 0x7fffffff || headdim > 0x7fffffff)
    return fail(SSM_ERR_INVALID_ARG, "nheads or headdim exceeds int32");
  if (dtype != SSM_BF16 && dtype != SSM_F32) return fail(SSM_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "the SSD kernels take bf16 storage only");
  if (dstate != 32 && dstate != 64 && dstate != 128 && dstate != 256)
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not in {32, 64, 128, 256}", (long long)dstate);
  if (headdim % 16 != 0) return fail(SSM_ERR_UNSUPPORTED, "headdim %lld is not a multiple of 16", (long long)headdim);
  int slice = 0, segments = 0, gram = 0;
  if (opts) {
    for (int r : opts->reserved)
      if (r != 0) return fail(SSM_ERR_INVALID_ARG, "reserved option fields must be zero");
    slice = opts->head_slice;
    segments = opts->segments;
    gram = opts->gram;
    if (gram < -1 || gram > 1) return fail(SSM_ERR_INVALID_ARG, "gram %d not in {-1, 0, 1}", gram);
    if (segments < 0) return fail(SSM_ERR_INVALID_ARG, "segments %d is negative", segments);
    if (slice != 0 && slice != 16 && slice != 32 && slice != 64)
      return fail(SSM_ERR_INVALID_ARG, "head_slice %d not in {0, 16, 32, 64}", slice);
    if (slice != 0 && headdim % slice != 0)
      return fail(SSM_ERR_INVALID_ARG, "head_slice %d does not divide headdim %lld", slice, (long long)headdim);
  }
  int64_t nbh, n_tok, n_x, n_bc, n_dt, n_fs;
  if (!mul_ok(batch, nheads, &nbh) || !mul_ok(batch, seqlen, &n_tok) || !mul_ok(n_tok, nheads * headdim * 2, &n_x) ||
      !mul_ok(n_tok, ngroups * dstate * 2, &n_bc) || !mul_ok(n_tok, nheads * 2, &n_dt) ||
      !mul_ok(nbh, headdim * dstate * 4, &n_fs))
    return fail(SSM_ERR_INVALID_ARG, "tensor size overflows int64");
  if (nbh == 0 || (seqlen == 0 && !final_state)) return SSM_OK;
  if (seqlen == 0 && initial_state) {
    // nothing to run: the final state is the entering state
    const hipError_t e = hipMemcpyAsync(final_state, initial_state, static_cast<size_t>(n_fs),
                                        hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
    return SSM_OK;
  }
  if (!A || (seqlen > 0 && (!x || !dt || !B || !C || !y)))
    return fail(SSM_ERR_INVALID_ARG, "NULL required pointer (A, and x, dt, B, C, y when seqlen > 0)");
  const Arg args[] = {{x, 16, "x"}, {z, 16, "z"}, {y, 16, "y"}, {B, 16, "B"}, {C, 16, "C"}, {dt, 2, "dt"},
                      {A, 4, "A"}, {D, 4, "D"}, {dt_bias, 4, "dt_bias"}, {final_state, 16, "final_state"},
                      {initial_state, 16, "initial_state"}};
  if (const Arg* bad = misaligned(args, sizeof args / sizeof args[0]))
    return fail(SSM_ERR_MISALIGNED, "%s (%p) is not aligned to %lld bytes", bad->name, bad->p, (long long)bad->align);
  const Range ry{seqlen > 0 ? y : nullptr, n_x}, rf{final_state, n_fs};
  const Range ins[] = {{x, n_x}, {z, n_x}, {dt, n_dt}, {B, n_bc}, {C, n_bc}, {A, nheads * 4}, {D, nheads * 4},
                       {dt_bias, nheads * 4}, {initial_state, n_fs}};
  for (Range in : ins)
    if (overlap(ry, in) || overlap(rf, in)) return fail(SSM_ERR_INVALID_ARG, "an output overlaps an input");
  if (overlap(ry, rf)) return fail(SSM_ERR_INVALID_ARG, "y overlaps final_state");

  // waves per workgroup (16 head channels each): the largest instantiated count.  Measured on
  // MI355X (dstate 128, headdim 64): 64 workgroups of 4 waves beat 128 of 2 waves (71 vs 82 us on
  // 1 x 1024 steps x 64 heads), and 512 of 4 beat 1024 of 2 (209 vs 344 us on 8 x 2048): fewer
  // waves per head repeat the chunk's C.B^T over fewer channels and hold more registers each.
  int waves = slice / 16;
  if (waves == 0) {
    for (int w : {4, 2, 1}) {
      if (headdim % (16 * w) == 0 && ssm::ssd_kernel(dstate, w, ssm::kSsdOutputs)) {
        waves = w;
        break;
      }
    }
  }
  const ssm::SsdKernel k0 = ssm::ssd_kernel(dstate, waves, ssm::kSsdOutputs);
  if (!k0)
    return fail(SSM_ERR_UNSUPPORTED,
                "no SSD kernel for dstate %lld with headdim %lld (head_slice %d): dstate 256 takes 64-channel "
                "slices, 128 takes 32 or 64",
                (long long)dstate, (long long)headdim, 16 * waves);
  const int64_t nslices = headdim / (16 * waves);
  int64_t blocks;
  if (!mul_ok(nbh, nslices, &blocks) || blocks > 0x7fffffff) return fail(SSM_ERR_UNSUPPORTED, "grid too large");
  ssm::SsdArgs a{};
  a.x = static_cast<const uint16_t*>(x); a.dt = static_cast<const uint16_t*>(dt); a.A = A;
  a.B = static_cast<const uint16_t*>(B); a.C = static_cast<const uint16_t*>(C); a.D = D;
  a.z = static_cast<const uint16_t*>(z); a.dt_bias = dt_bias; a.y = static_cast<uint16_t*>(y);
  a.final_state = final_state;
  a.init_state = initial_state;
  a.batch = batch; a.seqlen = seqlen;
  a.nheads = static_cast<int32_t>(nheads); a.headdim = static_cast<int32_t>(headdim);
  a.ngroups = static_cast<int32_t>(ngroups); a.nslices = static_cast<int32_t>(nslices);
  a.softplus = dt_softplus ? 1 : 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);

  constexpr int64_t kSsdComposeMax = 8;
  // Sequence split: when the (batch row, head, slice) workgroups cannot fill the chip, cut the
  // 64-step chunks into segments, one workgroup per compute unit.  Measured on MI355X (1 x 1024
  // steps x 64 heads, dstate 128): 60 us unsplit, 50 us with 2 segments, 34 us with 4 or 8, 44 us
  // with 16; 4 moves the least segment state through scratch.
  const int64_t nch = (seqlen + ssm::kSsdChunk - 1) / ssm::kSsdChunk;
  int64_t nseg = segments;
  if (nseg == 0) nseg = blocks < device_cus() ? device_cus() / blocks : 1;
  if (nseg > nch) nseg = nch;
  if (nseg < 1) nseg = 1;
  const int64_t seg_chunks = (nch + nseg - 1) / nseg;
  if (nch > 0) nseg = (nch + seg_chunks - 1) / seg_chunks;  // no empty segment
  a.nseg = static_cast<int32_t>(nseg);
  a.seg_chunks = static_cast<int32_t>(seg_chunks > 0 ? seg_chunks : 1);
  // The Gram matrix C B^T of a chunk is the same for every head of a group and every slice of a
  // head: with 4-wave workgroups (the tiles' layout), at least kSsdGramShare workgroups per (batch
  // row, group) and at least kSsdGramChunks chunks per workgroup, a separate pass computes each
  // chunk's tiles once and the chunk kernels read them (the same bits as computing them in place).
  // Measured on MI355X (64 heads x 64 channels, dstate 128): 8 x 2048 steps 142 us against 153;
  // 1 x 1024 steps in 4 segments of 4 chunks 33.8 us against 32.6 (the pass's ~5 us is not
  // repaid by 4 chunks).
  constexpr int64_t kSsdGramShare = 4, kSsdGramChunks = 8;
  const int64_t share = (nheads / ngroups) * nslices;
  if (gram == 1 && waves != 4)
    return fail(SSM_ERR_UNSUPPORTED, "the separate C B^T pass needs 64-channel slices (head_slice %d)", 16 * waves);
  const bool use_gram = nch > 0 && waves == 4 &&
                        (gram == 1 || (gram == 0 && share >= kSsdGramShare && seg_chunks >= kSsdGramChunks));
  int64_t n_gram = 0, g_gram = 0;
  if (use_gram && (!mul_ok(batch * ngroups, nch, &g_gram) || g_gram > 0x7fffffff || !mul_ok(g_gram, 3072, &n_gram)))
    return fail(SSM_ERR_UNSUPPORTED, "C B^T buffer too large");
  // scratch: the C B^T tiles (n_gram fp32, a multiple of 4), then with a sequence split (nseg-1)
  // segment states of batch*nheads*headdim*dstate fp32 and nseg*batch*nheads sums
  int64_t per_seg = 0, n_state = 0, n_seg = 0, g1 = 0, grid = blocks;
  if (nseg > 1 && (!mul_ok(nbh, headdim * dstate, &per_seg) || !mul_ok(per_seg, nseg - 1, &n_state) ||
                   __builtin_add_overflow(n_state, nseg * nbh, &n_seg) || !mul_ok(blocks, nseg, &grid) ||
                   grid > 0x7fffffff || !mul_ok(blocks, nseg - 1, &g1)))
    return fail(SSM_ERR_UNSUPPORTED, "sequence split too large");
  float* scratch = nullptr;
  if (n_gram + n_seg > 0) {
    ssm_status_t s = get_scratch(st, n_gram + n_seg, &scratch);
    if (s != SSM_OK) return s;
  }
  if (use_gram) {
    const ssm::SsdKernel kg = ssm::ssd_gram_kernel_for(dstate);
    if (!kg) return fail(SSM_ERR_UNSUPPORTED, "no C B^T kernel for dstate %lld", (long long)dstate);
    a.gram = scratch;
    a.gram_out = scratch;
    hipLaunchKernelGGL(kg, dim3(static_cast<unsigned>(g_gram)), dim3(256), 0, st, a);
    ssm_status_t s = check_launch("SSD C B^T tiles");
    if (s != SSM_OK) return s;
  }
  if (nseg > 1) {
    a.seg_state = scratch + n_gram;
    a.seg_dsum = scratch + n_gram + n_state;
    ssm_status_t s;
    hipLaunchKernelGGL(ssm::ssd_kernel(dstate, waves, ssm::kSsdStateOnly), dim3(static_cast<unsigned>(g1)),
                       dim3(64 * waves), 0, st, a);
    if ((s = check_launch("SSD segment states")) != SSM_OK) return s;
    // With few segments every workgroup of the outputs pass composes its own entering state (it
    // reads at most kSsdComposeMax - 1 segment states), which saves the carry kernel and its
    // launch; with many, the carry kernel composes them once.
    if (nseg <= kSsdComposeMax) {
      a.compose = 1;
    } else {
      hipLaunchKernelGGL(ssm::ssd_carry_kernel<0>, dim3(static_cast<unsigned>((per_seg + 255) / 256)), dim3(256), 0,
                         st, a, static_cast<int32_t>(dstate));
      if ((s = check_launch("SSD segment carry")) != SSM_OK) return s;
      a.seg_init = a.seg_state;
    }
  }
  const ssm::SsdKernel k = use_gram ? ssm::ssd_kernel(dstate, waves, ssm::kSsdOutputsGram) : k0;
  if (!k) return fail(SSM_ERR_UNSUPPORTED, "no SSD kernel for dstate %lld with read C B^T tiles", (long long)dstate);
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(64 * waves), 0, st, a);
  return check_launch("SSD chunk kernel");
}

ssm_status_t ssm_ssd_state_update(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                                  ssm_dtype_t dtype, float* state, const void* x, const void* dt, const float* A,
                                  const void* B, const void* C, const float* D, const void* z, const float* dt_bias,
                                  int dt_softplus, void* y, void* stream) {
  g_err[0] = '\0';
  if (batch < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1)
    return fail(SSM_ERR_INVALID_ARG, "bad size (batch=%lld nheads=%lld headdim=%lld dstate=%lld ngroups=%lld)",
                (long long)batch, (long long)nheads, (long long)headdim, (long long)dstate, (long long)ngroups);
  if (nheads % ngroups != 0)
    return fail(SSM_ERR_INVALID_ARG, "ngroups %lld does not divide nheads %lld", (long long)ngroups,
                (long long)nheads);
  if (nheads > 0x7fffffff || headdim > 0x7fffffff)
    return fail(SSM_ERR_INVALID_ARG, "nheads or headdim exceeds int32");
  if (dtype != SSM_BF16 && dtype != SSM_F32) return fail(SSM_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (dtype != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "the SSD kernels take bf16 storage only");
  const ssm::SsdUpdateKernel k = ssm::ssd_update_kernel(dstate);
  if (!k) return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not in {32, 64, 128, 256}", (long long)dstate);
  int64_t nbh, nch, n_st, n_x, n_bc, quads;
  if (!mul_ok(batch, nheads, &nbh) || !mul_ok(nbh, headdim, &nch) || !mul_ok(nch, dstate * 4, &n_st) ||
      !mul_ok(nch, 2, &n_x) || !mul_ok(batch * ngroups, dstate * 2, &n_bc) || !mul_ok(nch, dstate / 4, &quads))
    return fail(SSM_ERR_INVALID_ARG, "tensor size overflows int64");
  if (nch == 0) return SSM_OK;
  if (!state || !x || !dt || !A || !B || !C || !y)
    return fail(SSM_ERR_INVALID_ARG, "NULL required pointer (state, x, dt, A, B, C, y)");
  const Arg args[] = {{state, 16, "state"}, {x, 2, "x"}, {dt, 2, "dt"}, {A, 4, "A"}, {B, 8, "B"}, {C, 8, "C"},
                      {D, 4, "D"}, {z, 2, "z"}, {dt_bias, 4, "dt_bias"}, {y, 2, "y"}};
  if (const Arg* bad = misaligned(args, sizeof args / sizeof args[0]))
    return fail(SSM_ERR_MISALIGNED, "%s (%p) is not aligned to %lld bytes", bad->name, bad->p, (long long)bad->align);
  const Range rs{state, n_st}, ry{y, n_x};
  const Range ins[] = {{x, n_x}, {z, n_x}, {dt, nbh * 2}, {B, n_bc}, {C, n_bc}, {A, nheads * 4}, {D, nheads * 4},
                       {dt_bias, nheads * 4}};
  for (Range in : ins)
    if (overlap(ry, in) || overlap(rs, in)) return fail(SSM_ERR_INVALID_ARG, "an output overlaps an input");
  if (overlap(ry, rs)) return fail(SSM_ERR_INVALID_ARG, "y overlaps state");
  const int64_t blocks = (quads + ssm::kSsdUpdateThreads - 1) / ssm::kSsdUpdateThreads;
  if (blocks > 0x7fffffff) return fail(SSM_ERR_UNSUPPORTED, "grid too large");
  ssm::SsdUpdateArgs a{};
  a.state = state; a.x = static_cast<const uint16_t*>(x); a.dt = static_cast<const uint16_t*>(dt); a.A = A;
  a.B = static_cast<const uint16_t*>(B); a.C = static_cast<const uint16_t*>(C); a.D = D;
  a.z = static_cast<const uint16_t*>(z); a.dt_bias = dt_bias; a.y = static_cast<uint16_t*>(y);
  a.batch = batch; a.nheads = static_cast<int32_t>(nheads); a.headdim = static_cast<int32_t>(headdim);
  a.ngroups = static_cast<int32_t>(ngroups); a.softplus = dt_softplus ? 1 : 0;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(blocks)), dim3(ssm::kSsdUpdateThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return check_launch("SSD state update");
}

}  // extern "C"
