// C ABI of libobl: argument validation, path dispatch and library scratch.
//
// Every check runs before the first HIP call, so a rejected call touches no
// device state (and the error paths can be exercised without a GPU).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <functional>
#include <initializer_list>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "obl.h"
#include "obl_internal.hpp"

namespace obl {
namespace {

constexpr int64_t kMaxBytes = int64_t(1) << 62;

int elem_size(obl_dtype d) {
  switch (d) {
    case OBL_F32: return 4;
    case OBL_F16: return 2;
    case OBL_BF16: return 2;
    case OBL_I8: return 1;
  }
  return 0;
}

bool valid_dtype(int d) { return d >= OBL_F32 && d <= OBL_I8; }

// a*b*c bytes without overflow past 2^62; returns -1 when too large.
int64_t checked_bytes(int64_t a, int64_t b, int64_t c) {
  if (a < 0 || b < 0 || c < 0) return -1;
  __int128 v = (__int128)a * b * c;
  return v >= kMaxBytes ? -1 : (int64_t)v;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}
bool overlap(Range a, Range b) {
  if (a.hi == a.lo || b.hi == b.lo) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, int64_t n) { return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)n) == 0; }

// Every dimension must fit in int32: kernel grids and per-block row counts are
// derived from them in 32 bits.
constexpr int64_t kMaxDim = 0x7fffffff;
bool dims_ok(std::initializer_list<int64_t> dims) {
  for (int64_t d : dims)
    if (d > kMaxDim) return false;
  return true;
}

// Path selection.  The test suite can force a path (to cover every kernel at
// every M it supports) through obl_internal_force_kernels, for its own thread
// only; otherwise the path follows from M.
enum Path { P_AUTO, P_LUT, P_DECODE, P_GEMM };
thread_local ForcedKernels t_forced;
thread_local uint64_t* t_span = nullptr;   // set only inside obl_internal_linear_span

Path forced_path() {
  switch (t_forced.path) {
    case 1: return P_LUT;
    case 2: return P_DECODE;
    case 3: return P_GEMM;
  }
  return P_AUTO;
}

// An older GEMM kernel forced (it cannot write the bf16 copy of T1): DBF
// stage 2 then keeps the fp32 workspace.
bool gemm_forced_any() { return t_forced.gemm == 1 || t_forced.gemm == 2; }

Path choose_path(int64_t M, obl_status* st) {
  Path p = forced_path();
  if (p == P_AUTO) {
    if (M <= kLutMaxM) return P_LUT;
    if (M <= kDecodeMaxM) return P_DECODE;
    return P_GEMM;
  }
  if ((p == P_LUT && M > kLutMaxM) || (p == P_DECODE && M > kDecodeWideMaxM)) *st = OBL_ERR_SHAPE;
  return p;
}

std::mutex g_mu;
std::unordered_map<int, DeviceInfo> g_info;

// The path the call actually runs: 17..32 rows take the decode path's
// whole-K kernel where it takes the call and is the faster choice (fp32
// contraction, one launch); a forced decode call it cannot take is refused.
obl_status resolve_path(const LinearArgs& la, Path path, Path* out) {
  if (path == P_DECODE && la.M > kDecodeMaxM && !decode_wide_ok(la)) return OBL_ERR_SHAPE;
  if (path == P_GEMM && forced_path() == P_AUTO && decode_wide_preferred(la)) path = P_DECODE;
  *out = path;
  return OBL_OK;
}

// Adds the scratch one contraction takes to `need` (the launchers carve the
// same amounts from the reserved context).
obl_status plan_linear(const LinearArgs& la, Path path, const DeviceInfo& dev, ScratchNeed* need) {
  Path p = P_AUTO;
  obl_status st = resolve_path(la, path, &p);
  if (st != OBL_OK) return st;
  if (p == P_DECODE) decode_scratch(la, dev, need);
  else if (p == P_GEMM) gemm_scratch(la, dev, need);
  return OBL_OK;
}

// ---------------------------------------------------------------------------
// Scratch sources.
//
// Pool: per device and per stream, two grow-only buffers (one per slot).
// Keying by stream keeps calls on different streams from sharing memory;
// calls on one stream are ordered by the stream.  A buffer that has to grow
// is replaced, never freed: work already enqueued -- or recorded in a HIP
// graph -- may still use it, so it stays valid until the process ends.
// Growth needs hipMalloc, which stream capture does not allow: a call whose
// stream is capturing and whose pool is too small returns OBL_ERR_CAPTURE
// before anything is enqueued, and the capture stays valid.
struct Pool {
  float* buf[kScratchSlots] = {nullptr, nullptr};
  size_t cap[kScratchSlots] = {0, 0};
};
struct PoolKey {
  int device;
  uintptr_t stream;
  bool operator==(const PoolKey& o) const { return device == o.device && stream == o.stream; }
};
struct PoolKeyHash {
  size_t operator()(const PoolKey& k) const { return std::hash<uintptr_t>()(k.stream) * 31u + (size_t)k.device; }
};
std::unordered_map<PoolKey, Pool, PoolKeyHash> g_pools;
std::vector<float*> g_retired;                        // replaced pool buffers, kept until exit
constexpr size_t kMinPoolFloats = size_t(1) << 20;    // 4 MiB

obl_status pool_scratch(const DeviceInfo& dev, hipStream_t stream, const ScratchNeed& need, ScratchCtx* out) {
  if (need.floats[0] == 0 && need.floats[1] == 0) return OBL_OK;
  std::lock_guard<std::mutex> lk(g_mu);
  Pool& p = g_pools[PoolKey{dev.device, reinterpret_cast<uintptr_t>(stream)}];
  for (int s = 0; s < kScratchSlots; ++s) {
    if (need.floats[s] <= p.cap[s]) continue;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
      (void)hipGetLastError();
      return OBL_ERR_CAPTURE;
    }
    size_t n = std::max(need.floats[s], std::max(2 * p.cap[s], kMinPoolFloats));
    // Relaxed capture mode for this thread while allocating, so that a
    // capture running on another stream is not invalidated by the call.
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    if (hipThreadExchangeStreamCaptureMode(&mode) != hipSuccess) return OBL_ERR_HIP;
    float* q = nullptr;
    const hipError_t e = hipMalloc(&q, n * sizeof(float));
    (void)hipThreadExchangeStreamCaptureMode(&mode);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return OBL_ERR_HIP;
    }
    if (p.buf[s]) g_retired.push_back(p.buf[s]);
    p.buf[s] = q;
    p.cap[s] = n;
  }
  for (int s = 0; s < kScratchSlots; ++s) {
    out->base[s] = p.buf[s];
    out->cap[s] = p.cap[s];
  }
  return OBL_OK;
}

}  // namespace
}  // namespace obl

// Fixed scratch of the allocation-free entry point: a device array of
// kFixedScratchFloats floats (64 MiB) that every GPU the library runs on
// holds from the first such call until the process ends, split evenly into
// the two slots.  In host code `scratch` only names the array; its device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kFixedScratchFloats = size_t(16) << 20;
static __device__ __align__(256) float scratch[kFixedScratchFloats];

namespace obl {
namespace {

std::unordered_map<int, float*> g_fixed;   // device -> address of `scratch` there

obl_status fixed_scratch(const DeviceInfo& dev, const ScratchNeed& need, ScratchCtx* out) {
  const size_t half = kFixedScratchFloats / 2;
  if (need.floats[0] > half || need.floats[1] > half) return OBL_ERR_SCRATCH;
  float* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_fixed.find(dev.device);
    if (it == g_fixed.end()) {
      // The current device is dev.device (device_info read it just now).
      if (hipGetSymbolAddress(reinterpret_cast<void**>(&ptr), HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
        (void)hipGetLastError();
        return OBL_ERR_HIP;
      }
      g_fixed.emplace(dev.device, ptr);
    } else {
      ptr = it->second;
    }
  }
  out->base[0] = ptr;
  out->cap[0] = half;
  out->base[1] = ptr + half;
  out->cap[1] = half;
  return OBL_OK;
}

enum ScratchSource { SRC_POOL, SRC_FIXED };

obl_status acquire_scratch(ScratchSource src, const DeviceInfo& dev, hipStream_t stream, const ScratchNeed& need,
                           ScratchCtx* out) {
  return src == SRC_FIXED ? fixed_scratch(dev, need, out) : pool_scratch(dev, stream, need, out);
}

// Launches one contraction whose scratch (la.sx) is already reserved.
obl_status run_linear(const LinearArgs& la, Path path, const DeviceInfo& dev) {
  obl_status st = resolve_path(la, path, &path);
  if (st != OBL_OK) return st;
  hipError_t e;
  switch (path) {
    case P_LUT: e = launch_gemv_lut(la, dev); break;
    case P_DECODE: e = launch_decode_mfma(la, dev); break;
    default: e = launch_gemm_mfma(la, dev); break;
  }
  if (e != hipSuccess) return OBL_ERR_HIP;
  if (hipGetLastError() != hipSuccess) return OBL_ERR_HIP;
  return OBL_OK;
}

// One contraction end to end: plan its scratch, reserve it from the pool of
// the call's stream, launch.
obl_status plan_and_run(LinearArgs la, Path path) {
  Path p = P_AUTO;
  obl_status st = resolve_path(la, path, &p);   // may refuse the call: before any HIP call
  if (st != OBL_OK) return st;
  DeviceInfo dev;
  if (device_info(&dev) != hipSuccess) return OBL_ERR_HIP;
  ScratchNeed need;
  st = plan_linear(la, path, dev, &need);
  if (st != OBL_OK) return st;
  ScratchCtx sx;
  st = acquire_scratch(SRC_POOL, dev, la.stream, need, &sx);
  if (st != OBL_OK) return st;
  la.sx = &sx;
  return run_linear(la, path, dev);
}

bool linear_dtypes_ok(obl_dtype x, obl_dtype s, obl_dtype y) {
  return (x == OBL_F32 || x == OBL_BF16) && (s == OBL_F32 || s == OBL_F16) &&
         (y == OBL_F32 || y == OBL_BF16);
}

// Checks shared by obl_layernorm and obl_linear_layernorm on the LayerNorm
// operands: eps, the optional affine vectors and Z.  `ins` are the ranges Z
// must not overlap.
obl_status check_layernorm(int64_t M, int64_t N, float eps, const void* gamma, const void* beta,
                           obl_dtype g_dtype, const void* Z, obl_dtype z_dtype, const Range* ins, int n_ins) {
  if (M > 0 && !Z) return OBL_ERR_NULL;
  if (!valid_dtype(z_dtype) || (z_dtype != OBL_F32 && z_dtype != OBL_BF16)) return OBL_ERR_DTYPE;
  if ((gamma || beta) && g_dtype != OBL_F32 && g_dtype != OBL_F16) return OBL_ERR_DTYPE;
  if (!std::isfinite(eps) || eps < 0.f) return OBL_ERR_VALUE;
  const int gs = (gamma || beta) ? elem_size(g_dtype) : 1, zs = elem_size(z_dtype);
  const int64_t gb = checked_bytes(N, 1, gs), zb = checked_bytes(M, N, zs);
  if (gb < 0 || zb < 0 || M > 0x7fffffff) return OBL_ERR_SHAPE;
  if ((gamma && !aligned(gamma, gs)) || (beta && !aligned(beta, gs)) || (M > 0 && !aligned(Z, zs)))
    return OBL_ERR_ALIGN;
  const Range rz = range_of(Z, zb);
  if ((gamma && overlap(rz, range_of(gamma, gb))) || (beta && overlap(rz, range_of(beta, gb))))
    return OBL_ERR_ALIAS;
  for (int i = 0; i < n_ins; ++i)
    if (overlap(rz, ins[i])) return OBL_ERR_ALIAS;
  return OBL_OK;
}

}  // namespace

hipError_t device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_info.find(dev);
  if (it == g_info.end()) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    it = g_info.emplace(dev, DeviceInfo{dev, cus > 0 ? cus : 1}).first;
  }
  *out = it->second;
  return hipSuccess;
}

const ForcedKernels& forced_kernels() { return t_forced; }

}  // namespace obl

namespace obl {
namespace {

// dbf_linear and its allocation-free variant: identical but for where their
// scratch comes from.
obl_status dbf_impl(const void* X, obl_dtype x_dtype, int64_t M, int64_t K, const uint32_t* S2_packed, int64_t Kmid,
                    const uint32_t* S1_packed, int64_t N, const void* b, const void* m, const void* a,
                    obl_dtype scale_dtype, float* workspace, void* Y, obl_dtype y_dtype, void* stream,
                    ScratchSource src) {
  try {
    if (M < 0 || K < 1 || Kmid < 1 || N < 1 || K % 32 != 0 || Kmid % 32 != 0 || !dims_ok({M, K, Kmid, N}))
      return OBL_ERR_SHAPE;
    if (!S2_packed || !S1_packed || !b || !m || !a) return OBL_ERR_NULL;
    if (M > 0 && (!X || !Y || !workspace)) return OBL_ERR_NULL;
    if (!valid_dtype(x_dtype) || !valid_dtype(scale_dtype) || !valid_dtype(y_dtype))
      return OBL_ERR_DTYPE;
    if (!linear_dtypes_ok(x_dtype, scale_dtype, y_dtype)) return OBL_ERR_DTYPE;
    const int xs = elem_size(x_dtype), ss = elem_size(scale_dtype), ys = elem_size(y_dtype);
    int64_t xb = checked_bytes(M, K, xs);
    int64_t s2b = checked_bytes(Kmid, K / 32, 4), s1b = checked_bytes(N, Kmid / 32, 4);
    int64_t bb = checked_bytes(K, 1, ss), mb = checked_bytes(Kmid, 1, ss), ab = checked_bytes(N, 1, ss);
    int64_t wsb = checked_bytes(M, Kmid, 4), yb = checked_bytes(M, N, ys);
    if (xb < 0 || s2b < 0 || s1b < 0 || bb < 0 || mb < 0 || ab < 0 || wsb < 0 || yb < 0)
      return OBL_ERR_SHAPE;
    if ((M > 0 && !aligned(X, xs)) || !aligned(S2_packed, 4) || !aligned(S1_packed, 4) ||
        !aligned(b, ss) || !aligned(m, ss) || !aligned(a, ss) ||
        (M > 0 && (!aligned(workspace, 4) || !aligned(Y, ys))))
      return OBL_ERR_ALIGN;
    const Range ins[6] = {range_of(X, xb), range_of(S2_packed, s2b), range_of(S1_packed, s1b),
                          range_of(b, bb), range_of(m, mb), range_of(a, ab)};
    Range ry = range_of(Y, yb), rw = range_of(workspace, wsb);
    for (const Range& r : ins)
      if (overlap(ry, r) || overlap(rw, r)) return OBL_ERR_ALIAS;
    if (overlap(ry, rw)) return OBL_ERR_ALIAS;
    obl_status st = OBL_OK;
    Path path = choose_path(M, &st);
    if (st != OBL_OK) return st;
    if (M == 0) return OBL_OK;
    hipStream_t hs = (hipStream_t)stream;
    // Stage 1: T1 = ((X ⊙ b) S2^T) ⊙ m, kept in fp32 in the workspace.
    LinearArgs s1{X, x_dtype, M, K, S2_packed, Kmid, b, m, scale_dtype, workspace, OBL_F32, hs};
    // Stage 2: Y = (T1 S1^T) ⊙ a (no input-side scale).
    LinearArgs s2{workspace, OBL_F32, M, Kmid, S1_packed, N, nullptr, a, scale_dtype, Y, y_dtype, hs};
    // Where stage 2 reads a copy of T1 from slot 0 of the scratch (its first
    // t1_floats floats, 256-byte aligned), that copy's form: none, bf16, or
    // the exact bf16 terms.  Decided from shapes and alignment alone, before
    // the scratch exists (an aligned stand-in address for the copy).
    const void* kAlignedStandIn = reinterpret_cast<const void*>(uintptr_t(256));
    size_t t1_floats = 0;
    // Prefill: the GEMM rounds T1 to bf16 for stage 2 anyway (one rounding of
    // the input-side operand), so stage 1 also writes that bf16 copy and
    // stage 2 reads it with the bf16 prefill kernel.
    const bool t1_bf16 = path == P_GEMM && !gemm_forced_any() && x_dtype == OBL_BF16 &&
                         gemm_wide_shape_ok(M, K, Kmid, true, X, S2_packed) &&
                         gemm_wide_shape_ok(M, Kmid, N, false, kAlignedStandIn, S1_packed);
    // Decode (up to 8 rows): stage 1 on the whole-K kernel also writes the
    // exact bf16 terms of T1 (hi + mid + lo), and stage 2 reads those terms on
    // the same kernel: one launch per stage, and the products stay exact.
    const bool t1_terms = !t1_bf16 && path == P_DECODE && decode_terms_ok(s1, s2);
    if (t1_bf16) {
      t1_floats = scratch_round((size_t)((M * Kmid + 1) / 2));
      s1.Y2 = const_cast<void*>(kAlignedStandIn);
      s2.X = kAlignedStandIn;
      s2.x_dtype = OBL_BF16;
    } else if (t1_terms) {
      t1_floats = scratch_round((size_t)((3 * M * Kmid + 1) / 2));
      s1.T3 = const_cast<void*>(kAlignedStandIn);
      s2.X = kAlignedStandIn;
      s2.x_dtype = DT_BF16X3;
    }
    Path p1 = P_AUTO, p2 = P_AUTO;   // refusals before any HIP call
    if ((st = resolve_path(s1, path, &p1)) != OBL_OK || (st = resolve_path(s2, path, &p2)) != OBL_OK) return st;
    DeviceInfo dev;
    if (device_info(&dev) != hipSuccess) return OBL_ERR_HIP;
    // Each stage's own scratch follows the T1 copy in slot 0.
    ScratchNeed stages;
    if ((st = plan_linear(s1, path, dev, &stages)) != OBL_OK) return st;
    if ((st = plan_linear(s2, path, dev, &stages)) != OBL_OK) return st;
    ScratchNeed need = stages;
    need.floats[0] = t1_floats + stages.floats[0];
    ScratchCtx sx;
    if ((st = acquire_scratch(src, dev, hs, need, &sx)) != OBL_OK) return st;
    sx.taken[0] = t1_floats;
    if (t1_bf16) {
      s1.Y2 = sx.base[0];
      s2.X = sx.base[0];
    } else if (t1_terms) {
      s1.T3 = sx.base[0];
      s2.X = sx.base[0];
    }
    s1.sx = s2.sx = &sx;
    st = run_linear(s1, path, dev);
    if (st != OBL_OK) return st;
    return run_linear(s2, path, dev);
  } catch (...) {
    return OBL_ERR_INTERNAL;
  }
}

}  // namespace
}  // namespace obl

using namespace obl;

extern "C" {

const char* obl_status_string(obl_status s) {
  switch (s) {
    case OBL_OK: return "OBL_OK";
    case OBL_ERR_NULL: return "OBL_ERR_NULL: a required pointer is NULL";
    case OBL_ERR_SHAPE: return "OBL_ERR_SHAPE: invalid dimension";
    case OBL_ERR_DTYPE: return "OBL_ERR_DTYPE: unsupported dtype combination";
    case OBL_ERR_ALIGN: return "OBL_ERR_ALIGN: misaligned pointer";
    case OBL_ERR_ALIAS: return "OBL_ERR_ALIAS: output overlaps another argument";
    case OBL_ERR_HIP: return "OBL_ERR_HIP: HIP runtime error";
    case OBL_ERR_INTERNAL: return "OBL_ERR_INTERNAL: internal error";
    case OBL_ERR_VALUE: return "OBL_ERR_VALUE: scalar argument out of range";
    case OBL_ERR_CAPTURE:
      return "OBL_ERR_CAPTURE: the call needs more library scratch than its stream holds and the stream is "
             "capturing; make one call of this size on that stream before capturing";
    case OBL_ERR_SCRATCH: return "OBL_ERR_SCRATCH: the call needs more scratch than the fixed array holds";
  }
  return "OBL_ERR_UNKNOWN";
}

// 0.3.0: per-stream scratch that is never freed, OBL_ERR_CAPTURE, the
// allocation-free dbf_linear_noalloc.
int obl_version(void) { return 300; }

obl_status obl_pack_signs(const void* S, obl_dtype s_dtype, int64_t rows, int64_t K,
                          uint32_t* packed, void* stream) {
  try {
    if (!S || !packed) return OBL_ERR_NULL;
    if (rows < 1 || K < 1 || K % 32 != 0 || !dims_ok({rows, K})) return OBL_ERR_SHAPE;
    if (!valid_dtype(s_dtype)) return OBL_ERR_DTYPE;
    int64_t sb = checked_bytes(rows, K, elem_size(s_dtype));
    int64_t pb = checked_bytes(rows, K / 32, 4);
    if (sb < 0 || pb < 0) return OBL_ERR_SHAPE;
    if (!aligned(S, elem_size(s_dtype)) || !aligned(packed, 4)) return OBL_ERR_ALIGN;
    if (overlap(range_of(S, sb), range_of(packed, pb))) return OBL_ERR_ALIAS;
    hipError_t e = launch_pack_signs(S, s_dtype, rows, K, packed, (hipStream_t)stream);
    if (e != hipSuccess || hipGetLastError() != hipSuccess) return OBL_ERR_HIP;
    return OBL_OK;
  } catch (...) {
    return OBL_ERR_INTERNAL;
  }
}

obl_status obl_linear(const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                      const uint32_t* W_packed, int64_t N,
                      const void* a, const void* b, obl_dtype scale_dtype,
                      void* Y, obl_dtype y_dtype, void* stream) {
  try {
    if (M < 0 || K < 1 || N < 1 || K % 32 != 0 || !dims_ok({M, K, N})) return OBL_ERR_SHAPE;
    if (!W_packed || !a || !b) return OBL_ERR_NULL;
    if (M > 0 && (!X || !Y)) return OBL_ERR_NULL;
    if (!valid_dtype(x_dtype) || !valid_dtype(scale_dtype) || !valid_dtype(y_dtype))
      return OBL_ERR_DTYPE;
    if (!linear_dtypes_ok(x_dtype, scale_dtype, y_dtype)) return OBL_ERR_DTYPE;
    const int xs = elem_size(x_dtype), ss = elem_size(scale_dtype), ys = elem_size(y_dtype);
    int64_t xb = checked_bytes(M, K, xs), wb = checked_bytes(N, K / 32, 4);
    int64_t ab = checked_bytes(N, 1, ss), bb = checked_bytes(K, 1, ss);
    int64_t yb = checked_bytes(M, N, ys);
    if (xb < 0 || wb < 0 || ab < 0 || bb < 0 || yb < 0) return OBL_ERR_SHAPE;
    if ((M > 0 && !aligned(X, xs)) || !aligned(W_packed, 4) || !aligned(a, ss) ||
        !aligned(b, ss) || (M > 0 && !aligned(Y, ys)))
      return OBL_ERR_ALIGN;
    Range ry = range_of(Y, yb);
    if (overlap(ry, range_of(X, xb)) || overlap(ry, range_of(W_packed, wb)) ||
        overlap(ry, range_of(a, ab)) || overlap(ry, range_of(b, bb)))
      return OBL_ERR_ALIAS;
    obl_status st = OBL_OK;
    Path path = choose_path(M, &st);
    if (st != OBL_OK) return st;
    if (M == 0) return OBL_OK;
    LinearArgs la{X, x_dtype, M, K, W_packed, N, b, a, scale_dtype, Y, y_dtype, (hipStream_t)stream};
    la.span = t_span;
    return plan_and_run(la, path);
  } catch (...) {
    return OBL_ERR_INTERNAL;
  }
}

obl_status obl_svid(const void* W, obl_dtype w_dtype, int64_t N, int64_t K, int iters, uint32_t* packed,
                    void* a, void* b, obl_dtype scale_dtype, void* stream) {
  try {
    if (!W || !packed || !a || !b) return OBL_ERR_NULL;
    if (N < 1 || K < 1 || K % 32 != 0 || iters < 1 || iters > 100000 || !dims_ok({N, K})) return OBL_ERR_SHAPE;
    if (w_dtype != OBL_F32 && w_dtype != OBL_F16 && w_dtype != OBL_BF16) return OBL_ERR_DTYPE;
    if (scale_dtype != OBL_F32 && scale_dtype != OBL_F16) return OBL_ERR_DTYPE;
    const int ws = elem_size(w_dtype), ss = elem_size(scale_dtype);
    int64_t wb = checked_bytes(N, K, ws), pb = checked_bytes(N, K / 32, 4);
    int64_t ab = checked_bytes(N, 1, ss), bb = checked_bytes(K, 1, ss);
    if (wb < 0 || pb < 0 || ab < 0 || bb < 0) return OBL_ERR_SHAPE;
    if (!aligned(W, ws) || !aligned(packed, 4) || !aligned(a, ss) || !aligned(b, ss)) return OBL_ERR_ALIGN;
    const Range rw = range_of(W, wb);
    const Range outs[3] = {range_of(packed, pb), range_of(a, ab), range_of(b, bb)};
    for (int o = 0; o < 3; ++o) {
      if (overlap(outs[o], rw)) return OBL_ERR_ALIAS;
      for (int p = o + 1; p < 3; ++p)
        if (overlap(outs[o], outs[p])) return OBL_ERR_ALIAS;
    }
    DeviceInfo dev;
    if (device_info(&dev) != hipSuccess) return OBL_ERR_HIP;
    hipStream_t hs = (hipStream_t)stream;
    ScratchNeed need;
    need.need(0, svid_workspace_floats(N, K));
    ScratchCtx sx;
    obl_status st = acquire_scratch(SRC_POOL, dev, hs, need, &sx);
    if (st != OBL_OK) return st;
    hipError_t e = launch_pack_signs(W, w_dtype, N, K, packed, hs);
    if (e == hipSuccess) e = launch_svid(W, w_dtype, N, K, iters, a, b, scale_dtype, sx.base[0], hs);
    if (e != hipSuccess || hipGetLastError() != hipSuccess) return OBL_ERR_HIP;
    return OBL_OK;
  } catch (...) {
    return OBL_ERR_INTERNAL;
  }
}

obl_status obl_transpose_signs(const uint32_t* packed, int64_t rows, int64_t K, uint32_t* packed_t,
                               void* stream) {
  try {
    if (!packed || !packed_t) return OBL_ERR_NULL;
    if (rows < 1 || K < 1 || K % 32 != 0 || rows % 32 != 0 || !dims_ok({rows, K})) return OBL_ERR_SHAPE;
    int64_t pb = checked_bytes(rows, K / 32, 4), tb = checked_bytes(K, rows / 32, 4);
    if (pb < 0 || tb < 0) return OBL_ERR_SHAPE;
    if (!aligned(packed, 4) || !aligned(packed_t, 4)) return OBL_ERR_ALIGN;
    if (overlap(range_of(packed, pb), range_of(packed_t, tb))) return OBL_ERR_ALIAS;
    hipError_t e = launch_transpose_signs(packed, rows, K, packed_t, (hipStream_t)stream);
    if (e != hipSuccess || hipGetLastError() != hipSuccess) return OBL_ERR_HIP;
    return OBL_OK;
  } catch (...) {
    return OBL_ERR_INTERNAL;
  }
}

obl_status obl_linear_backward(const void* dY, const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                               const uint32_t* W_packed, const uint32_t* Wt_packed, int64_t N,
                               const void* a, const void* b, obl_dtype scale_dtype,
                               void* dX, obl_dtype dx_dtype, float* da, float* db,
                               float* workspace, void* stream) {
  try {
    if (M < 0 || K < 1 || N < 1 || K % 32 != 0 || N % 32 != 0 || !dims_ok({M, K, N})) return OBL_ERR_SHAPE;
    if (!W_packed || !Wt_packed || !a || !b || !da || !db) return OBL_ERR_NULL;
    if (M > 0 && (!dY || !X || !dX || !workspace)) return OBL_ERR_NULL;
    if (!valid_dtype(x_dtype) || !valid_dtype(scale_dtype) || !valid_dtype(dx_dtype))
      return OBL_ERR_DTYPE;
    if (!linear_dtypes_ok(x_dtype, scale_dtype, dx_dtype)) return OBL_ERR_DTYPE;
    const int xs = elem_size(x_dtype), ss = elem_size(scale_dtype), ds = elem_size(dx_dtype);
    int64_t gyb = checked_bytes(M, N, xs), xb = checked_bytes(M, K, xs);
    int64_t wb = checked_bytes(N, K / 32, 4), wtb = checked_bytes(K, N / 32, 4);
    int64_t ab = checked_bytes(N, 1, ss), bb = checked_bytes(K, 1, ss);
    int64_t dxb = checked_bytes(M, K, ds), dab = checked_bytes(N, 1, 4), dbb = checked_bytes(K, 1, 4);
    int64_t wsb = checked_bytes(M, N + K, 4);
    if (gyb < 0 || xb < 0 || wb < 0 || wtb < 0 || ab < 0 || bb < 0 || dxb < 0 || dab < 0 || dbb < 0 ||
        wsb < 0)
      return OBL_ERR_SHAPE;
    if ((M > 0 && (!aligned(dY, xs) || !aligned(X, xs) || !aligned(dX, ds) || !aligned(workspace, 4))) ||
        !aligned(W_packed, 4) || !aligned(Wt_packed, 4) || !aligned(a, ss) || !aligned(b, ss) ||
        !aligned(da, 4) || !aligned(db, 4))
      return OBL_ERR_ALIGN;
    const Range ins[6] = {range_of(dY, gyb), range_of(X, xb), range_of(W_packed, wb),
                          range_of(Wt_packed, wtb), range_of(a, ab), range_of(b, bb)};
    const Range outs[4] = {range_of(dX, dxb), range_of(da, dab), range_of(db, dbb), range_of(workspace, wsb)};
    for (int o = 0; o < 4; ++o) {
      for (const Range& r : ins)
        if (overlap(outs[o], r)) return OBL_ERR_ALIAS;
      for (int p = o + 1; p < 4; ++p)
        if (overlap(outs[o], outs[p])) return OBL_ERR_ALIAS;
    }
    obl_status st = OBL_OK;
    Path path = choose_path(M, &st);
    if (st != OBL_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    if (M == 0) {
      // Empty batch: the reduction kernel writes the zero sums da = db = 0.
      hipError_t e = launch_backward_grads(x_dtype, scale_dtype, dx_dtype, dY, X, nullptr, nullptr, b, 0, K,
                                           N, dX, da, db, hs);
      return (e != hipSuccess || hipGetLastError() != hipSuccess) ? OBL_ERR_HIP : OBL_OK;
    }
    float* T = workspace;                 // [M][N]
    float* U = workspace + M * N;         // [M][K]
    // T = (X ⊙ b^T) W_sign^T and U = (dY ⊙ a^T) W_sign, both without an output scale.
    LinearArgs t{X, x_dtype, M, K, W_packed, N, b, nullptr, scale_dtype, T, OBL_F32, hs};
    LinearArgs u{dY, x_dtype, M, N, Wt_packed, K, a, nullptr, scale_dtype, U, OBL_F32, hs};
    // Both contractions on the decode path's whole-K kernel: its epilogue
    // forms the gradients (da from T and dY; dX and db from U, b and X), so no
    // separate reduction launch.
    const bool auto_wide = path == P_GEMM && forced_path() == P_AUTO && decode_wide_preferred(t) &&
                           decode_wide_preferred(u);
    const bool fused = (path == P_DECODE || auto_wide) && decode_wide_ok(t) && decode_wide_ok(u);
    if (fused) {
      t.gin = dY;
      t.gsum = da;
      u.gin = X;
      u.gsum = db;
      u.gscale = b;
      u.gout = dX;
      u.gout_dtype = dx_dtype;
    }
    Path pt = P_AUTO, pu = P_AUTO;   // refusals before any HIP call
    if ((st = resolve_path(t, path, &pt)) != OBL_OK || (st = resolve_path(u, path, &pu)) != OBL_OK) return st;
    DeviceInfo dev;
    if (device_info(&dev) != hipSuccess) return OBL_ERR_HIP;
    ScratchNeed need;   // the two contractions run one after the other on the stream: one reservation serves both
    if ((st = plan_linear(t, path, dev, &need)) != OBL_OK) return st;
    if ((st = plan_linear(u, path, dev, &need)) != OBL_OK) return st;
    ScratchCtx sx;
    if ((st = acquire_scratch(SRC_POOL, dev, hs, need, &sx)) != OBL_OK) return st;
    t.sx = u.sx = &sx;
    if (fused && t_forced.pair != 1) {
      // Both contractions in one launch where they take one kernel instance.
      const hipError_t e = launch_decode_pair(t, u, dev);
      if (e == hipSuccess) return hipGetLastError() == hipSuccess ? OBL_OK : OBL_ERR_HIP;
      if (e != hipErrorNotSupported) return OBL_ERR_HIP;
    }
    st = run_linear(t, path, dev);
    if (st != OBL_OK) return st;
    st = run_linear(u, path, dev);
    if (st != OBL_OK || fused) return st;
    hipError_t e = launch_backward_grads(x_dtype, scale_dtype, dx_dtype, dY, X, T, U, b, M, K, N, dX, da,
                                         db, hs);
    if (e != hipSuccess || hipGetLastError() != hipSuccess) return OBL_ERR_HIP;
    return OBL_OK;
  } catch (...) {
    return OBL_ERR_INTERNAL;
  }
}

obl_status obl_layernorm(const void* Y, obl_dtype y_dtype, int64_t M, int64_t N, float eps,
                         const void* gamma, const void* beta, obl_dtype affine_dtype,
                         void* Z, obl_dtype z_dtype, void* stream) {
  try {
    if (M < 0 || N < 1 || !dims_ok({M, N})) return OBL_ERR_SHAPE;
    if (M > 0 && !Y) return OBL_ERR_NULL;
    if (!valid_dtype(y_dtype) || (y_dtype != OBL_F32 && y_dtype != OBL_BF16)) return OBL_ERR_DTYPE;
    const int ys = elem_size(y_dtype);
    const int64_t yb = checked_bytes(M, N, ys);
    if (yb < 0) return OBL_ERR_SHAPE;
    const Range ry = range_of(Y, yb);
    obl_status st = check_layernorm(M, N, eps, gamma, beta, affine_dtype, Z, z_dtype, &ry, 1);
    if (st != OBL_OK) return st;
    if (M > 0 && !aligned(Y, ys)) return OBL_ERR_ALIGN;
    if (M == 0) return OBL_OK;
    hipError_t e = launch_layernorm_rows(Y, y_dtype, M, N, eps, gamma, beta, affine_dtype, Z, z_dtype,
                                         (hipStream_t)stream);
    if (e != hipSuccess || hipGetLastError() != hipSuccess) return OBL_ERR_HIP;
    return OBL_OK;
  } catch (...) {
    return OBL_ERR_INTERNAL;
  }
}

obl_status obl_linear_layernorm(const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                                const uint32_t* W_packed, int64_t N,
                                const void* a, const void* b, obl_dtype scale_dtype,
                                float eps, const void* gamma, const void* beta,
                                float* workspace, void* Z, obl_dtype z_dtype, void* stream) {
  try {
    if (M < 0 || K < 1 || N < 1 || K % 32 != 0 || !dims_ok({M, K, N})) return OBL_ERR_SHAPE;
    if (!W_packed || !a || !b) return OBL_ERR_NULL;
    if (M > 0 && (!X || !workspace)) return OBL_ERR_NULL;
    if (!valid_dtype(x_dtype) || !valid_dtype(scale_dtype)) return OBL_ERR_DTYPE;
    if (!linear_dtypes_ok(x_dtype, scale_dtype, OBL_F32)) return OBL_ERR_DTYPE;
    const int xs = elem_size(x_dtype), ss = elem_size(scale_dtype);
    int64_t xb = checked_bytes(M, K, xs), wb = checked_bytes(N, K / 32, 4);
    int64_t ab = checked_bytes(N, 1, ss), bb = checked_bytes(K, 1, ss);
    int64_t yb = checked_bytes(M, N, 4);
    if (xb < 0 || wb < 0 || ab < 0 || bb < 0 || yb < 0) return OBL_ERR_SHAPE;
    if ((M > 0 && (!aligned(X, xs) || !aligned(workspace, 4))) || !aligned(W_packed, 4) || !aligned(a, ss) ||
        !aligned(b, ss))
      return OBL_ERR_ALIGN;
    const int64_t gb = (gamma || beta) ? checked_bytes(N, 1, ss) : 0;
    const Range ins[7] = {range_of(X, xb), range_of(W_packed, wb), range_of(a, ab), range_of(b, bb),
                          range_of(workspace, yb), range_of(gamma, gamma ? gb : 0),
                          range_of(beta, beta ? gb : 0)};
    // The workspace (Y) must not overlap the linear's inputs or gamma / beta.
    for (int i = 0; i < 7; ++i)
      if (i != 4 && overlap(ins[4], ins[i])) return OBL_ERR_ALIAS;
    obl_status st = check_layernorm(M, N, eps, gamma, beta, scale_dtype, Z, z_dtype, ins, 5);
    if (st != OBL_OK) return st;
    Path path = choose_path(M, &st);
    if (st != OBL_OK) return st;
    if (M == 0) return OBL_OK;
    hipStream_t hs = (hipStream_t)stream;
    LinearArgs la{X, x_dtype, M, K, W_packed, N, b, a, scale_dtype, workspace, OBL_F32, hs};
    st = plan_and_run(la, path);
    if (st != OBL_OK) return st;
    hipError_t e = launch_layernorm_rows(workspace, OBL_F32, M, N, eps, gamma, beta, scale_dtype, Z, z_dtype, hs);
    if (e != hipSuccess || hipGetLastError() != hipSuccess) return OBL_ERR_HIP;
    return OBL_OK;
  } catch (...) {
    return OBL_ERR_INTERNAL;
  }
}

obl_status dbf_linear(const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                      const uint32_t* S2_packed, int64_t Kmid,
                      const uint32_t* S1_packed, int64_t N,
                      const void* b, const void* m, const void* a, obl_dtype scale_dtype,
                      float* workspace, void* Y, obl_dtype y_dtype, void* stream) {
  return dbf_impl(X, x_dtype, M, K, S2_packed, Kmid, S1_packed, N, b, m, a, scale_dtype, workspace, Y, y_dtype,
                  stream, SRC_POOL);
}

obl_status dbf_linear_noalloc(const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                              const uint32_t* S2_packed, int64_t Kmid,
                              const uint32_t* S1_packed, int64_t N,
                              const void* b, const void* m, const void* a, obl_dtype scale_dtype,
                              float* workspace, void* Y, obl_dtype y_dtype, void* stream) {
  return dbf_impl(X, x_dtype, M, K, S2_packed, Kmid, S1_packed, N, b, m, a, scale_dtype, workspace, Y, y_dtype,
                  stream, SRC_FIXED);
}

// Internal export for the benchmark, not declared in obl.h: obl_linear whose
// LUT GEMV launch (M <= 2) also writes a span record -- for each workgroup,
// the constant-clock ticks (s_memrealtime) at its first wave's start and at
// its end -- to span[2 * blocks], 16-byte aligned.  Other paths ignore span.
obl_status obl_internal_linear_span(const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                                    const uint32_t* W_packed, int64_t N, const void* a, const void* b,
                                    obl_dtype scale_dtype, void* Y, obl_dtype y_dtype, uint64_t* span,
                                    void* stream) {
  if (!span || reinterpret_cast<uintptr_t>(span) % 16 != 0) return OBL_ERR_ALIGN;
  t_span = span;
  const obl_status st = obl_linear(X, x_dtype, M, K, W_packed, N, a, b, scale_dtype, Y, y_dtype, stream);
  t_span = nullptr;
  return st;
}

// Internal export for the benchmark, not declared in obl.h: the frequency of
// the constant clock s_memrealtime counts (kHz) on the current device, or a
// negative value on error.
int obl_internal_wallclock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return khz;
}

// Internal export for the test suite, not declared in obl.h: forces a path
// and kernel choice (codes in obl_internal.hpp, ForcedKernels) for the
// calling thread's later calls; all zeros restores the automatic choice.
// Nothing else reads or sets it, so ordinary callers always get the kernel
// their arguments select.
void obl_internal_force_kernels(int path, int gemm, int decode, int pair) {
  t_forced.path = path;
  t_forced.gemm = gemm;
  t_forced.decode = decode;
  t_forced.pair = pair;
}

}  // extern "C"
