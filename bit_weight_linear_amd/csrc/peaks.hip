// Measurement kernels for the benchmark, not part of the layer: the part's
// achievable streaming-read bandwidth and bf16 matrix-core rate, measured on
// the same box as the layer so its roofline fractions can be read against
// both the published peaks and what this part reaches.  Reached only through
// internal exports that obl.h does not declare.
#include "obl_common.hpp"
#include "obl_internal.hpp"
#include "obl.h"

namespace obl {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Reads n16 16-byte words once (non-temporal, four loads in flight per
// thread), XOR-folds them, and stores only if the fold equals a constant the
// benchmark's buffers never produce: the loads cannot be dropped, nothing is
// written.
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                        uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(p + i);
    const u32x4 v1 = __builtin_nontemporal_load(p + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(p + i + 3 * stride);
    x ^= (v0.x ^ v0.y ^ v0.z ^ v0.w) ^ (v1.x ^ v1.y ^ v1.z ^ v1.w) ^ (v2.x ^ v2.y ^ v2.z ^ v2.w) ^
         (v3.x ^ v3.y ^ v3.z ^ v3.w);
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9E3779B9u) out[blockIdx.x] = x;
}

// Every wave issues `iters` rounds of four independent 32x32x16 bf16 MFMAs
// (fp32 accumulate) on fixed pseudo-random operands (normal bf16 values with
// varied mantissas: the matrix core's power, and so its clock, depends on the
// data), then stores only if a sum equals a constant it never reaches.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int64_t iters, float* __restrict__ out) {
  const uint32_t lane = threadIdx.x;
  u32x4 a, b;
  uint32_t h = (lane + 1u) * 0x9E3779B9u ^ blockIdx.x * 0x85EBCA6Bu;
  auto next = [&]() {
    h ^= h << 13; h ^= h >> 17; h ^= h << 5;
    // two bf16 values in [1, 2) or [-2, -1): sign and mantissa from the hash
    return (0x3F803F80u | (h & 0x007F007Fu)) ^ (h & 0x80008000u);
  };
  a = u32x4{next(), next(), next(), next()};
  b = u32x4{next(), next(), next(), next()};
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (s == 1234.5f) out[blockIdx.x * 256 + lane] = s;
}

}  // namespace
}  // namespace obl

using namespace obl;

extern "C" {

// Streaming read of `bytes` (a multiple of 16, 16-byte aligned device memory)
// with 8 workgroups of 256 threads per CU.  `out` receives nothing in
// practice (see the kernel) but must hold one uint32 per workgroup.
obl_status obl_internal_peak_read(const void* p, int64_t bytes, uint32_t* out, void* stream) {
  if (!p || !out) return OBL_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(p) % 16 != 0) return OBL_ERR_SHAPE;
  DeviceInfo dev;
  if (device_info(&dev) != hipSuccess) return OBL_ERR_HIP;
  hipLaunchKernelGGL(peak_read_kernel, dim3((unsigned)(8 * dev.num_cus)), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(p), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? OBL_OK : OBL_ERR_HIP;
}

// Matrix-core loop: 2 workgroups of 4 waves per CU (two waves per SIMD), each
// wave `iters` rounds of four 32x32x16 bf16 MFMAs.  *flops receives the dense
// flop count of the launch (2 * 32 * 32 * 16 per MFMA).  `out` must hold 256
// floats per workgroup (written in practice never).
obl_status obl_internal_peak_mfma(int64_t iters, float* out, double* flops, void* stream) {
  if (!out || !flops) return OBL_ERR_NULL;
  if (iters < 1) return OBL_ERR_SHAPE;
  DeviceInfo dev;
  if (device_info(&dev) != hipSuccess) return OBL_ERR_HIP;
  const int blocks = 2 * dev.num_cus;
  hipLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  *flops = 2.0 * 32 * 32 * 16 * 4.0 * (double)iters * (blocks * 4.0);
  return hipGetLastError() == hipSuccess ? OBL_OK : OBL_ERR_HIP;
}

}  // extern "C"
