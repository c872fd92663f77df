// obl_pack_signs: W_sign = Sign(S), bit-packed along K.
//
// OneBit page ("1bit量化"), the sign/value split W = W_sign ⊙ |W|.  A value
// packs as -1 (bit set) exactly when it compares below zero.
//
// One wave packs 64 consecutive words of a row range: lane l owns word l and
// reads its 32 source values with wide loads (32 B for int8, 64 B for 16-bit,
// 128 B for fp32).  The kernel is offline (weight conversion) and
// bandwidth-bound; it is not on the timed inference path.
#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

__device__ __forceinline__ uint32_t neg_bits(int8_t v) { return v < 0; }
__device__ __forceinline__ uint32_t neg_bits(float v) { return v < 0.0f; }
__device__ __forceinline__ uint32_t neg_bits(bf16_t v) { return to_f32(v) < 0.0f; }
__device__ __forceinline__ uint32_t neg_bits(f16_t v) { return to_f32(v) < 0.0f; }

template <typename T>
__global__ __launch_bounds__(256) void pack_signs_kernel(const T* __restrict__ S, int64_t total_words,
                                                         uint32_t* __restrict__ P) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_words; i += stride) {
    // Word i covers source elements [32 i, 32 i + 32): rows are contiguous and
    // K is a multiple of 32, so the flat index needs no row arithmetic.
    const T* src = S + i * 32;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) w |= neg_bits(src[j]) << j;
    P[i] = w;
  }
}

template <typename T>
hipError_t launch_t(const void* S, int64_t words, uint32_t* P, hipStream_t stream) {
  const int threads = 256;
  int64_t blocks = (words + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_signs_kernel<T>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<const T*>(S), words, P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_signs(const void* S, int s_dtype, int64_t rows, int64_t K, uint32_t* P,
                             hipStream_t stream) {
  const int64_t words = rows * (K / 32);
  switch (s_dtype) {
    case DT_I8: return launch_t<int8_t>(S, words, P, stream);
    case DT_F32: return launch_t<float>(S, words, P, stream);
    case DT_F16: return launch_t<f16_t>(S, words, P, stream);
    case DT_BF16: return launch_t<bf16_t>(S, words, P, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace obl
