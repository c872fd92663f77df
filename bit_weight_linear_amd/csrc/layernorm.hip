// Row LayerNorm after the layer: Z = LayerNorm(Y).
//
// OneBit page ("1bit量化"), knowledge-distillation block: the layer output Y
// is normalised per row before it is compared with the teacher.  The page
// names only the operation; epsilon and the optional elementwise gamma/beta
// are the caller's.  For row i:
//   μ_i = (1/N) Σ_j y_ij,  σ²_i = (1/N) Σ_j (y_ij - μ_i)²  (two passes),
//   z_ij = (y_ij - μ_i) / sqrt(σ²_i + eps) · γ_j + β_j.
//
// HBM-bound: one workgroup per row.  Register path (N % 4 == 0, aligned, and
// N <= 4 · BS · NC): the row is read once into registers, NC chunks of one
// 4-element vector per thread, and held there for both passes and the output,
// so the kernel moves exactly N input and N output elements per row.  Every
// load of a chunk is issued unconditionally (an index past the row is clamped
// to its last vector and masked out of the sums): loads under a per-lane
// branch would each wait for their data at the end of the branch, turning
// one memory round trip per row into one per chunk.  Longer or odd rows take
// the window path: windows of 8 chunks, read three times (sum, squared
// deviations, output), the re-reads served by L2.
// Every sum runs in a fixed order (per-thread chunks in order, a DPP butterfly
// inside each 16-lane row, the four rows, then the waves in order): results
// are bitwise reproducible.
#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

constexpr int LN_WIN = 8;  // chunks per window on the window path

// ---------------------------------------------------------------- element I/O
template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ void load(const float* p, float v[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  static __device__ __forceinline__ void store(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct Vec4<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float v[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float v[4]) {
    bf16_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) Store<bf16_t>::put(&h[e], v[e]);
    uint2 q;
    q.x = uint32_t(h[0].bits) | (uint32_t(h[1].bits) << 16);
    q.y = uint32_t(h[2].bits) | (uint32_t(h[3].bits) << 16);
    *reinterpret_cast<uint2*>(p) = q;
  }
};
template <> struct Vec4<f16_t> {
  static __device__ __forceinline__ void load(const f16_t* p, float v[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    const f16_t* h = reinterpret_cast<const f16_t*>(&q);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = to_f32(h[e]);
  }
};

template <int VEC, typename T>
__device__ __forceinline__ void load_v(const T* p, float v[VEC]) {
  if constexpr (VEC == 4) Vec4<T>::load(p, v);
  else v[0] = to_f32(p[0]);
}
template <int VEC, typename T>
__device__ __forceinline__ void store_v(T* p, const float v[VEC]) {
  if constexpr (VEC == 4) Vec4<T>::store(p, v);
  else Store<T>::put(p, v[0]);
}

// ---------------------------------------------------------------- reductions
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes, returned as a wave-uniform value.  Inside each row
// of 16 lanes: xor 1 and xor 2 within quads, then half-mirror (quad pairs)
// and mirror (8-lane halves); then the four row sums in lane order.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

// Workgroup sum (every thread gets it).  `red` is used by this call only, so
// one barrier suffices.
template <int BS>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < BS / 64; ++w) t += red[w];
  return t;
}

// NC chunks starting at chunk c0 of a row of nv vectors: v[c] <- vector
// (c0 + c) · BS + tid, clamped to nv - 1; ok[c] tells whether it is real.
template <int VEC, int NC, int BS, typename T>
__device__ __forceinline__ void load_window(const T* __restrict__ p, int64_t nv, int64_t c0, float v[NC][VEC],
                                            bool ok[NC]) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t i = (c0 + c) * BS + threadIdx.x;
    ok[c] = i < nv;
    load_v<VEC>(p + (ok[c] ? i : nv - 1) * VEC, v[c]);
  }
}

// ---------------------------------------------------------------- kernels
// AFF bit 0: gamma present, bit 1: beta present.
template <typename YT, typename ZT, typename ST, int BS, int NC, int AFF>
__global__ __launch_bounds__(BS) void layernorm_reg_kernel(const YT* __restrict__ Y, int64_t N, float eps,
                                                           const ST* __restrict__ gamma,
                                                           const ST* __restrict__ beta, ZT* __restrict__ Z) {
  __shared__ float red[2][BS / 64];
  const int64_t row = blockIdx.x;
  const YT* y = Y + row * N;
  ZT* z = Z + row * N;
  const int64_t nv = N / 4;
  const float inv_n = 1.f / (float)N;
  float v[NC][4];
  bool ok[NC];
  load_window<4, NC, BS>(y, nv, 0, v, ok);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += ok[c] ? v[c][e] : 0.f;
  const float mu = block_sum<BS>(s, red[0]) * inv_n;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = v[c][e] - mu;
      q += ok[c] ? d * d : 0.f;
    }
  const float rstd = 1.f / sqrtf(block_sum<BS>(q, red[1]) * inv_n + eps);
  // Affine vectors for the whole row are loaded together (one L2 round trip);
  // loading them in groups of chunks to save registers measured slower.
  float g[NC][4], bt[NC][4];
  bool okg[NC];
  if constexpr (AFF & 1) load_window<4, NC, BS>(gamma, nv, 0, g, okg);
  if constexpr (AFF & 2) load_window<4, NC, BS>(beta, nv, 0, bt, okg);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = (v[c][e] - mu) * rstd;
      if constexpr (AFF & 1) o[e] *= g[c][e];
      if constexpr (AFF & 2) o[e] += bt[c][e];
    }
    if (ok[c]) store_v<4>(z + ((int64_t)c * BS + threadIdx.x) * 4, o);
  }
}

// Any N and alignment: windows of LN_WIN chunks, three reads of the row.
template <typename YT, typename ZT, typename ST, int VEC>
__global__ __launch_bounds__(256) void layernorm_win_kernel(const YT* __restrict__ Y, int64_t N, float eps,
                                                            const ST* __restrict__ gamma,
                                                            const ST* __restrict__ beta, ZT* __restrict__ Z) {
  constexpr int BS = 256;
  __shared__ float red[2][BS / 64];
  const int64_t row = blockIdx.x;
  const YT* y = Y + row * N;
  ZT* z = Z + row * N;
  const int64_t nv = N / VEC;
  const int64_t chunks = (nv + BS - 1) / BS;
  const float inv_n = 1.f / (float)N;
  float v[LN_WIN][VEC];
  bool ok[LN_WIN];
  float s = 0.f;
  for (int64_t c0 = 0; c0 < chunks; c0 += LN_WIN) {
    load_window<VEC, LN_WIN, BS>(y, nv, c0, v, ok);
#pragma unroll
    for (int c = 0; c < LN_WIN; ++c)
#pragma unroll
      for (int e = 0; e < VEC; ++e) s += ok[c] ? v[c][e] : 0.f;
  }
  const float mu = block_sum<BS>(s, red[0]) * inv_n;
  float q = 0.f;
  for (int64_t c0 = 0; c0 < chunks; c0 += LN_WIN) {
    load_window<VEC, LN_WIN, BS>(y, nv, c0, v, ok);
#pragma unroll
    for (int c = 0; c < LN_WIN; ++c)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float d = v[c][e] - mu;
        q += ok[c] ? d * d : 0.f;
      }
  }
  const float rstd = 1.f / sqrtf(block_sum<BS>(q, red[1]) * inv_n + eps);
  for (int64_t c0 = 0; c0 < chunks; c0 += LN_WIN) {
    float g[LN_WIN][VEC], bt[LN_WIN][VEC];
    bool okg[LN_WIN];
    load_window<VEC, LN_WIN, BS>(y, nv, c0, v, ok);
    if (gamma) load_window<VEC, LN_WIN, BS>(gamma, nv, c0, g, okg);
    if (beta) load_window<VEC, LN_WIN, BS>(beta, nv, c0, bt, okg);
#pragma unroll
    for (int c = 0; c < LN_WIN; ++c) {
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        o[e] = (v[c][e] - mu) * rstd;
        if (gamma) o[e] *= g[c][e];
        if (beta) o[e] += bt[c][e];
      }
      if (ok[c]) store_v<VEC>(z + ((c0 + c) * BS + threadIdx.x) * VEC, o);
    }
  }
}

// ---------------------------------------------------------------- dispatch
template <typename YT, typename ZT, typename ST, int BS, int NC>
void launch_reg(dim3 grid, const YT* y, int64_t N, float eps, const ST* g, const ST* b, ZT* z, hipStream_t st) {
  const int aff = (g ? 1 : 0) | (b ? 2 : 0);
  if (aff == 3)
    hipLaunchKernelGGL((layernorm_reg_kernel<YT, ZT, ST, BS, NC, 3>), grid, dim3(BS), 0, st, y, N, eps, g, b, z);
  else if (aff == 2)
    hipLaunchKernelGGL((layernorm_reg_kernel<YT, ZT, ST, BS, NC, 2>), grid, dim3(BS), 0, st, y, N, eps, g, b, z);
  else if (aff == 1)
    hipLaunchKernelGGL((layernorm_reg_kernel<YT, ZT, ST, BS, NC, 1>), grid, dim3(BS), 0, st, y, N, eps, g, b, z);
  else
    hipLaunchKernelGGL((layernorm_reg_kernel<YT, ZT, ST, BS, NC, 0>), grid, dim3(BS), 0, st, y, N, eps, g, b, z);
}

template <typename YT, typename ZT, typename ST>
hipError_t launch_t(const void* Y, int64_t M, int64_t N, float eps, const void* gamma, const void* beta, void* Z,
                    hipStream_t st) {
  const YT* y = static_cast<const YT*>(Y);
  ZT* z = static_cast<ZT*>(Z);
  const ST* g = static_cast<const ST*>(gamma);
  const ST* b = static_cast<const ST*>(beta);
  const dim3 grid((unsigned)M);
  // Vector path: N % 4 == 0 and 4-element alignment of Y, Z, gamma, beta
  // (then every row start is aligned too).
  const auto al = [](const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; };
  const bool vec = N % 4 == 0 && al(Y, 4 * sizeof(YT)) && al(Z, 4 * sizeof(ZT)) && al(gamma, 4 * sizeof(ST)) &&
                   al(beta, 4 * sizeof(ST));
  const int64_t nv = N / 4;
  // Few rows: 16 waves per row so that one row is not bound by one CU's issue.
  if (vec && M < 256) {
    if (nv <= 1024 * 4) { launch_reg<YT, ZT, ST, 1024, 4>(grid, y, N, eps, g, b, z, st); return hipGetLastError(); }
    if (nv <= 1024 * 8) { launch_reg<YT, ZT, ST, 1024, 8>(grid, y, N, eps, g, b, z, st); return hipGetLastError(); }
  } else if (vec) {
    if (nv <= 256 * 4) { launch_reg<YT, ZT, ST, 256, 4>(grid, y, N, eps, g, b, z, st); return hipGetLastError(); }
    if (nv <= 256 * 8) { launch_reg<YT, ZT, ST, 256, 8>(grid, y, N, eps, g, b, z, st); return hipGetLastError(); }
    // 2 K..4 K vectors: 512 threads of 8 chunks rather than 256 of 16, which
    // halves the per-thread registers of the affine vectors (more waves per
    // CU): 2048 x 14336 with fp16 gamma, beta 35.2 -> 33.9 us, neutral without.
    if (nv <= 512 * 8) { launch_reg<YT, ZT, ST, 512, 8>(grid, y, N, eps, g, b, z, st); return hipGetLastError(); }
    if (nv <= 256 * 16) { launch_reg<YT, ZT, ST, 256, 16>(grid, y, N, eps, g, b, z, st); return hipGetLastError(); }
  }
  if (vec)
    hipLaunchKernelGGL((layernorm_win_kernel<YT, ZT, ST, 4>), grid, dim3(256), 0, st, y, N, eps, g, b, z);
  else
    hipLaunchKernelGGL((layernorm_win_kernel<YT, ZT, ST, 1>), grid, dim3(256), 0, st, y, N, eps, g, b, z);
  return hipGetLastError();
}

template <typename YT, typename ZT>
hipError_t launch_s(int g_dtype, const void* Y, int64_t M, int64_t N, float eps, const void* gamma,
                    const void* beta, void* Z, hipStream_t st) {
  return g_dtype == DT_F16 ? launch_t<YT, ZT, f16_t>(Y, M, N, eps, gamma, beta, Z, st)
                           : launch_t<YT, ZT, float>(Y, M, N, eps, gamma, beta, Z, st);
}

template <typename YT>
hipError_t launch_z(int z_dtype, int g_dtype, const void* Y, int64_t M, int64_t N, float eps, const void* gamma,
                    const void* beta, void* Z, hipStream_t st) {
  return z_dtype == DT_BF16 ? launch_s<YT, bf16_t>(g_dtype, Y, M, N, eps, gamma, beta, Z, st)
                            : launch_s<YT, float>(g_dtype, Y, M, N, eps, gamma, beta, Z, st);
}

}  // namespace

hipError_t launch_layernorm_rows(const void* Y, int y_dtype, int64_t M, int64_t N, float eps, const void* gamma,
                                 const void* beta, int g_dtype, void* Z, int z_dtype, hipStream_t st) {
  if (M < 1) return hipSuccess;
  if (M > 0x7fffffff) return hipErrorInvalidValue;
  // Without affine vectors their dtype is irrelevant: one instantiation serves.
  if (!gamma && !beta) g_dtype = DT_F32;
  return y_dtype == DT_BF16 ? launch_z<bf16_t>(z_dtype, g_dtype, Y, M, N, eps, gamma, beta, Z, st)
                            : launch_z<float>(z_dtype, g_dtype, Y, M, N, eps, gamma, beta, Z, st);
}

}  // namespace obl
