// SVID conversion on the GPU: W ≈ W_sign ⊙ (a b^T).
//
// OneBit page ("1bit量化"), "rank-1 approximation" block and proposition 2:
// W_sign = Sign(W), and a b^T is the best rank-1 approximation of |W|, i.e.
// σ1 u1 v1^T from its leading singular triple.  The split of σ1 is
// a = sqrt(σ1) u1, b = sqrt(σ1) v1 with nonnegative singular vectors (|W| is
// entrywise nonnegative, so power iteration from a positive start stays
// positive and converges to them).
//
// Power iteration, every pass a bandwidth-bound read of the dense |W|:
//   v̂ = 1/sqrt(K);  repeat: u = |W| v̂, û = u / ||u||;  v = |W|^T û, v̂ = v / ||v||
//   finally u = |W| v̂, σ1 = ||u||, a = sqrt(σ1) u / σ1, b = sqrt(σ1) v̂.
// Row pass: one wave per row, lanes over k, fixed-order wave reduction.
// Column pass: blocks of 256 columns x 64 rows write partial column sums; a
// second kernel adds the row chunks in order and applies the 1/||u|| scale.
// Norms: one block, fixed order.  All sums are fp32 and reproducible.
#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

constexpr int SV_COLS = 256;     // columns per column-pass block
constexpr int SV_ROWS = 64;      // rows per column-pass block

template <typename T> __device__ __forceinline__ float absval(T v) { return fabsf(to_f32(v)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// u[i] = scale · Σ_k |W_ik| v[k], scale = 1 / *vnorm.
template <typename WT>
__global__ __launch_bounds__(256) void svid_rows_kernel(const WT* __restrict__ W, int64_t N, int64_t K,
                                                        const float* __restrict__ v,
                                                        const float* __restrict__ vnorm,
                                                        float* __restrict__ u) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;                                  // whole wave
  const WT* w = W + row * K;
  float acc = 0.f;
  for (int64_t k = lane; k < K; k += 64) acc += absval(w[k]) * v[k];
  acc = wave_sum(acc);
  if (lane == 0) u[row] = acc / *vnorm;
}

// part[c][k] = Σ_{i in chunk c} |W_ik| u[i].
template <typename WT>
__global__ __launch_bounds__(SV_COLS) void svid_cols_kernel(const WT* __restrict__ W, int64_t N, int64_t K,
                                                            const float* __restrict__ u,
                                                            float* __restrict__ part) {
  const int64_t k = (int64_t)blockIdx.x * SV_COLS + threadIdx.x;
  const int64_t c = blockIdx.y;
  const int64_t i0 = c * SV_ROWS, i1 = min(i0 + SV_ROWS, N);
  if (k >= K) return;
  float acc = 0.f;
  for (int64_t i = i0; i < i1; ++i) acc += absval(W[i * K + k]) * u[i];
  part[c * K + k] = acc;
}

// v[k] = (Σ_c part[c][k]) / *unorm, chunks added in order.
__global__ __launch_bounds__(256) void svid_cols_reduce_kernel(const float* __restrict__ part, int64_t chunks,
                                                               int64_t K, const float* __restrict__ unorm,
                                                               float* __restrict__ v) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  float acc = 0.f;
  for (int64_t c = 0; c < chunks; ++c) acc += part[c * K + k];
  v[k] = acc / *unorm;
}

// *out = sqrt(Σ x²), one block of 1024 threads, fixed order.
__global__ __launch_bounds__(1024) void svid_norm_kernel(const float* __restrict__ x, int64_t n,
                                                         float* __restrict__ out) {
  __shared__ float s[16];
  float acc = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += 1024) acc += x[i] * x[i];
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < 16; ++w) t += s[w];
    *out = sqrtf(t);
  }
}

// x[k] /= *norm in place.
__global__ __launch_bounds__(256) void svid_scale_kernel(float* x, int64_t n, const float* __restrict__ norm) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < n) x[k] = x[k] / *norm;
}

__global__ void svid_init_kernel(float* __restrict__ v, int64_t K, float* __restrict__ vnorm) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < K) v[k] = 1.f;
  if (k == 0) *vnorm = sqrtf((float)K);
}

// a = sqrt(σ) u / σ (σ = *unorm), b = sqrt(σ) v (v already unit length).
template <typename ST>
__global__ __launch_bounds__(256) void svid_final_kernel(const float* __restrict__ u, int64_t N,
                                                         const float* __restrict__ v, int64_t K,
                                                         const float* __restrict__ unorm,
                                                         ST* __restrict__ a, ST* __restrict__ b) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float sigma = *unorm;
  const float root = sqrtf(sigma);
  if (i < N) Store<ST>::put(&a[i], root * (u[i] / sigma));
  if (i < K) Store<ST>::put(&b[i], root * v[i]);
}

template <typename WT, typename ST>
hipError_t run(const void* Wv, int64_t N, int64_t K, int iters, void* av, void* bv, float* ws, hipStream_t st) {
  const WT* W = static_cast<const WT*>(Wv);
  const int64_t chunks = (N + SV_ROWS - 1) / SV_ROWS;
  float* u = ws;                     // [N]
  float* v = u + N;                  // [K]
  float* part = v + K;               // [chunks][K]
  float* scal = part + chunks * K;   // [0] = ||v||, [1] = ||u||
  const dim3 gr((unsigned)((N + 3) / 4)), gc((unsigned)((K + SV_COLS - 1) / SV_COLS), (unsigned)chunks);
  const dim3 gk((unsigned)((K + 255) / 256));
  hipLaunchKernelGGL(svid_init_kernel, gk, dim3(256), 0, st, v, K, scal);
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL((svid_rows_kernel<WT>), gr, dim3(256), 0, st, W, N, K, v, scal, u);
    hipLaunchKernelGGL(svid_norm_kernel, dim3(1), dim3(1024), 0, st, u, N, scal + 1);
    hipLaunchKernelGGL((svid_cols_kernel<WT>), gc, dim3(SV_COLS), 0, st, W, N, K, u, part);
    hipLaunchKernelGGL(svid_cols_reduce_kernel, gk, dim3(256), 0, st, part, chunks, K, scal + 1, v);
    hipLaunchKernelGGL(svid_norm_kernel, dim3(1), dim3(1024), 0, st, v, K, scal);
  }
  // v̂ = v / ||v||: fold into the last row pass (u = |W| v̂) and the final scale.
  hipLaunchKernelGGL((svid_rows_kernel<WT>), gr, dim3(256), 0, st, W, N, K, v, scal, u);
  hipLaunchKernelGGL(svid_norm_kernel, dim3(1), dim3(1024), 0, st, u, N, scal + 1);
  // b needs v̂.
  hipLaunchKernelGGL(svid_scale_kernel, gk, dim3(256), 0, st, v, K, scal);
  const int64_t nmax = N > K ? N : K;
  hipLaunchKernelGGL((svid_final_kernel<ST>), dim3((unsigned)((nmax + 255) / 256)), dim3(256), 0, st, u, N, v,
                     K, scal + 1, static_cast<ST*>(av), static_cast<ST*>(bv));
  return hipGetLastError();
}

template <typename WT>
hipError_t run_s(int scale_dtype, const void* W, int64_t N, int64_t K, int iters, void* a, void* b, float* ws,
                 hipStream_t st) {
  return scale_dtype == DT_F32 ? run<WT, float>(W, N, K, iters, a, b, ws, st)
                               : run<WT, f16_t>(W, N, K, iters, a, b, ws, st);
}

}  // namespace

size_t svid_workspace_floats(int64_t N, int64_t K) {
  const int64_t chunks = (N + SV_ROWS - 1) / SV_ROWS;
  return (size_t)(N + K + chunks * K + 8);
}

hipError_t launch_svid(const void* W, int w_dtype, int64_t N, int64_t K, int iters, void* a, void* b,
                       int scale_dtype, float* ws, hipStream_t st) {
  if (w_dtype == DT_F32) return run_s<float>(scale_dtype, W, N, K, iters, a, b, ws, st);
  if (w_dtype == DT_F16) return run_s<f16_t>(scale_dtype, W, N, K, iters, a, b, ws, st);
  return run_s<bf16_t>(scale_dtype, W, N, K, iters, a, b, ws, st);
}

}  // namespace obl
