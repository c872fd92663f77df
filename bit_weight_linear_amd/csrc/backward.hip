// Backward of the sign-binarised linear layer, and transposed sign packing.
//
// OneBit page ("1bit量化"), the knowledge-distillation block: the layer
// Y = [(X ⊙ g) W_±1^T] ⊙ h is trained by distillation, so its input and scale
// gradients are needed.  With g = b^T, h = a^T and an upstream gradient dY:
//   T  = (X ⊙ b^T) W_sign^T            [M][N]  (the forward sum before ⊙ a)
//   U  = (dY ⊙ a^T) W_sign             [M][K]
//   dX = U ⊙ b^T,   da_j = Σ_i dY_ij T_ij,   db_k = Σ_i x_ik U_ik.
// T and U are sign contractions; U contracts over N, so it runs the forward
// kernels on the transposed packing W_sign^T (packed along N), which
// transpose_signs_kernel builds once per weight.  This file holds that
// transpose and the reduction kernel that forms dX, da and db from T and U.
#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

// P[rows][K/32] -> PT[K][rows/32] (rows % 32 == 0).  One wave per (64 rows,
// one packed column word): lane l holds word w of row r0 + l; the ballot of
// bit j over the wave is the 64 signs of column 32w + j for those rows, i.e.
// two words of PT.  Lane j keeps the low word of ballot j, lane 32 + j the
// high word, and each lane writes its word.
__global__ __launch_bounds__(256) void transpose_signs_kernel(const uint32_t* __restrict__ P, int64_t rows,
                                                              int64_t kw, uint32_t* __restrict__ PT) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rblocks = (rows + 63) / 64;
  if (wid >= rblocks * kw) return;                       // whole wave exits together
  const int64_t rb = wid % rblocks, w = wid / rblocks;
  const int64_t r0 = rb * 64;
  const int64_t r = r0 + lane;
  const uint32_t word = r < rows ? P[r * kw + w] : 0u;
  uint32_t mine = 0u;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint64_t m = __ballot((word >> j) & 1u);
    if (lane == j) mine = (uint32_t)m;
    if (lane == 32 + j) mine = (uint32_t)(m >> 32);
  }
  const int64_t rw = rows / 32;                          // words per row of PT
  const int j = lane & 31;
  const int64_t col = 32 * w + j;                        // row of PT
  const int64_t word_idx = r0 / 32 + (lane >> 5);
  if (word_idx < rw) PT[col * rw + word_idx] = mine;
}

// Gradient reduction.  Blocks [0, bk) own 64 columns k of dX / db, blocks
// [bk, bk + bn) own 64 columns j of da.  Wave w of a block sums rows
// i = w, w + 4, ..., eight rows per batch: the batch's loads are issued
// together (row indexes clamped, terms masked) so a wave waits once per batch,
// not once per row.  The four wave partials are added in wave order in LDS
// (fixed order: bitwise reproducible).
template <typename XT, typename ST, typename DT>
__global__ __launch_bounds__(256) void backward_grads_kernel(
    const XT* __restrict__ dY, const XT* __restrict__ X, const float* __restrict__ T,
    const float* __restrict__ U, const ST* __restrict__ b, int64_t M, int64_t K, int64_t N,
    DT* __restrict__ dX, float* __restrict__ da, float* __restrict__ db, int bk) {
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float acc = 0.f;
  int64_t col;
  bool ok;
  if ((int)blockIdx.x < bk) {
    col = (int64_t)blockIdx.x * 64 + lane;
    ok = col < K;
    const int64_t cc = ok ? col : K - 1;
    const float bk_s = to_f32(b[cc]);
    for (int64_t i0 = wave; i0 < M; i0 += 4 * 8) {
      float u[8], x[8];
      bool okr[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        okr[r] = i0 + 4 * r < M;
        const int64_t i = okr[r] ? i0 + 4 * r : wave;   // row `wave` exists when the loop runs
        u[r] = U[i * K + cc];
        x[r] = to_f32(X[i * K + cc]);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        acc += okr[r] ? x[r] * u[r] : 0.f;
        if (okr[r] && ok) Store<DT>::put(&dX[(i0 + 4 * r) * K + col], u[r] * bk_s);
      }
    }
  } else {
    col = (int64_t)(blockIdx.x - bk) * 64 + lane;
    ok = col < N;
    const int64_t cc = ok ? col : N - 1;
    for (int64_t i0 = wave; i0 < M; i0 += 4 * 8) {
      float g[8], t[8];
      bool okr[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        okr[r] = i0 + 4 * r < M;
        const int64_t i = okr[r] ? i0 + 4 * r : wave;
        g[r] = to_f32(dY[i * N + cc]);
        t[r] = T[i * N + cc];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) acc += okr[r] ? g[r] * t[r] : 0.f;
    }
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && ok) {
    const float s = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
    if ((int)blockIdx.x < bk) db[col] = s;
    else da[col] = s;
  }
}

template <typename XT, typename ST, typename DT>
hipError_t launch_grads(const void* dY, const void* X, const float* T, const float* U, const void* b,
                        int64_t M, int64_t K, int64_t N, void* dX, float* da, float* db, hipStream_t st) {
  const int64_t bk = (K + 63) / 64, bn = (N + 63) / 64;
  hipLaunchKernelGGL((backward_grads_kernel<XT, ST, DT>), dim3((unsigned)(bk + bn)), dim3(256), 0, st,
                     static_cast<const XT*>(dY), static_cast<const XT*>(X), T, U, static_cast<const ST*>(b),
                     M, K, N, static_cast<DT*>(dX), da, db, (int)bk);
  return hipGetLastError();
}

template <typename XT, typename ST>
hipError_t launch_grads_d(int dx_dtype, const void* dY, const void* X, const float* T, const float* U,
                          const void* b, int64_t M, int64_t K, int64_t N, void* dX, float* da, float* db,
                          hipStream_t st) {
  return dx_dtype == DT_F32 ? launch_grads<XT, ST, float>(dY, X, T, U, b, M, K, N, dX, da, db, st)
                            : launch_grads<XT, ST, bf16_t>(dY, X, T, U, b, M, K, N, dX, da, db, st);
}

}  // namespace

hipError_t launch_transpose_signs(const uint32_t* P, int64_t rows, int64_t K, uint32_t* PT, hipStream_t st) {
  const int64_t kw = K / 32;
  const int64_t waves = ((rows + 63) / 64) * kw;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_signs_kernel, dim3((unsigned)blocks), dim3(256), 0, st, P, rows, kw, PT);
  return hipGetLastError();
}

hipError_t launch_backward_grads(int x_dtype, int scale_dtype, int dx_dtype, const void* dY, const void* X,
                                 const float* T, const float* U, const void* b, int64_t M, int64_t K,
                                 int64_t N, void* dX, float* da, float* db, hipStream_t st) {
  if (x_dtype == DT_F32)
    return scale_dtype == DT_F32 ? launch_grads_d<float, float>(dx_dtype, dY, X, T, U, b, M, K, N, dX, da, db, st)
                                 : launch_grads_d<float, f16_t>(dx_dtype, dY, X, T, U, b, M, K, N, dX, da, db, st);
  return scale_dtype == DT_F32 ? launch_grads_d<bf16_t, float>(dx_dtype, dY, X, T, U, b, M, K, N, dX, da, db, st)
                               : launch_grads_d<bf16_t, f16_t>(dx_dtype, dY, X, T, U, b, M, K, N, dX, da, db, st);
}

}  // namespace obl
