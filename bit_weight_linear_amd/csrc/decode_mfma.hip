// Decode contraction for 1 <= M <= 16 rows on the matrix cores, fp32-exact
// products: Y = ((X ⊙ b) W_sign^T) ⊙ a.
//
// OneBit page ("1bit量化"), proposition 1; DBF page ("Methodologie") for the
// two DBF stages, which call this kernel with (pre, post) = (b, m) and then
// (none, a).
//
// Why matrix cores at decode sizes: with M rows every weight feeds M signed
// additions, so plain fp32 VALU adds cost M operations per weight and are far
// slower than HBM for M >= 4.  A 16x16x32 bf16 MFMA performs 16 rows x 32 k of
// those additions at once.  To keep fp32 accuracy, x' = x ⊙ b is formed in fp32
// and split exactly into three bf16 terms hi + mid + lo (x' has at most 24
// significant bits); each term is multiplied by the +-1 matrix exactly and
// accumulated in fp32, so the only rounding is the fp32 accumulation, as in a
// plain fp32 add/sub loop.
//
// Work split: block = 4 waves x 16 columns (64 output columns) x one K-slice
// of 512 k.  Each block expands the A operand of its slice once into LDS
// (M padded to 16 rows, three terms, pair order -- see obl_common.hpp); each
// wave streams the sign words of its 16 columns and expands them to +-1 bf16
// in registers.  Slices of one column tile write fp32 partial sums to scratch;
// the last block to finish (device-scope counter) adds the slices in slice
// order, applies the post scale and writes Y.  The order of every sum is fixed,
// so results are bitwise reproducible; there are no float atomics.
#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_BN = 64;      // output columns per block (16 per wave)
constexpr int DEC_STEPS = 16;   // 32-k steps per K-slice

template <typename XT, typename ST, typename YT, bool PRE, bool VEC4>
__global__ __launch_bounds__(DEC_THREADS) void decode_mfma_kernel(
    const XT* __restrict__ X, int M, int64_t K, const uint32_t* __restrict__ W, int64_t N,
    const ST* __restrict__ pre, const ST* __restrict__ post, YT* __restrict__ Y, int nslices,
    float* __restrict__ partials, unsigned* __restrict__ counters) {
  __shared__ u32x4 afrag[3][DEC_STEPS][64];
  __shared__ int s_last;

  const int tile = blockIdx.x / nslices;
  const int slice = blockIdx.x - tile * nslices;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int64_t kw = K >> 5;
  const int64_t step0 = (int64_t)slice * DEC_STEPS;
  const int nsteps = (int)min((int64_t)DEC_STEPS, kw - step0);

  // 1. Sign words of this lane's column for the slice (all four lane groups of
  //    a column read the same 64 bytes).
  const int64_t col = (int64_t)tile * DEC_BN + wave * 16 + (lane & 15);
  uint32_t wreg[DEC_STEPS];
  {
    const uint32_t* src = W + col * kw + step0;
    const bool ok = col < N;
#pragma unroll
    for (int q = 0; q < DEC_STEPS / 4; ++q) {
      if (VEC4) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (ok && 4 * q < nsteps) v = *reinterpret_cast<const u32x4*>(src + 4 * q);
        wreg[4 * q + 0] = v.x;
        wreg[4 * q + 1] = v.y;
        wreg[4 * q + 2] = v.z;
        wreg[4 * q + 3] = v.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) wreg[4 * q + i] = (ok && 4 * q + i < nsteps) ? src[4 * q + i] : 0u;
      }
    }
  }

  // 2. A operand of the slice: x' = x·pre in fp32, split into three bf16 terms,
  //    in pair order.  Rows m >= M and steps past K are zero.
  for (int slot = tid; slot < DEC_STEPS * 64; slot += DEC_THREADS) {
    const int t = slot >> 6, l = slot & 63;
    const int m = l & 15, gg = l >> 4;
    u32x4 hi = u32x4{0u, 0u, 0u, 0u}, mid = hi, lo = hi;
    if (t < nsteps && m < M) {
      const int64_t kb = (step0 + t) * 32 + 4 * gg;
      const XT* xr = X + (int64_t)m * K + kb;
      uint32_t h[4], md[4], lw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float va = to_f32(xr[j]);
        float vb = to_f32(xr[j + 16]);
        if (PRE) {
          va *= to_f32(pre[kb + j]);
          vb *= to_f32(pre[kb + j + 16]);
        }
        const Split3 sa = split3(va), sb = split3(vb);
        h[j] = pack_bf16_pair(sa.hi, sb.hi);
        md[j] = pack_bf16_pair(sa.mid, sb.mid);
        lw[j] = pack_bf16_pair(sa.lo, sb.lo);
      }
      hi = u32x4{h[0], h[1], h[2], h[3]};
      mid = u32x4{md[0], md[1], md[2], md[3]};
      lo = u32x4{lw[0], lw[1], lw[2], lw[3]};
    }
    afrag[0][t][l] = hi;
    afrag[1][t][l] = mid;
    afrag[2][t][l] = lo;
  }
  __syncthreads();

  // 3. Contraction: two independent accumulators (even / odd steps).
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
  for (int t = 0; t < DEC_STEPS; ++t) {
    if (t < nsteps) {
      const u32x4 b = expand_signs_pm1(wreg[t] >> (4 * g));
      f32x4& acc = (t & 1) ? acc1 : acc0;
      acc = mfma16x16x32(afrag[0][t][lane], b, acc);
      acc = mfma16x16x32(afrag[1][t][lane], b, acc);
      acc = mfma16x16x32(afrag[2][t][lane], b, acc);
    }
  }
  const f32x4 acc = acc0 + acc1;

  // 4. Output: lane holds rows 4g .. 4g+3 of column `col`.
  if (nslices == 1) {
    if (col < N) {
      const float s = to_f32(post[col]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < M) Store<YT>::put(&Y[(int64_t)m * N + col], acc[i] * s);
      }
    }
    return;
  }
  if (col < N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < M) partials[((int64_t)slice * M + m) * N + col] = acc[i];
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&counters[tile], 1u) == (unsigned)(nslices - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int e = tid; e < M * DEC_BN; e += DEC_THREADS) {
    const int m = e / DEC_BN;
    const int64_t n = (int64_t)tile * DEC_BN + (e - m * DEC_BN);
    if (n >= N) continue;
    float s = 0.f;
    for (int sl = 0; sl < nslices; ++sl)
      s += __hip_atomic_load(&partials[((int64_t)sl * M + m) * N + n], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    Store<YT>::put(&Y[(int64_t)m * N + n], s * to_f32(post[n]));
  }
  if (tid == 0) atomicExch(&counters[tile], 0u);  // leave the counter at zero
}

template <typename XT, typename ST, typename YT, bool PRE>
hipError_t launch_t(const LinearArgs& a, const DeviceInfo& dev) {
  const int64_t kw = a.K / 32;
  const int64_t tiles = (a.N + DEC_BN - 1) / DEC_BN;
  const int64_t nslices = (kw + DEC_STEPS - 1) / DEC_STEPS;
  Scratch sc{};
  if (nslices > 1) {
    hipError_t e = scratch_reserve(dev.device, (size_t)(nslices * a.M * a.N), (size_t)tiles, &sc);
    if (e != hipSuccess) return e;
  }
  const bool vec4 = (kw % 4 == 0) && (reinterpret_cast<uintptr_t>(a.W) % 16 == 0);
  const int64_t blocks = tiles * nslices;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  auto X = static_cast<const XT*>(a.X);
  auto pre = static_cast<const ST*>(a.pre);
  auto post = static_cast<const ST*>(a.post);
  auto Y = static_cast<YT*>(a.Y);
  if (vec4)
    hipLaunchKernelGGL((decode_mfma_kernel<XT, ST, YT, PRE, true>), dim3((unsigned)blocks),
                       dim3(DEC_THREADS), 0, a.stream, X, (int)a.M, a.K, a.W, a.N, pre, post, Y,
                       (int)nslices, sc.partials, sc.counters);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<XT, ST, YT, PRE, false>), dim3((unsigned)blocks),
                       dim3(DEC_THREADS), 0, a.stream, X, (int)a.M, a.K, a.W, a.N, pre, post, Y,
                       (int)nslices, sc.partials, sc.counters);
  return hipGetLastError();
}

template <typename XT, typename ST, typename YT>
hipError_t launch_pre(const LinearArgs& a, const DeviceInfo& dev) {
  return a.pre ? launch_t<XT, ST, YT, true>(a, dev) : launch_t<XT, ST, YT, false>(a, dev);
}
template <typename XT, typename ST>
hipError_t launch_y(const LinearArgs& a, const DeviceInfo& dev) {
  return a.y_dtype == DT_F32 ? launch_pre<XT, ST, float>(a, dev) : launch_pre<XT, ST, bf16_t>(a, dev);
}
template <typename XT>
hipError_t launch_s(const LinearArgs& a, const DeviceInfo& dev) {
  return a.scale_dtype == DT_F32 ? launch_y<XT, float>(a, dev) : launch_y<XT, f16_t>(a, dev);
}

}  // namespace

hipError_t launch_decode_mfma(const LinearArgs& a, const DeviceInfo& dev) {
  if (a.M < 1 || a.M > kDecodeMaxM) return hipErrorInvalidValue;
  return a.x_dtype == DT_F32 ? launch_s<float>(a, dev) : launch_s<bf16_t>(a, dev);
}

}  // namespace obl
