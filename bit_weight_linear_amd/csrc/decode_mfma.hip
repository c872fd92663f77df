// Decode contraction for 1 <= M <= 16 rows on the matrix cores with
// fp32-exact products: Y = ((X ⊙ b) W_sign^T) ⊙ a.
//
// OneBit page ("1bit量化"), proposition 1; DBF page ("Methodologie") for the
// two DBF stages, which run this kernel with (pre, post) = (b, m) and then
// (none, a).
//
// Why matrix cores at decode sizes: with M rows every weight feeds M signed
// additions, so plain fp32 VALU adds cost M operations per weight and fall far
// behind HBM for M >= 4.  A 16x16x32 bf16 MFMA does 16 rows x 32 k of those
// additions at once.  fp32 accuracy is kept by making every product exact and
// accumulating in fp32 (the only rounding, as in a plain fp32 add/sub loop):
//   mode B2 (bf16 x, fp16 b): A = x as stored; b is split exactly into two
//       bf16 terms b = b_hi + b_lo (fp16 has 11 significant bits) which are
//       folded into the sign operand: x·(±b_hi) + x·(±b_lo), 2 MFMAs per step;
//   mode B1 (bf16 x, no b):   A = x, B = ±1, 1 MFMA per step;
//   mode S3 (fp32 x or fp32 b): x' = x·b in fp32, split exactly into three
//       bf16 terms hi + mid + lo (24 significant bits), B = ±1, 3 MFMAs.
// The sign operand is expanded in registers from the packed words (pair
// order, obl_common.hpp).
//
// Work split: block = 4 waves x 16 columns (64 output columns) x one K-slice
// of 512 k, so each block reads only its slice of X.  With one slice the
// block applies the post scale and writes Y; otherwise slices write fp32
// partial sums to scratch and a second small kernel adds them in slice order
// (the kernel boundary orders the memory traffic; no fences, no atomics), so
// results are bitwise reproducible.
#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_BN = 64;      // output columns per block (16 per wave)
constexpr int DEC_STEPS = 16;   // 32-k steps per K-slice
constexpr int DEC_SLOTS = DEC_STEPS * 64;
constexpr int DEC_SLOTS_PER_THREAD = DEC_SLOTS / DEC_THREADS;

enum DecMode { MODE_B2 = 0, MODE_B1 = 1, MODE_S3 = 2 };

template <int MODE> struct DecTerms { static constexpr int A = (MODE == MODE_S3) ? 3 : 1; };

__device__ __forceinline__ u32x4 interleave_runs(u32x2 r0, u32x2 r1) {
  u32x4 o;
  o.x = __builtin_amdgcn_perm(r1.x, r0.x, 0x05040100u);
  o.y = __builtin_amdgcn_perm(r1.x, r0.x, 0x07060302u);
  o.z = __builtin_amdgcn_perm(r1.y, r0.y, 0x05040100u);
  o.w = __builtin_amdgcn_perm(r1.y, r0.y, 0x07060302u);
  return o;
}

template <int MODE, typename XT, typename ST, typename YT, bool PRE, bool VEC4>
__global__ __launch_bounds__(DEC_THREADS) void decode_mfma_kernel(
    const XT* __restrict__ X, int M, int64_t K, const uint32_t* __restrict__ W, int64_t N,
    const ST* __restrict__ pre, const ST* __restrict__ post, YT* __restrict__ Y, int nslices,
    float* __restrict__ partials) {
  constexpr int TA = DecTerms<MODE>::A;
  __shared__ u32x4 afrag[TA][DEC_STEPS][64];
  __shared__ u32x4 mag[DEC_STEPS][4][2];  // mode B2: (b_hi, b_lo) bf16 pairs per (step, lane group)

  const int tile = blockIdx.x / nslices;
  const int slice = blockIdx.x - tile * nslices;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int64_t kw = K >> 5;
  const int64_t step0 = (int64_t)slice * DEC_STEPS;
  const int nsteps = (int)min((int64_t)DEC_STEPS, kw - step0);

  // ---- 1. Issue every global load of the block, branch-free.
  // A operand (slot = (step t, lane l)): rows m = l % 16, k runs 4g..4g+3 and 4g+16..4g+19.
  u32x2 xr0[DEC_SLOTS_PER_THREAD], xr1[DEC_SLOTS_PER_THREAD];   // bf16 modes
  float xs[DEC_SLOTS_PER_THREAD][8];                              // S3 mode
  uint32_t aval = 0;
#pragma unroll
  for (int i = 0; i < DEC_SLOTS_PER_THREAD; ++i) {
    const int slot = tid + DEC_THREADS * i;
    const int t = slot >> 6, l = slot & 63;
    const int m = l & 15, gg = l >> 4;
    const bool ok = t < nsteps && m < M;
    aval |= uint32_t(ok) << i;
    const int64_t kb = (step0 + t) * 32 + 4 * gg;
    const XT* xp = X + (ok ? (int64_t)m * K + kb : 0);
    if constexpr (MODE != MODE_S3) {
      xr0[i] = *reinterpret_cast<const u32x2*>(xp);
      xr1[i] = *reinterpret_cast<const u32x2*>(xp + 16);
    } else {
      const ST* pp = pre + (ok ? kb : 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float lo = to_f32(xp[j]), hi = to_f32(xp[j + 16]);
        if constexpr (PRE) {
          lo *= to_f32(pp[j]);
          hi *= to_f32(pp[j + 16]);
        }
        xs[i][j] = lo;
        xs[i][4 + j] = hi;
      }
    }
  }
  // Sign words of this lane's column for the slice.
  const int64_t col = (int64_t)tile * DEC_BN + wave * 16 + (lane & 15);
  const bool colok = col < N;
  uint32_t wreg[DEC_STEPS];
  {
    const uint32_t* src = W + (colok ? col : 0) * kw + step0;
#pragma unroll
    for (int q = 0; q < DEC_STEPS / 4; ++q) {
      if (VEC4) {
        const bool ok = colok && 4 * q < nsteps;
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + (4 * q < nsteps ? 4 * q : 0));
        wreg[4 * q + 0] = ok ? v.x : 0u;
        wreg[4 * q + 1] = ok ? v.y : 0u;
        wreg[4 * q + 2] = ok ? v.z : 0u;
        wreg[4 * q + 3] = ok ? v.w : 0u;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = colok && 4 * q + i < nsteps;
          const uint32_t v = src[4 * q + i < nsteps ? 4 * q + i : 0];
          wreg[4 * q + i] = ok ? v : 0u;
        }
      }
    }
  }
  // Mode B2: b for (step, lane group) = tid < 64.
  float bl[8];
  const bool magok = tid < DEC_STEPS * 4 && (tid >> 2) < nsteps;
  if constexpr (MODE == MODE_B2) {
    const int64_t kb = (step0 + (tid >> 2)) * 32 + 4 * (tid & 3);
    const ST* pp = pre + (magok ? kb : 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bl[j] = to_f32(pp[j]);
      bl[4 + j] = to_f32(pp[j + 16]);
    }
  }
  const float post_c = to_f32(post[colok ? col : 0]);

  // ---- 2. Operands into LDS.
#pragma unroll
  for (int i = 0; i < DEC_SLOTS_PER_THREAD; ++i) {
    const int slot = tid + DEC_THREADS * i;
    const int t = slot >> 6, l = slot & 63;
    const bool ok = (aval >> i) & 1u;
    if constexpr (MODE != MODE_S3) {
      const u32x4 v = interleave_runs(xr0[i], xr1[i]);
      afrag[0][t][l] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    } else {
      uint32_t h[4], md[4], lw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const Split3 sa = split3(ok ? xs[i][j] : 0.f), sb = split3(ok ? xs[i][4 + j] : 0.f);
        h[j] = pack_bf16_pair(sa.hi, sb.hi);
        md[j] = pack_bf16_pair(sa.mid, sb.mid);
        lw[j] = pack_bf16_pair(sa.lo, sb.lo);
      }
      afrag[0][t][l] = u32x4{h[0], h[1], h[2], h[3]};
      afrag[TA > 1 ? 1 : 0][t][l] = u32x4{md[0], md[1], md[2], md[3]};
      afrag[TA > 2 ? 2 : 0][t][l] = u32x4{lw[0], lw[1], lw[2], lw[3]};
    }
  }
  if constexpr (MODE == MODE_B2) {
    if (tid < DEC_STEPS * 4) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a0 = magok ? bl[j] : 0.f, a1 = magok ? bl[4 + j] : 0.f;
        const float h0 = bf16_round(a0), h1 = bf16_round(a1);
        hi[j] = pack_bf16_pair(h0, h1);
        lo[j] = pack_bf16_pair(a0 - h0, a1 - h1);  // exact: fp16 residual fits bf16
      }
      mag[tid >> 2][tid & 3][0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      mag[tid >> 2][tid & 3][1] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  }
  __syncthreads();

  // ---- 3. Contraction: two independent accumulators (even / odd steps).
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
  for (int t = 0; t < DEC_STEPS; ++t) {
    if (t < nsteps) {
      const uint32_t ws = wreg[t] >> (4 * g);
      f32x4& acc = (t & 1) ? acc1 : acc0;
      if constexpr (MODE == MODE_B2) {
        const u32x4 a = afrag[0][t][lane];
        acc = mfma16x16x32(a, expand_signs_scaled(ws, mag[t][g][0]), acc);
        acc = mfma16x16x32(a, expand_signs_scaled(ws, mag[t][g][1]), acc);
      } else {
        const u32x4 b = expand_signs_pm1(ws);
#pragma unroll
        for (int u = 0; u < TA; ++u) acc = mfma16x16x32(afrag[u][t][lane], b, acc);
      }
    }
  }
  const f32x4 acc = acc0 + acc1;

  // ---- 4. Output: lane holds rows 4g .. 4g+3 of column `col`.
  if (!colok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * g + i;
    if (m >= M) break;
    if (nslices == 1) Store<YT>::put(&Y[(int64_t)m * N + col], acc[i] * post_c);
    else partials[((int64_t)slice * M + m) * N + col] = acc[i];
  }
}

// Y[m][n] = (Σ_s partials[s][m][n]) · post[n], slices added in order.
template <typename ST, typename YT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partials,
                                                            int nslices, int64_t MN, int64_t N,
                                                            const ST* __restrict__ post,
                                                            YT* __restrict__ Y) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= MN) return;
  const int64_t n = e % N;
  const float s = to_f32(post[n]);
  float acc = 0.f;
  int sl = 0;
  for (; sl + 8 <= nslices; sl += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partials[(int64_t)(sl + u) * MN + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; sl < nslices; ++sl) acc += partials[(int64_t)sl * MN + e];
  Store<YT>::put(&Y[e], acc * s);
}

template <int MODE, typename XT, typename ST, typename YT, bool PRE>
hipError_t launch_t(const LinearArgs& a, const DeviceInfo& dev) {
  const int64_t kw = a.K / 32;
  const int64_t tiles = (a.N + DEC_BN - 1) / DEC_BN;
  const int64_t nslices = (kw + DEC_STEPS - 1) / DEC_STEPS;
  Scratch sc{};
  if (nslices > 1) {
    hipError_t e = scratch_reserve(dev.device, (size_t)(nslices * a.M * a.N), &sc);
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
    hipLaunchKernelGGL((decode_mfma_kernel<MODE, XT, ST, YT, PRE, true>), dim3((unsigned)blocks),
                       dim3(DEC_THREADS), 0, a.stream, X, (int)a.M, a.K, a.W, a.N, pre, post, Y,
                       (int)nslices, sc.partials);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<MODE, XT, ST, YT, PRE, false>), dim3((unsigned)blocks),
                       dim3(DEC_THREADS), 0, a.stream, X, (int)a.M, a.K, a.W, a.N, pre, post, Y,
                       (int)nslices, sc.partials);
  if (nslices > 1) {
    const int64_t MN = a.M * a.N;
    hipLaunchKernelGGL((splitk_reduce_kernel<ST, YT>), dim3((unsigned)((MN + 255) / 256)), dim3(256), 0,
                       a.stream, sc.partials, (int)nslices, MN, a.N, post, Y);
  }
  return hipGetLastError();
}

template <typename ST, typename YT>
hipError_t launch_mode(const LinearArgs& a, const DeviceInfo& dev) {
  // bf16 x with an 8-byte aligned base: A is x itself.
  const bool raw = a.x_dtype == DT_BF16 && (reinterpret_cast<uintptr_t>(a.X) % 8 == 0);
  if (raw && !a.pre) return launch_t<MODE_B1, bf16_t, ST, YT, false>(a, dev);
  if (raw && a.scale_dtype == DT_F16) return launch_t<MODE_B2, bf16_t, ST, YT, true>(a, dev);
  if (a.x_dtype == DT_BF16)
    return a.pre ? launch_t<MODE_S3, bf16_t, ST, YT, true>(a, dev)
                 : launch_t<MODE_S3, bf16_t, ST, YT, false>(a, dev);
  return a.pre ? launch_t<MODE_S3, float, ST, YT, true>(a, dev)
               : launch_t<MODE_S3, float, ST, YT, false>(a, dev);
}
template <typename ST>
hipError_t launch_y(const LinearArgs& a, const DeviceInfo& dev) {
  return a.y_dtype == DT_F32 ? launch_mode<ST, float>(a, dev) : launch_mode<ST, bf16_t>(a, dev);
}

}  // namespace

hipError_t launch_decode_mfma(const LinearArgs& a, const DeviceInfo& dev) {
  if (a.M < 1 || a.M > kDecodeMaxM) return hipErrorInvalidValue;
  return a.scale_dtype == DT_F32 ? launch_y<float>(a, dev) : launch_y<f16_t>(a, dev);
}

}  // namespace obl
