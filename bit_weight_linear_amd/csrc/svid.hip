// SVID conversion on the GPU: W ≈ W_sign ⊙ (a b^T).
//
// OneBit page ("1bit量化"), "rank-1 approximation" block and proposition 2:
// W_sign = Sign(W), and a b^T is the best rank-1 approximation of |W|, i.e.
// σ1 u1 v1^T from its leading singular triple.  The split of σ1 is
// a = sqrt(σ1) u1, b = sqrt(σ1) v1 with nonnegative singular vectors (|W| is
// entrywise nonnegative, so power iteration from a positive start stays
// positive and converges to them).
//
// Power iteration; every pass is a bandwidth-bound read of the dense |W|:
//   v = 1;  repeat: u = |W| v / ||v||;  v = |W|^T u / ||u||
//   finally u = |W| v / ||v||, σ1 = ||u||, a = u / sqrt(σ1), b = sqrt(σ1) v / ||v||.
// Three kernels per iteration, none of them a single workgroup:
//  * row pass: a workgroup takes 8 rows (2 per wave), stages v through LDS
//    in tiles shared by its 4 waves (the staging overlaps the weight loads),
//    reads W with 16-byte loads, and also
//    forms ||v||^2 from the tiles it stages (the same fixed-order sum in every
//    workgroup, so every u_i is divided by the same value); it writes u and
//    the workgroup's Σ u_i^2 (rows in order);
//  * column pass: 4 columns per thread (one 8- or 16-byte load per row),
//    64 rows per workgroup, partial column sums part[chunk][k];
//  * column reduction: 32 threads per 4 columns add the chunks (lane l takes
//    chunks l, l + 32, ...; lanes added in order), ||u|| from the row pass's
//    per-workgroup sums (fixed order), v = Σ part / ||u||.
// Loads are issued unconditionally with indexes clamped inside the matrix and
// masked out of the sums (no per-lane branch around a load, so a thread's loads
// are in flight together).  All sums are fp32 in a fixed order: bitwise
// reproducible.
#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

constexpr int SV_RPB = 8;        // rows per row-pass workgroup (2 per wave)
constexpr int SV_CHUNK = 64;     // rows per column-pass workgroup
constexpr int SV_CPT = 4;        // columns per column-pass thread
constexpr int SV_CLANES = 32;    // chunk lanes per column quad in the reduction
constexpr int SV_RCOLS = 4 * (256 / SV_CLANES);   // columns per reduction workgroup (32)

template <typename T> __device__ __forceinline__ float absval(T v) { return fabsf(to_f32(v)); }

// V consecutive elements as one raw load (16 bytes for V = 16 / sizeof(T), 8
// bytes for 16-bit types at V = 4, one element at V = 1), and their absolute
// values as floats.  Loading and converting are separate so that the loads of
// a thread can all be issued before any of them is waited for.
template <int V, typename T> struct Raw;
template <typename T> struct Raw<1, T> {
  using type = T;
  static __device__ __forceinline__ type load(const T* p) { return *p; }
  static __device__ __forceinline__ void abs(const type& q, float o[1]) { o[0] = absval(q); }
};
template <> struct Raw<4, float> {
  using type = float4;
  static __device__ __forceinline__ type load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  static __device__ __forceinline__ void abs(const type& q, float o[4]) {
    o[0] = fabsf(q.x); o[1] = fabsf(q.y); o[2] = fabsf(q.z); o[3] = fabsf(q.w);
  }
};
template <typename T> struct Raw<4, T> {   // 16-bit types: 8 bytes
  using type = uint2;
  static __device__ __forceinline__ type load(const T* p) { return *reinterpret_cast<const uint2*>(p); }
  static __device__ __forceinline__ void abs(const type& q, float o[4]) {
    const T* h = reinterpret_cast<const T*>(&q);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = absval(h[e]);
  }
};
template <typename T> struct Raw<8, T> {   // 16-bit types: 16 bytes
  using type = uint4;
  static __device__ __forceinline__ type load(const T* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ void abs(const type& q, float o[8]) {
    const T* h = reinterpret_cast<const T*>(&q);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = absval(h[e]);
  }
};

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Fixed-order sum over the 64 lanes (quad xors, half-mirror, mirror, then the
// four 16-lane rows in order); wave-uniform result.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// Sum over a 256-thread workgroup (waves in order); `red` is used once.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Σ over x[0..n) of x^2, or of x, by a 256-thread workgroup in a fixed order
// (n >= 1).  Loads go out 8 at a time (clamped indexes, masked terms) rather
// than one round trip per element.
template <bool SQUARE>
__device__ __forceinline__ float block_total(const float* __restrict__ x, int64_t n, float* red) {
  float s = 0.f;
  for (int64_t i0 = threadIdx.x; i0 < n; i0 += 8 * 256) {
    float t[8];
    bool ok[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t i = i0 + (int64_t)r * 256;
      ok[r] = i < n;
      t[r] = x[ok[r] ? i : 0];
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) s += ok[r] ? (SQUARE ? t[r] * t[r] : t[r]) : 0.f;
  }
  return block_sum(s, red);
}

// ---------------------------------------------------------------- row pass
// Barrier for LDS traffic only: wait for this wave's LDS operations, then
// s_barrier.  __syncthreads() would also wait for every global load in flight
// (its fence drains vmcnt), i.e. for the weight loads issued ahead of it.  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// u[i] = Σ_k |W_ik| v[k] / ||v||;  upart[block] = Σ over its rows of u[i]^2.
// Element (j, e) of lane l in a tile is column t0 + (64 j + l) · V + e.  Per
// tile: the v loads for staging (L2), then the 16 weight loads (HBM), then v is
// written to LDS once its loads land (memory returns in issue order, so this
// waits only for v) and the weights stream in behind the barrier.
template <typename WT, int V>
__global__ __launch_bounds__(256) void svid_rows_kernel(const WT* __restrict__ W, int64_t N, int64_t K,
                                                        const float* __restrict__ v, float* __restrict__ u,
                                                        float* __restrict__ upart) {
  constexpr int TILE = 512 * V;
  constexpr int NVL = TILE >= 1024 ? TILE / 1024 : 1;    // float4 staging loads per thread
  // At least NVL · 1024 floats: every staging store lands inside, also past
  // the tile's end (those slots are never read).
  __shared__ __align__(16) float vs[TILE < 1024 ? 1024 : TILE];
  __shared__ float red[4];
  __shared__ float uu[SV_RPB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * SV_RPB + 2 * wave;
  const WT* w0 = W + min(r0, N - 1) * K;
  const WT* w1 = W + min(r0 + 1, N - 1) * K;
  float acc0 = 0.f, acc1 = 0.f, vsq = 0.f;
  for (int64_t t0 = 0; t0 < K; t0 += TILE) {
    const int tl = (int)min((int64_t)TILE, K - t0);      // a multiple of 32 (K % 32 == 0)
    float4 vv[NVL];
    bool okv[NVL];
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int f = (256 * i + tid) * 4;
      okv[i] = f < tl;
      vv[i] = *reinterpret_cast<const float4*>(v + t0 + (okv[i] ? f : 0));
    }
    __builtin_amdgcn_sched_barrier(0);
    typename Raw<V, WT>::type q0[8], q1[8];
    bool ok[8];
    int ec[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = (64 * j + lane) * V;
      ok[j] = e < tl;
      ec[j] = ok[j] ? e : tl - V;
      q0[j] = Raw<V, WT>::load(w0 + t0 + ec[j]);
      q1[j] = Raw<V, WT>::load(w1 + t0 + ec[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (t0 > 0) lds_barrier();                           // every wave is done reading the previous tile
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int f = (256 * i + tid) * 4;
      reinterpret_cast<float4*>(vs)[f >> 2] = vv[i];     // unconditional: no branch for the load to sink into
      vsq += okv[i] ? ((vv[i].x * vv[i].x + vv[i].y * vv[i].y) + (vv[i].z * vv[i].z + vv[i].w * vv[i].w)) : 0.f;
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a0[V], a1[V], x[V];
      Raw<V, WT>::abs(q0[j], a0);
      Raw<V, WT>::abs(q1[j], a1);
      if constexpr (V % 4 == 0) {
#pragma unroll
        for (int e = 0; e < V; e += 4) {
          const float4 t = reinterpret_cast<const float4*>(vs)[(ec[j] + e) >> 2];
          x[e] = t.x; x[e + 1] = t.y; x[e + 2] = t.z; x[e + 3] = t.w;
        }
      } else {
        x[0] = vs[ec[j]];
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        acc0 += ok[j] ? a0[e] * x[e] : 0.f;
        acc1 += ok[j] ? a1[e] * x[e] : 0.f;
      }
    }
  }
  const float vnorm = sqrtf(block_sum(vsq, red));
  const float s0 = wave_sum(acc0) / vnorm, s1 = wave_sum(acc1) / vnorm;
  if (lane == 0) {
    if (r0 < N) u[r0] = s0;
    if (r0 + 1 < N) u[r0 + 1] = s1;
    uu[2 * wave] = r0 < N ? s0 * s0 : 0.f;
    uu[2 * wave + 1] = r0 + 1 < N ? s1 * s1 : 0.f;
  }
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < SV_RPB; ++r) t += uu[r];
    upart[blockIdx.x] = t;
  }
}

// ---------------------------------------------------------------- column pass
// part[c][k..k+CV) = Σ_{i in chunk c} |W_ik| u[i].
template <typename WT, int CV>
__global__ __launch_bounds__(256) void svid_cols_kernel(const WT* __restrict__ W, int64_t N, int64_t K,
                                                        const float* __restrict__ u, float* __restrict__ part) {
  const int64_t k = ((int64_t)blockIdx.x * 256 + threadIdx.x) * CV;
  const int64_t c = blockIdx.y;
  const int64_t i0 = c * SV_CHUNK, i1 = min(i0 + SV_CHUNK, N);
  if (k >= K) return;                                    // no barrier in this kernel
  float acc[CV];
#pragma unroll
  for (int e = 0; e < CV; ++e) acc[e] = 0.f;
  for (int64_t i = i0; i < i1; i += 8) {
    typename Raw<CV, WT>::type q[8];
    float ui[8];
    bool ok[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      ok[r] = i + r < i1;
      const int64_t ri = ok[r] ? i + r : i1 - 1;
      q[r] = Raw<CV, WT>::load(W + ri * K + k);
      ui[r] = u[ri];
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float w[CV];
      Raw<CV, WT>::abs(q[r], w);
#pragma unroll
      for (int e = 0; e < CV; ++e) acc[e] += ok[r] ? w[e] * ui[r] : 0.f;
    }
  }
#pragma unroll
  for (int e = 0; e < CV; ++e) part[c * K + k + e] = acc[e];
}

// ---------------------------------------------------------------- fused pass
// One read of W per iteration (rows of at most 512·V elements): a workgroup
// of 4 waves takes rows [rb, rb + rpw), two per wave at a time (the next two
// already loading), with v in LDS.  From the same registers it forms
// u_i = |W_i| · v / ||v|| and adds |W_ik| u_i into per-lane column sums, so
// the column pass no longer reads W again.  At the end the four waves' column
// sums are added in wave order into part[block][K], and upart[block] = Σ u_i^2
// over its rows (rows in order within a wave, then the waves in order).  The
// column reduction then forms v from the blocks' partial rows as before.
// Element (j, e) of lane l is column (64 j + l) · V + e (j < SV_FJ).
constexpr int SV_FJ = 8;
template <typename WT, int V>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void svid_fused_kernel(const WT* __restrict__ W, int64_t N, int64_t K, int64_t rpw, const float* __restrict__ v,
                       float* __restrict__ u, float* __restrict__ upart, float* __restrict__ part,
                       float* __restrict__ sink) {
  using RT = typename Raw<V, WT>::type;
  constexpr int KMAX = 64 * SV_FJ * V;
  __shared__ __align__(16) float vs[KMAX];
  __shared__ __align__(16) float cs[4][KMAX];
  __shared__ float red[4];
  __shared__ float usw[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // v into LDS and ||v||^2 (the same fixed order in every workgroup).
  float vsq = 0.f;
#pragma unroll
  for (int i = 0; i < KMAX / 1024; ++i) {
    const int f = (256 * i + tid) * 4;
    const bool okv = f < K;
    const float4 t = *reinterpret_cast<const float4*>(v + (okv ? f : 0));
    // Zeros past K: the dot products below then need no mask (|w| · 0).
    reinterpret_cast<float4*>(vs)[f >> 2] = okv ? t : float4{0.f, 0.f, 0.f, 0.f};
    vsq += okv ? ((t.x * t.x + t.y * t.y) + (t.z * t.z + t.w * t.w)) : 0.f;
  }
  const float vnorm = sqrtf(block_sum(vsq, red));   // its barrier also publishes vs

  const int64_t rb = (int64_t)blockIdx.x * rpw, re = min(rb + rpw, N);
  // Weight loads past K re-read the last V columns (in bounds, finite); the
  // products use the unclamped column, whose v slot past K is zero.
  int ec[SV_FJ];
#pragma unroll
  for (int j = 0; j < SV_FJ; ++j) {
    const int e = (64 * j + lane) * V;
    ec[j] = e < K ? e : (int)K - V;
  }
  auto load = [&](int64_t r, RT (&q)[SV_FJ]) {   // rows past N re-read row N - 1 (unused)
    const WT* w = W + min(r, N - 1) * K;
#pragma unroll
    for (int j = 0; j < SV_FJ; ++j) q[j] = Raw<V, WT>::load(w + ec[j]);
  };
  float cp[SV_FJ][V];
#pragma unroll
  for (int j = 0; j < SV_FJ; ++j)
#pragma unroll
    for (int e = 0; e < V; ++e) cp[j][e] = 0.f;
  float usq = 0.f;
  // Rows r and r + 1 from q0, q1: dot products, u, column sums.
  auto process = [&](int64_t r, const RT (&q0)[SV_FJ], const RT (&q1)[SV_FJ]) {
    float a0[SV_FJ][V], a1[SV_FJ][V];
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < SV_FJ; ++j) {
      Raw<V, WT>::abs(q0[j], a0[j]);
      Raw<V, WT>::abs(q1[j], a1[j]);
      float x[V];
#pragma unroll
      for (int e = 0; e < V; e += 4) {
        const float4 t = reinterpret_cast<const float4*>(vs)[((64 * j + lane) * V + e) >> 2];
        x[e] = t.x; x[e + 1] = t.y; x[e + 2] = t.z; x[e + 3] = t.w;
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {   // columns past K meet v = 0
        s0 += a0[j][e] * x[e];
        s1 += a1[j][e] * x[e];
      }
    }
    const float u0 = wave_sum(s0) / vnorm, u1 = wave_sum(s1) / vnorm;
    const float m0 = r < re ? u0 : 0.f, m1 = r + 1 < re ? u1 : 0.f;
    // Every lane stores the (wave-uniform) values, rows past re into the sink
    // slot: no branch around a store (its join would wait for every load in
    // flight, the prefetched rows included).
    *(r < re ? u + r : sink) = u0;
    *(r + 1 < re ? u + r + 1 : sink) = u1;
    usq += m0 * m0;
    usq += m1 * m1;
#pragma unroll
    for (int j = 0; j < SV_FJ; ++j)
#pragma unroll
      for (int e = 0; e < V; ++e) {
        cp[j][e] += a0[j][e] * m0;
        cp[j][e] += a1[j][e] * m1;
      }
  };
  // Wave w takes rows rb + 2w + 8i and the next, two at a time, the next
  // two already loading.  Both halves of a step are unconditional (rows past
  // re are masked inside process).
  RT qa0[SV_FJ], qa1[SV_FJ], qb0[SV_FJ], qb1[SV_FJ];
  int64_t r = rb + 2 * wave;
  load(r, qa0);
  load(r + 1, qa1);
  for (; r < re; r += 16) {   // uniform per wave
    load(r + 8, qb0);
    load(r + 9, qb1);
    process(r, qa0, qa1);
    load(r + 16, qa0);
    load(r + 17, qa1);
    process(r + 8, qb0, qb1);
  }
  // Column sums of the four waves, added in wave order.
#pragma unroll
  for (int j = 0; j < SV_FJ; ++j)
#pragma unroll
    for (int e = 0; e < V; e += 4)
      reinterpret_cast<float4*>(cs[wave])[((64 * j + lane) * V + e) >> 2] =
          float4{cp[j][e], cp[j][e + 1], cp[j][e + 2], cp[j][e + 3]};
  if (lane == 0) usw[wave] = usq;
  __syncthreads();
  for (int k = tid; k < K; k += 256)
    part[(int64_t)blockIdx.x * K + k] = ((cs[0][k] + cs[1][k]) + cs[2][k]) + cs[3][k];
  if (tid == 0) upart[blockIdx.x] = ((usw[0] + usw[1]) + usw[2]) + usw[3];
}

// ---------------------------------------------------------------- column reduction
// v[k] = Σ_c part[c][k] / ||u||, ||u||^2 = Σ_b upart[b].  Workgroup = SV_RCOLS
// columns: thread (l, q) sums chunks l, l + SV_CLANES, ... of columns
// 4q..4q+3; the SV_CLANES lane sums are then added in lane order.
__global__ __launch_bounds__(256) void svid_vreduce_kernel(const float* __restrict__ part, int64_t chunks,
                                                           int64_t K, const float* __restrict__ upart,
                                                           int64_t nub, float* __restrict__ v) {
  __shared__ float ps[SV_CLANES][SV_RCOLS + 1];
  __shared__ float red[4];
  const int tid = threadIdx.x, q = tid % (SV_RCOLS / 4), l = tid / (SV_RCOLS / 4);
  const int64_t k = (int64_t)blockIdx.x * SV_RCOLS + 4 * q;
  const float unorm = sqrtf(block_total<false>(upart, nub, red));
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int64_t kc = k < K ? k : K - 4;                  // K % 4 == 0
  for (int64_t c0 = l; c0 < chunks; c0 += 8 * SV_CLANES) {
    float4 p[8];
    bool ok[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t cr = c0 + (int64_t)r * SV_CLANES;
      ok[r] = cr < chunks;
      p[r] = *reinterpret_cast<const float4*>(part + (ok[r] ? cr : 0) * K + kc);   // chunk 0 always exists
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      acc[0] += ok[r] ? p[r].x : 0.f;
      acc[1] += ok[r] ? p[r].y : 0.f;
      acc[2] += ok[r] ? p[r].z : 0.f;
      acc[3] += ok[r] ? p[r].w : 0.f;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) ps[l][4 * q + e] = acc[e];
  __syncthreads();
  if (tid < SV_RCOLS) {
    const int64_t col = (int64_t)blockIdx.x * SV_RCOLS + tid;
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < SV_CLANES; ++r) s += ps[r][tid];
    if (col < K) v[col] = s / unorm;
  }
}

__global__ __launch_bounds__(256) void svid_init_kernel(float* __restrict__ v, int64_t K) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < K) v[k] = 1.f;
}

// a = u / sqrt(σ), b = sqrt(σ) v / ||v||, σ^2 = Σ upart (u is |W| v / ||v||).
template <typename ST>
__global__ __launch_bounds__(256) void svid_final_kernel(const float* __restrict__ u, int64_t N,
                                                         const float* __restrict__ v, int64_t K,
                                                         const float* __restrict__ upart, int64_t nub,
                                                         ST* __restrict__ a, ST* __restrict__ b) {
  __shared__ float red[2][4];
  const float sigma = sqrtf(block_total<false>(upart, nub, red[0]));
  const float vnorm = sqrtf(block_total<true>(v, K, red[1]));
  const float root = sqrtf(sigma);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < N) Store<ST>::put(&a[i], u[i] / root);
  if (i < K) Store<ST>::put(&b[i], root * (v[i] / vnorm));
}

struct Layout {
  int64_t chunks, nub;
  float *part, *v, *u, *upart;
};

// Fused pass: rows per workgroup, so that the grid is one workgroup per CU
// (256 on MI355X) and its partial rows stay small (K floats each).
constexpr int64_t SV_FUSED_BLOCKS = 256;
inline int64_t fused_rpw(int64_t N) {
  const int64_t r = (N + SV_FUSED_BLOCKS - 1) / SV_FUSED_BLOCKS;
  return r < SV_RPB ? SV_RPB : r;
}
inline int64_t part_rows(int64_t N) {   // partial rows of the column pass or of the fused pass
  const int64_t c = (N + SV_CHUNK - 1) / SV_CHUNK, f = (N + fused_rpw(N) - 1) / fused_rpw(N);
  return c > f ? c : f;
}

// Workspace: part [part_rows][K] first (16-byte aligned rows, K % 4 == 0), then
// v [K], u [N], upart [nub], then slack (the fused pass's sink slot).
Layout layout(float* ws, int64_t N, int64_t K) {
  Layout L;
  L.chunks = (N + SV_CHUNK - 1) / SV_CHUNK;
  L.nub = (N + SV_RPB - 1) / SV_RPB;
  L.part = ws;
  L.v = L.part + part_rows(N) * K;
  L.u = L.v + K;
  L.upart = L.u + N;
  return L;
}

template <typename WT, typename ST, int V, int CV>
hipError_t run(const WT* W, int64_t N, int64_t K, int iters, void* av, void* bv, float* ws, hipStream_t st) {
  const Layout L = layout(ws, N, K);
  const dim3 gr((unsigned)L.nub);
  const dim3 gc((unsigned)((K / CV + 255) / 256), (unsigned)L.chunks);
  const dim3 gv((unsigned)((K + SV_RCOLS - 1) / SV_RCOLS));
  hipLaunchKernelGGL(svid_init_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, L.v, K);
  // Rows of at most 512·V elements (16-byte loads) take the fused pass: one
  // read of W per iteration instead of two.
  const bool fused = V > 1 && K <= 64 * SV_FJ * V;
  const int64_t rpw = fused_rpw(N), nf = (N + rpw - 1) / rpw;
  for (int it = 0; it < iters; ++it) {
    if constexpr (V > 1) {
      if (fused) {
        hipLaunchKernelGGL((svid_fused_kernel<WT, V>), dim3((unsigned)nf), dim3(256), 0, st, W, N, K, rpw, L.v, L.u,
                           L.upart, L.part, L.upart + L.nub);
        hipLaunchKernelGGL(svid_vreduce_kernel, gv, dim3(256), 0, st, L.part, nf, K, L.upart, nf, L.v);
        continue;
      }
    }
    hipLaunchKernelGGL((svid_rows_kernel<WT, V>), gr, dim3(256), 0, st, W, N, K, L.v, L.u, L.upart);
    hipLaunchKernelGGL((svid_cols_kernel<WT, CV>), gc, dim3(256), 0, st, W, N, K, L.u, L.part);
    hipLaunchKernelGGL(svid_vreduce_kernel, gv, dim3(256), 0, st, L.part, L.chunks, K, L.upart, L.nub, L.v);
  }
  hipLaunchKernelGGL((svid_rows_kernel<WT, V>), gr, dim3(256), 0, st, W, N, K, L.v, L.u, L.upart);
  const int64_t nmax = N > K ? N : K;
  hipLaunchKernelGGL((svid_final_kernel<ST>), dim3((unsigned)((nmax + 255) / 256)), dim3(256), 0, st, L.u, N,
                     L.v, K, L.upart, L.nub, static_cast<ST*>(av), static_cast<ST*>(bv));
  return hipGetLastError();
}

template <typename WT, typename ST>
hipError_t run_v(const void* Wv, int64_t N, int64_t K, int iters, void* a, void* b, float* ws, hipStream_t st) {
  const WT* W = static_cast<const WT*>(Wv);
  // Vector loads need a 16-byte aligned base (rows are K · sizeof(WT) bytes,
  // a multiple of 64 since K % 32 == 0).
  constexpr int V = 16 / sizeof(WT);
  if (reinterpret_cast<uintptr_t>(Wv) % 16 == 0) return run<WT, ST, V, SV_CPT>(W, N, K, iters, a, b, ws, st);
  return run<WT, ST, 1, 1>(W, N, K, iters, a, b, ws, st);
}

template <typename WT>
hipError_t run_s(int scale_dtype, const void* W, int64_t N, int64_t K, int iters, void* a, void* b, float* ws,
                 hipStream_t st) {
  return scale_dtype == DT_F32 ? run_v<WT, float>(W, N, K, iters, a, b, ws, st)
                               : run_v<WT, f16_t>(W, N, K, iters, a, b, ws, st);
}

}  // namespace

size_t svid_workspace_floats(int64_t N, int64_t K) {
  const int64_t nub = (N + SV_RPB - 1) / SV_RPB;
  return (size_t)(part_rows(N) * K + K + N + nub + 64);
}

hipError_t launch_svid(const void* W, int w_dtype, int64_t N, int64_t K, int iters, void* a, void* b,
                       int scale_dtype, float* ws, hipStream_t st) {
  if ((N + SV_RPB - 1) / SV_RPB > 0x7fffffff || (N + SV_CHUNK - 1) / SV_CHUNK > 65535) return hipErrorInvalidValue;
  if (w_dtype == DT_F32) return run_s<float>(scale_dtype, W, N, K, iters, a, b, ws, st);
  if (w_dtype == DT_F16) return run_s<f16_t>(scale_dtype, W, N, K, iters, a, b, ws, st);
  return run_s<bf16_t>(scale_dtype, W, N, K, iters, a, b, ws, st);
}

}  // namespace obl
