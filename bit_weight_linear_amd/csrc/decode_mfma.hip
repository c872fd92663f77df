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
// The sign operand is expanded in registers from the packed words.
//
// Two kernels share the contraction below.  The whole-K kernel (further down)
// serves bf16 x with fp16 b and aligned operands in one launch: a workgroup
// owns a column block over all of K and adds its waves' slice sums in LDS.
// The split kernel serves everything else (fp32 x or b, misaligned operands).
//
// Split kernel work split: block = 4 waves x 16 columns (64 output columns) x
// one K-slice of 512 k, so each block reads only its slice of X.  With one slice the
// block applies the post scale and writes Y; otherwise slices write fp32
// partial sums to scratch and a second small kernel adds them in slice order
// (the kernel boundary orders the memory traffic; no fences, no atomics), so
// results are bitwise reproducible.  (Counting the slices in and letting the
// last one reduce needs system-coherent stores, atomics and loads across the
// XCDs, three memory round trips, and measured slower than the second launch.)
//
// Staging (all in LDS, one barrier):
//  * the X slice (bf16 modes: by DMA, global_load_lds_dwordx4, 1 KiB per
//    instruction, coalesced rows), natural k order, 16-byte chunk c of row r at slot
//    c ^ (r % 16): an A fragment -- lane (row m = lane % 16, quarter g =
//    lane / 16) takes x[m][32t + 8g .. +7] -- is one conflict-free
//    ds_read_b128;
//  * the 64 columns' sign words with one 16-byte load per thread, transposed
//    into [step][column] (stride 65 words) so a wave's 16 columns of one step
//    are 16 consecutive banks;
//  * mode B2: the slice's (b_hi, b_lo) bf16 pair tables; mode S3: the three
//    bf16 terms of x·b, split once per block (the four waves share them).
// Sign expansion in natural k order: dword r of quarter g pairs k = 32t + 8g +
// 2r and k + 1, whose sign bits sit side by side in half g / 2 of word t; one
// packed 16-bit shift (v_pk_lshlrev_b16, both halves fed from that half) puts
// them at bits 15 and 31 and one v_bitop3 applies them to the magnitudes.
// The contraction takes four steps at a time: all LDS reads of the four are
// issued before the first MFMA and each step owns its accumulators.
#include <type_traits>

#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int DEC_THREADS = 256;
constexpr int DEC_BN = 64;      // output columns per block (16 per wave)
constexpr int DEC_STEPS = 16;   // 32-k steps per K-slice
constexpr int DEC_SK = DEC_STEPS * 32;          // k per slice
constexpr int DEC_WSTRIDE = DEC_BN + 1;         // words per step row of the sign table

enum DecMode { MODE_B2 = 0, MODE_B1 = 1, MODE_S3 = 2 };

// B operand of one step for quarter g: dword r takes bits p = 8(g & 1) + 2r and
// p + 1 of the 16-bit half g / 2 of the word (sh[r] = (15 - p, 14 - p)).
__device__ __forceinline__ u32x4 expand_nat(uint32_t word, int h, const u16x2* sh, u32x4 mag) {
  const uint32_t half = h ? (word >> 16) : (word & 0xFFFFu);
  const u16x2 d = u16x2{(unsigned short)half, (unsigned short)half};
  u32x4 r;
  r.x = (__builtin_bit_cast(uint32_t, d << sh[0]) & 0x80008000u) ^ mag.x;
  r.y = (__builtin_bit_cast(uint32_t, d << sh[1]) & 0x80008000u) ^ mag.y;
  r.z = (__builtin_bit_cast(uint32_t, d << sh[2]) & 0x80008000u) ^ mag.z;
  r.w = (__builtin_bit_cast(uint32_t, d << sh[3]) & 0x80008000u) ^ mag.w;
  return r;
}

// FAST: X and W 16-byte aligned and K % 128 == 0 (DMA / vector loads, one
// 16-byte sign load per thread); otherwise plain element loads.
template <int MODE, typename XT, typename ST, typename YT, bool PRE, bool FAST>
__global__ __launch_bounds__(DEC_THREADS) void decode_mfma_kernel(
    const XT* __restrict__ X, int M, int64_t K, const uint32_t* __restrict__ W, int64_t N,
    const ST* __restrict__ pre, const ST* __restrict__ post, YT* __restrict__ Y, int nslices,
    float* __restrict__ partials) {
  constexpr int TA = MODE == MODE_S3 ? 3 : 1;          // bf16 A term arrays
  constexpr int CPR = DEC_SK * 2 / 16;                 // 16-byte chunks (8 bf16) per row of a term array
  __shared__ u32x4 xs[TA][16 * CPR];
  __shared__ uint32_t ws[DEC_STEPS * DEC_WSTRIDE];
  __shared__ uint32_t ms[MODE == MODE_B2 ? DEC_SK : 1];   // B2: (b_hi) pairs then (b_lo) pairs

  const int tile = blockIdx.x / nslices;
  const int slice = blockIdx.x - tile * nslices;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15;
  const int g = lane >> 4;
  const int64_t kw = K >> 5;
  const int64_t step0 = (int64_t)slice * DEC_STEPS;
  const int64_t k0 = step0 * 32;
  const int nsteps = (int)min((int64_t)DEC_STEPS, kw - step0);
  const int64_t n0 = (int64_t)tile * DEC_BN;
  const int xslots = M * CPR;                          // slot q = (row q / CPR, slot q % CPR)

  // ---- 1. Raw bf16 X (modes B1, B2) by DMA: slot (r, s) receives chunk
  // s ^ (r % 16) of the row's slice; chunks past K re-read chunk 0 (never used).
  if constexpr (MODE != MODE_S3 && FAST) {
    const int rounds = (xslots + DEC_THREADS - 1) / DEC_THREADS;
    for (int i = 0; i < rounds; ++i) {
      const int base = (i * (DEC_THREADS / 64) + wave) * 64;
      const int q = min(base + lane, xslots - 1);
      const int r = q / CPR, sl = q - r * CPR;
      int64_t ke = k0 + 8 * (int64_t)(sl ^ (r & 15));
      if (ke >= K) ke = k0;
      load_lds16(X + (int64_t)r * K + ke, &xs[0][base]);
    }
  }
  // Mode S3: x and b of this thread's slots, loaded now and split after the
  // sign loads are issued.  Slots: q = tid + 256 i.
  constexpr int S3N = MODE == MODE_S3 ? (16 * CPR) / DEC_THREADS : 1;   // 4
  float xv[S3N][8];
  if constexpr (MODE == MODE_S3) {
#pragma unroll
    for (int i = 0; i < S3N; ++i) {
      const int q = tid + DEC_THREADS * i;
      const int r = q / CPR, sl = q - r * CPR;
      const int64_t ke = k0 + 8 * (int64_t)(sl ^ (r & 15));
      const bool ok = q < xslots && ke < K;
      const int64_t kc = ok ? ke : 0;
      const XT* xp = X + (ok ? (int64_t)r * K : 0) + kc;
      if constexpr (FAST && sizeof(XT) == 4) {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(xp), v1 = *reinterpret_cast<const f32x4*>(xp + 4);
        xv[i][0] = v0.x; xv[i][1] = v0.y; xv[i][2] = v0.z; xv[i][3] = v0.w;
        xv[i][4] = v1.x; xv[i][5] = v1.y; xv[i][6] = v1.z; xv[i][7] = v1.w;
      } else if constexpr (FAST) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(xp);
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[i][2 * e] = __uint_as_float(d[e] << 16);
          xv[i][2 * e + 1] = __uint_as_float(d[e] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[i][e] = to_f32(xp[e]);
      }
      if constexpr (PRE) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[i][e] *= to_f32(pre[kc + e]);
      }
      if (!ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[i][e] = 0.f;
      }
    }
  }
  // ---- 2. Sign words: thread -> (column tid / 4, quad tid % 4 of the slice).
  u32x4 wq;
  {
    const int col = tid >> 2, quad = tid & 3;
    const int64_t n = min(n0 + col, N - 1);
    const uint32_t* src = W + n * kw + step0;
    if constexpr (FAST) {
      const int qq = 4 * quad < nsteps ? 4 * quad : 0;
      wq = *reinterpret_cast<const u32x4*>(src + qq);
    } else {
      uint32_t t4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int st = 4 * quad + e;
        t4[e] = src[st < nsteps ? st : 0];
      }
      wq = u32x4{t4[0], t4[1], t4[2], t4[3]};
    }
  }
  // ---- 3. Mode B2: the slice's b, thread -> k pair (2 tid, 2 tid + 1).
  float b0 = 0.f, b1 = 0.f;
  if constexpr (MODE == MODE_B2) {
    const int64_t k = k0 + 2 * tid;
    const int64_t kc = k < K ? k : 0;
    b0 = to_f32(pre[kc]);
    b1 = to_f32(pre[kc + 1]);
    if (k >= K) b0 = b1 = 0.f;
  }
  const float post_c = scale_or_one(post, min(n0 + 16 * wave + j, N - 1), W);   // W: >= 4N bytes

  // ---- 4. Remaining LDS writes, then one barrier.
  if constexpr (MODE != MODE_S3 && !FAST) {
    // Element loads into the same swizzled slots (any alignment).
    for (int q = tid; q < xslots; q += DEC_THREADS) {
      const int r = q / CPR, sl = q - r * CPR;
      const int64_t ke = k0 + 8 * (int64_t)(sl ^ (r & 15));
      const uint16_t* xr = reinterpret_cast<const uint16_t*>(X) + (int64_t)r * K;
      uint32_t d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t k = ke + 2 * e;
        d[e] = k < K ? (uint32_t(xr[k]) | (uint32_t(xr[k + 1]) << 16)) : 0u;
      }
      xs[0][q] = u32x4{d[0], d[1], d[2], d[3]};
    }
  }
  if constexpr (MODE == MODE_S3) {
    // x' = x·b split exactly into three bf16 terms (24 significant bits).
#pragma unroll
    for (int i = 0; i < S3N; ++i) {
      const int q = tid + DEC_THREADS * i;
      uint32_t th[4], tm[4], tl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const Split3 s0 = split3(xv[i][2 * e]), s1 = split3(xv[i][2 * e + 1]);
        th[e] = pack_bf16_pair(s0.hi, s1.hi);
        tm[e] = pack_bf16_pair(s0.mid, s1.mid);
        tl[e] = pack_bf16_pair(s0.lo, s1.lo);
      }
      if (q < xslots) {
        xs[0][q] = u32x4{th[0], th[1], th[2], th[3]};
        xs[TA > 1 ? 1 : 0][q] = u32x4{tm[0], tm[1], tm[2], tm[3]};
        xs[TA > 2 ? 2 : 0][q] = u32x4{tl[0], tl[1], tl[2], tl[3]};
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): every load of this thread landed
  {
    const int col = tid >> 2, quad = tid & 3;
    uint32_t* d = ws + (4 * quad) * DEC_WSTRIDE + col;
    const bool ok = 4 * quad < nsteps;
    d[0] = ok ? wq.x : 0u;
    d[DEC_WSTRIDE] = ok ? wq.y : 0u;
    d[2 * DEC_WSTRIDE] = ok ? wq.z : 0u;
    d[3 * DEC_WSTRIDE] = ok ? wq.w : 0u;
  }
  if constexpr (MODE == MODE_B2) {
    const float h0 = bf16_round(b0), h1 = bf16_round(b1);
    ms[tid] = pack_bf16_pair(h0, h1);
    ms[DEC_SK / 2 + tid] = pack_bf16_pair(b0 - h0, b1 - h1);   // exact: an fp16 residual fits bf16
  }
  __syncthreads();

  // ---- 5. Contraction: this wave's 16 columns over the slice, four steps at
  // a time (every LDS read of the four before the first MFMA; each step owns
  // its accumulators).
  u16x2 sh[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = 8 * (g & 1) + 2 * r;
    sh[r] = u16x2{(unsigned short)(15 - p), (unsigned short)(14 - p)};
  }
  const int h = g >> 1;
  const bool mrow = j < M;
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  const int xrow = (mrow ? j : 0) * CPR;
  const int swz = j & 15;
  const int wcol = 16 * wave + j;
  constexpr int NA = MODE == MODE_B1 ? 1 : 2;

  f32x4 acc[4][NA];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[u][a] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int t = 0; t < DEC_STEPS; t += 4) {
    uint32_t word[4];
    u32x4 xf[4][TA], mh[4], ml[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      word[u] = ws[(t + u) * DEC_WSTRIDE + wcol];
      const int kb = 32 * (t + u) + 8 * g;             // first k of this lane's quarter
#pragma unroll
      for (int ta = 0; ta < TA; ++ta) xf[u][ta] = xs[ta][xrow + ((kb / 8) ^ swz)];
      if constexpr (MODE == MODE_B2) {
        mh[u] = *reinterpret_cast<const u32x4*>(ms + kb / 2);
        ml[u] = *reinterpret_cast<const u32x4*>(ms + DEC_SK / 2 + kb / 2);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = mrow && (t + u < nsteps);
      if constexpr (MODE == MODE_B2) {
        const u32x4 a = ok ? xf[u][0] : zero4;
        acc[u][0] = mfma16x16x32(a, expand_nat(word[u], h, sh, mh[u]), acc[u][0]);
        acc[u][1] = mfma16x16x32(a, expand_nat(word[u], h, sh, ml[u]), acc[u][1]);
      } else if constexpr (MODE == MODE_B1) {
        const u32x4 a = ok ? xf[u][0] : zero4;
        acc[u][0] = mfma16x16x32(a, expand_nat(word[u], h, sh, ones), acc[u][0]);
      } else {
        const u32x4 bsg = expand_nat(word[u], h, sh, ones);
        acc[u][0] = mfma16x16x32(ok ? xf[u][0] : zero4, bsg, acc[u][0]);
        acc[u][1] = mfma16x16x32(ok ? xf[u][1] : zero4, bsg, acc[u][1]);
        acc[u][0] = mfma16x16x32(ok ? xf[u][2] : zero4, bsg, acc[u][0]);
      }
    }
  }
  // Fixed summation order: terms of a step, then steps in order.
  f32x4 tot = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    f32x4 su = acc[u][0];
#pragma unroll
    for (int a = 1; a < NA; ++a) su = su + acc[u][a];
    tot = tot + su;
  }

  // ---- 6. Output: lane holds rows 4g .. 4g+3 of column n0 + wcol.
  const int64_t col = n0 + wcol;
  if (nslices == 1) {
    if (col < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < M) Store<YT>::put(&Y[(int64_t)m * N + col], tot[i] * post_c);
      }
    }
    return;
  }
  if (col < N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < M) partials[((int64_t)slice * M + m) * N + col] = tot[i];
    }
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
  const float s = scale_or_one(post, n, partials);   // partials: >= MN floats
  // Slices in batches of 8 (clamped indexes, masked terms): every load of a
  // batch is in flight together, also for slice counts that are not a multiple
  // of 8 (a plain tail loop would wait once per slice).
  // The slices' sums in slice order: plainly up to 8 slices (K <= 4096, the
  // whole-K kernel's cross-wave order), beyond that with compensated (Kahan)
  // summation, so the error stays that of one slice plus a few roundings
  // however many slices K spans.
  float acc = 0.f, comp = 0.f;
  const bool kahan = nslices > 8;   // uniform over the grid
  for (int s0 = 0; s0 < nslices; s0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partials[(int64_t)(s0 + u < nslices ? s0 + u : 0) * MN + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u < nslices) {   // uniform over the grid
        if (kahan) {
          const float y = v[u] - comp;
          const float t = acc + y;
          comp = (t - acc) - y;
          acc = t;
        } else {
          acc += v[u];
        }
      }
    }
  }
  Store<YT>::put(&Y[e], acc * s);
}

// ---------------------------------------------------------------------------
// Whole-K variant (bf16 x and fp16 b, mode B2; 16-byte aligned X, W and b,
// K % 128 == 0; up to 32 rows).  A workgroup of 8 waves (4 for 17..32 rows,
// whose X slices take twice the LDS) owns 16·CPW output columns over all of
// K; wave w takes the 512-k slices w, w + W, ... of them (W waves).  Rows come
// in fragments of 16 (one MFMA A operand each): a 32-row call contracts two
// fragments against every expanded sign operand.  Per slice the
// wave copies into its own LDS region, by DMA and in this order: the slice's
// sign words of its columns, the slice's b, and its M rows of X by k-quarter
// (128 k); it then contracts quarter q as soon as quarters <= q have landed,
// so the contraction overlaps the rest of the copy.  No workgroup barrier is
// needed until the end, where the per-wave sums of each output are added in
// wave order through LDS and the post scale applied.  One launch,
// and no partial sums through HBM: the split-K kernel needs a second launch
// for its slice reduction, which must wait for the first.  The price is that
// every workgroup reads all of X (M·K·2 bytes through its CU).  With one
// column group per wave and K <= 4096 (one slice per wave) the sums are added
// in exactly the split kernel's order: both give bitwise the same results.
//
// Every transfer of the slice is an LDS DMA, waited for with explicit vmcnt
// counts: a load into registers issued before the DMAs is waited for with
// vmcnt(0) at its first use (the compiler's count of transfers in flight
// does not include LDS DMAs), which would serialise the copy and the
// contraction.  Only where the sign words do not fit in LDS next to the rows
// of X (CPW = 4 with M > 8) are they loaded into registers, at that cost.
constexpr size_t WK_LDS_MAX = 160 * 1024;
constexpr size_t WK_LDS_UNITS = WK_LDS_MAX / 16;

// Input modes: WK_B2, bf16 x with fp16 b (mode B2 above); WK_T3, three bf16
// arrays [3][M][K] whose sum is an fp32 input exactly (hi + mid + lo, written
// by a previous whole-K call as its output's terms), no b: A = each term,
// B = ±1, three MFMAs per step.  A DBF decode runs stage 1 in WK_B2 writing
// the terms of T1 and stage 2 in WK_T3 reading them, each in one launch.
enum WkMode { WK_B2 = 0, WK_T3 = 1 };

// LDS of one wave, in 16-byte units: X as TT term arrays (TT = 1, or 3 for
// WK_T3), each four k-quarters of [4·PER rows][16 chunks] (PER = DMAs of 4
// rows per quarter, a template constant so the waits are immediates); WK_B2:
// 64 b_hi pair quads and 64 b_lo pair quads (the raw fp16 b of the slice
// lands in the b_lo area first); then, when they fit, the sign words as
// [CPW][quarter][16 columns].  After the contraction the area holds the
// reduction table.  Waves per workgroup: 8, or 4 for 17..32 rows (WK_B2);
// WK_T3 as many as fit, at most 8 (6 for 8 rows).
__host__ __device__ constexpr size_t wk_wave_units_nosigns(int xm, int per) {
  return xm == WK_T3 ? (size_t)per * 768 : (size_t)per * 256 + 128;
}
__host__ __device__ constexpr int wk_waves(int xm, int per, int cpw) {
  return xm == WK_B2 ? (per == 8 ? 4 : 8)
                     : (int)(WK_LDS_UNITS / (wk_wave_units_nosigns(xm, per) + 64 * (size_t)cpw) < 8
                                 ? WK_LDS_UNITS / (wk_wave_units_nosigns(xm, per) + 64 * (size_t)cpw)
                                 : 8);
}
__host__ __device__ constexpr bool wk_signs_in_lds(int xm, int per, int cpw) {
  return (size_t)wk_waves(xm, per, cpw) * (wk_wave_units_nosigns(xm, per) + 64 * (size_t)cpw) <= WK_LDS_UNITS;
}
__host__ __device__ constexpr size_t wk_wave_units(int xm, int per, int cpw) {
  return wk_wave_units_nosigns(xm, per) + (wk_signs_in_lds(xm, per, cpw) ? 64 * (size_t)cpw : 0);
}
inline int wk_per(int64_t M) { return M <= 4 ? 1 : (M <= 8 ? 2 : (M <= 16 ? 4 : 8)); }
inline size_t wk_lds_bytes(int xm, int per, int cpw) {
  const size_t waves = (size_t)wk_waves(xm, per, cpw);
  const size_t stage = waves * wk_wave_units(xm, per, cpw) * 16;
  const size_t rows = (size_t)(4 * per + 15) / 16 * 16;
  const size_t red = (waves * rows * (16 * cpw + 1) + rows * 16 * cpw) * sizeof(float);   // + gradient products
  return stage > red ? stage : red;
}

// Wait until at most N of this wave's vector-memory transfers are in flight.
template <int N>
__device__ __forceinline__ void wk_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | ((N >> 4) << 14));
}

// Order this wave's LDS writes before its later LDS reads (only this wave
// touches its region: no workgroup barrier).
__device__ __forceinline__ void wk_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Optional epilogue outputs (null when unused).  T3 (fp32 Y only): the
// output's exact bf16 terms, [3][M][N].  Gradient epilogue of the layer's
// backward (bf16 gin): gsum[n] = Σ_m gin[m][n] · y[m][n] over the block's
// rows in order, and, with gout, gout[m][n] = y[m][n] · gscale[n] (fp32 or
// bf16 as gout_bf16 says).
// The body of one workgroup: `bx` is its block index within its problem and
// wk_lds the workgroup's dynamic LDS.
template <int XM, typename ST, typename YT, int CPW, int PER, bool NT, bool MS>
__device__ __forceinline__ void decode_wk_body(
    u32x4* wk_lds, unsigned bx,
    const bf16_t* __restrict__ X, int M, int64_t K, const uint32_t* __restrict__ W, int64_t N,
    const f16_t* __restrict__ pre, const ST* __restrict__ post, YT* __restrict__ Y, bf16_t* __restrict__ T3,
    const bf16_t* __restrict__ gin, float* __restrict__ gsum, const ST* __restrict__ gscale,
    void* __restrict__ gout, int gout_bf16) {
  constexpr bool B2 = XM == WK_B2;
  constexpr int TT = B2 ? 1 : 3;                                  // A term arrays
  constexpr int NA = B2 ? 2 : 3;                                  // accumulators per set
  constexpr int WAVES = wk_waves(XM, PER, CPW);
  constexpr int THREADS = 64 * WAVES;
  constexpr int NC = 16 * CPW;                                    // columns per workgroup
  constexpr int RS = NC + 1;                                      // reduction table row stride (floats)
  constexpr int M4 = 4 * PER;                                     // X rows staged (>= M)
  constexpr int TS = 4 * M4 * 16;                                 // units per term array
  constexpr int RF = (M4 + 15) / 16;                              // 16-row fragments
  constexpr int NOUT = (16 * RF * NC + THREADS - 1) / THREADS;    // final outputs per thread
  constexpr bool SL = wk_signs_in_lds(XM, PER, CPW);              // sign words by DMA into LDS
  constexpr int XD = TT * PER;                                    // X DMAs per k-quarter

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15;
  const int g = lane >> 4;
  const int64_t kw = K >> 5;
  const int nslices = (int)((kw + DEC_STEPS - 1) / DEC_STEPS);
  const int64_t n0 = (int64_t)bx * NC;
  u32x4* xw = wk_lds + (size_t)wave * wk_wave_units(XM, PER, CPW);   // X terms and quarters
  u32x4* mq = xw + TT * TS;                                       // WK_B2: b_hi quads [64], b_lo quads [64]
  uint32_t* mw = reinterpret_cast<uint32_t*>(mq);
  u32x4* sg = mq + (B2 ? 128 : 0);                                // sign quads [CPW][4][16] (SL)
  // Buffer resources: offsets past the end of X, W or b read zeros, so the
  // DMAs need no clamping (what they read past the last slice's K is masked).
  // Byte offsets fit in 32 bits (checked by the launcher).
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)(TT * M * K * 2));
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W, (uint32_t)(N * kw * 4));
  const __amdgpu_buffer_rsrc_t br = make_rsrc(B2 ? (const void*)pre : (const void*)W, B2 ? (uint32_t)(K * 2) : 0u);
  // Per-lane DMA offsets, fixed over the slices: X row group i (row 4i +
  // lane / 16, chunk (lane % 16) ^ (row % 16) of a quarter), sign quad lane / 16
  // of column 16c + lane % 16, b chunk lane.
  uint32_t xo[PER], so[SL ? CPW : 1];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int row = 4 * i + (lane >> 4);
    xo[i] = (uint32_t)((min(row, M - 1) * K + 8 * ((lane & 15) ^ (row & 15))) * 2);
  }
#pragma unroll
  for (int c = 0; c < (SL ? CPW : 1); ++c)
    so[c] = (uint32_t)((min(n0 + 16 * c + j, N - 1) * kw + 4 * (lane >> 4)) * 4);

  // Output scales of this thread's final outputs (o = tid + THREADS r is
  // row o / NC, column o % NC), issued before the streams.
  float post_o[NOUT];
#pragma unroll
  for (int r = 0; r < NOUT; ++r)
    post_o[r] = scale_or_one(post, min(n0 + (tid + THREADS * r) % NC, N - 1), W);   // W: >= 4N bytes
  // Gradient epilogue inputs of the same outputs: unconditional loads
  // (clamped indexes; without gin, element 0 of W stands in and is unused).
  float gin_o[NOUT], gsc_o[NOUT];
  const bf16_t* gsrc = gin ? gin : reinterpret_cast<const bf16_t*>(W);
#pragma unroll
  for (int r = 0; r < NOUT; ++r) {
    const int o = tid + THREADS * r;
    const int64_t mm = min(o / NC, M - 1), nn = min(n0 + o % NC, N - 1);
    gin_o[r] = to_f32(gsrc[gin ? mm * N + nn : 0]);
    gsc_o[r] = scale_or_one(gscale, nn, W);
  }

  u16x2 sh[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = 8 * (g & 1) + 2 * r;
    sh[r] = u16x2{(unsigned short)(15 - p), (unsigned short)(14 - p)};
  }
  const int h = g >> 1;
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  bool mrow[RF];                                                  // row 16f + j of fragment f exists
  int xrow[RF];
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    mrow[f] = 16 * f + j < M;
    xrow[f] = (mrow[f] ? 16 * f + j : 0) * 16;
  }
  const int swz = j & 15;

  // Accumulator sets: step t adds into set t % AU.  With one column group
  // each of four consecutive steps owns a set (the split kernel's order);
  // with more, the column groups already give the MFMAs enough independent
  // chains and fewer sets keep the registers within two waves per SIMD.
  constexpr int AU = CPW == 1 ? 4 : (CPW == 2 ? 2 : 1);
  f32x4 acc[AU][CPW][RF][NA];
#pragma unroll
  for (int u = 0; u < AU; ++u)
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int f = 0; f < RF; ++f)
#pragma unroll
        for (int a = 0; a < NA; ++a) acc[u][c][f][a] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MS (K spans more slices than the workgroup has waves): a wave's slices
  // are summed one slice at a time (terms of a set, then the sets in order)
  // and each slice's sum is added into a running total with compensated
  // (Kahan) summation, so a lane's rounding error is that of one slice plus
  // about two roundings however long K is.  Without MS every wave has at most
  // one slice and the fold below never runs (an instance of its own: the
  // running total's registers and the fold measured 0.3 us slower at
  // 16 x 4096 x 4096 even unused).
  f32x4 ktot[MS ? CPW : 1][MS ? RF : 1], kcomp[MS ? CPW : 1][MS ? RF : 1];
  if constexpr (MS) {
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int f = 0; f < RF; ++f) ktot[c][f] = kcomp[c][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto fold_slice = [&]() {
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int f = 0; f < RF; ++f) {
        f32x4 sl = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < AU; ++u) {
          f32x4 su = acc[u][c][f][0];
#pragma unroll
          for (int a = 1; a < NA; ++a) su = su + acc[u][c][f][a];
          sl = sl + su;
#pragma unroll
          for (int a = 0; a < NA; ++a) acc[u][c][f][a] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if constexpr (MS) {
          const f32x4 y = sl - kcomp[c][f];
          const f32x4 t = ktot[c][f] + y;
          kcomp[c][f] = (t - ktot[c][f]) - y;
          ktot[c][f] = t;
        }
      }
  };

  for (int s = wave; s < nslices; s += WAVES) {
    if constexpr (MS) {
      if (s != wave) fold_slice();   // uniform: the previous slice's sums into the total
    }
    const int64_t step0 = (int64_t)s * DEC_STEPS;
    const int64_t k0 = step0 * 32;
    const int nsteps = (int)min((int64_t)DEC_STEPS, kw - step0);   // a multiple of 4
    // Sign words of the slice: quad q (steps 4q .. 4q+3) of column 16c + i.
    // SL: DMA c, lane l -> quad l / 16 of column l % 16, at sg[c][l / 16][l % 16];
    // otherwise the four lanes of a column load all four quads.  Quads past
    // the end re-read quad 0 (masked below).
    u32x4 wq[SL ? 1 : CPW][4];
    if constexpr (SL && PER <= 4 && NT) {
      // Up to 16 rows: the sign words marked non-temporal, which keeps the X
      // rows that every workgroup reads in L2.  Measured both ways: 16 x 4096
      // x 4096 5.67 -> 5.43 us, 4 x 4096 x 4096 5.15 -> 4.80, DBF decode 11.0
      // -> 10.7; 32 rows (and the register-staged signs below) measured 1-3 %
      // slower with it.  The choice is by template: a branch around the DMAs
      // made the compiler wait for every transfer at its join.  NT = false
      // for the backward's contractions (gradient epilogue): they follow the
      // forward over the same weights, which plain loads may find cached.
#pragma unroll
      for (int c = 0; c < CPW; ++c) dma16_nt(wr, sg + 64 * c, so[c], (uint32_t)(step0 * 4));
    } else if constexpr (SL) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) dma16(wr, sg + 64 * c, so[c], (uint32_t)(step0 * 4));
    } else {
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const uint32_t* src = W + min(n0 + 16 * c + j, N - 1) * kw + step0;
#pragma unroll
        for (int q = 0; q < 4; ++q) wq[c][q] = *reinterpret_cast<const u32x4*>(src + (4 * q < nsteps ? 4 * q : 0));
      }
    }
    // The waits below count transfers in issue order: scheduling barriers
    // keep the compiler from reordering the groups.
    __builtin_amdgcn_sched_barrier(0);
    // WK_B2: b of the slice, raw fp16, lane l -> k0 + 8l .. +7 into the b_lo
    // area (chunks past K read zeros or the next values; masked when converted).
    if constexpr (B2) dma16(br, mq + 64, (uint32_t)(16 * lane), (uint32_t)(k0 * 2));
    __builtin_amdgcn_sched_barrier(0);
    // X quarter q (k0 + 128q .. +127) of term array tt: DMA i writes rows 4i ..
    // 4i+3, lane l -> row 4i + l/16, slot l % 16 = chunk (l % 16) ^ (row % 16)
    // of the quarter.  Rows past M re-read row M - 1 (never used).
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < PER; ++i)
          dma16(xr, xw + tt * TS + (q * M4 + 4 * i) * 16, xo[i], (uint32_t)((tt * M * K + k0 + 128 * q) * 2));
      __builtin_amdgcn_sched_barrier(0);
    }
    wk_wait_vm<3 * XD>();   // signs, b and quarter 0 landed
    wk_wave_sync();
    if constexpr (B2) {
      // b pairs -> (b_hi, b_lo) tables: dword p = lane + 64 i holds k0 + 2p and
      // k0 + 2p + 1; every lane reads its four raw dwords before writing.
      uint32_t raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = mw[256 + lane + 64 * i];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = lane + 64 * i;
        const bool in = k0 + 2 * p < K;
        const float b0 = in ? to_f32(f16_t{(uint16_t)(raw[i] & 0xFFFFu)}) : 0.f;
        const float b1 = in ? to_f32(f16_t{(uint16_t)(raw[i] >> 16)}) : 0.f;
        const float h0 = bf16_round(b0), h1 = bf16_round(b1);
        mw[p] = pack_bf16_pair(h0, h1);
        mw[256 + p] = pack_bf16_pair(b0 - h0, b1 - h1);   // exact (fp16 residual)
      }
      wk_wave_sync();
    }

#pragma unroll
    for (int t = 0; t < DEC_STEPS; t += 4) {
      // Quarter t / 4: wait for its DMAs (the later quarters may still fly).
      if (t == 4) wk_wait_vm<2 * XD>();
      if (t == 8) wk_wait_vm<XD>();
      if (t == 12) wk_wait_vm<0>();
      if (t > 0) wk_wave_sync();
      u32x4 xf[4][RF][TT], mh[4], ml[4], wv[CPW];
#pragma unroll
      for (int c = 0; c < CPW; ++c) wv[c] = SL ? sg[(4 * c + t / 4) * 16 + j] : wq[SL ? 0 : c][t / 4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kb = 32 * (t + u) + 8 * g;
#pragma unroll
        for (int f = 0; f < RF; ++f)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) xf[u][f][tt] = xw[tt * TS + (t / 4) * M4 * 16 + xrow[f] + ((4 * u + g) ^ swz)];
        if constexpr (B2) {
          mh[u] = mq[kb / 8];
          ml[u] = mq[64 + kb / 8];
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // every LDS read of the quarter before its first MFMA
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool live = t + u < nsteps;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
          const uint32_t word = wv[c][u];
          if constexpr (B2) {
            const u32x4 bh = expand_nat(word, h, sh, mh[u]), bl = expand_nat(word, h, sh, ml[u]);
#pragma unroll
            for (int f = 0; f < RF; ++f) {
              const u32x4 a = (mrow[f] && live) ? xf[u][f][0] : zero4;
              f32x4* ac = acc[u % AU][c][f];
              ac[0] = mfma16x16x32(a, bh, ac[0]);
              ac[1] = mfma16x16x32(a, bl, ac[1]);
            }
          } else {
            const u32x4 bs = expand_nat(word, h, sh, ones);
#pragma unroll
            for (int f = 0; f < RF; ++f) {
              f32x4* ac = acc[u % AU][c][f];
#pragma unroll
              for (int tt = 0; tt < TT; ++tt)
                ac[tt] = mfma16x16x32((mrow[f] && live) ? xf[u][f][tt] : zero4, bs, ac[tt]);
            }
          }
        }
      }
    }
    wk_wave_sync();   // the next slice's DMAs overwrite this slice's LDS
  }

  // Fixed summation order: terms of a set, then the sets in order; with MS,
  // that sum of the last slice (or zeros) into the running total.
  f32x4 tot[CPW][RF];
  if constexpr (MS) {
    fold_slice();
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int f = 0; f < RF; ++f) tot[c][f] = ktot[c][f];
  } else {
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int f = 0; f < RF; ++f) {
        tot[c][f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < AU; ++u) {
          f32x4 su = acc[u][c][f][0];
#pragma unroll
          for (int a = 1; a < NA; ++a) su = su + acc[u][c][f][a];
          tot[c][f] = tot[c][f] + su;
        }
      }
  }
  // Waves' sums through LDS: red[wave][row][column]; lane holds rows
  // 16f + 4g .. +3 of column 16c + j.  Added in wave order.
  __syncthreads();   // every wave is done with its staging region
  float* red = reinterpret_cast<float*>(wk_lds);
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int f = 0; f < RF; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(wave * 16 * RF + 16 * f + 4 * g + i) * RS + 16 * c + j] = tot[c][f][i];
  __syncthreads();
  float* pg = red + WAVES * 16 * RF * RS;   // gradient products [16·RF rows][NC]
#pragma unroll
  for (int r = 0; r < NOUT; ++r) {
    const int o = tid + THREADS * r;
    const int m = o / NC, cl = o - (o / NC) * NC;
    if (o < 16 * RF * NC && m < M && n0 + cl < N) {
      // The waves' totals in wave order (at most 8 terms): with one slice
      // per wave this is the split kernel's slice reduction, term for term.
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) v += red[(w * 16 * RF + m) * RS + cl];
      const float y = v * post_o[r];
      const int64_t e = (int64_t)m * N + n0 + cl;
      Store<YT>::put(&Y[e], y);
      if (T3) {
        // Exact terms of the fp32 output for a following WK_T3 call.
        const Split3 sp = split3(y);
        Store<bf16_t>::put(&T3[e], sp.hi);
        Store<bf16_t>::put(&T3[(int64_t)M * N + e], sp.mid);
        Store<bf16_t>::put(&T3[2 * (int64_t)M * N + e], sp.lo);
      }
      if (gsum) pg[m * NC + cl] = gin_o[r] * y;
      if (gout) {
        const float d = y * gsc_o[r];
        if (gout_bf16) Store<bf16_t>::put(&static_cast<bf16_t*>(gout)[e], d);
        else static_cast<float*>(gout)[e] = d;
      }
    }
  }
  if (gsum) {   // uniform: every thread takes the same branch
    __syncthreads();
    if (tid < NC && n0 + tid < N) {
      float sum = 0.f;
      for (int m = 0; m < M; ++m) sum += pg[m * NC + tid];
      gsum[n0 + tid] = sum;
    }
  }
}

template <int XM, typename ST, typename YT, int CPW, int PER, bool NT, bool MS>
__global__ __launch_bounds__(64 * wk_waves(XM, PER, CPW)) void decode_wk_kernel(
    const bf16_t* __restrict__ X, int M, int64_t K, const uint32_t* __restrict__ W, int64_t N,
    const f16_t* __restrict__ pre, const ST* __restrict__ post, YT* __restrict__ Y, bf16_t* __restrict__ T3,
    const bf16_t* __restrict__ gin, float* __restrict__ gsum, const ST* __restrict__ gscale,
    void* __restrict__ gout, int gout_bf16) {
  extern __shared__ u32x4 wk_lds[];
  decode_wk_body<XM, ST, YT, CPW, PER, NT, MS>(wk_lds, blockIdx.x, X, M, K, W, N, pre, post, Y, T3, gin, gsum,
                                               gscale, gout, gout_bf16);
}

// The arguments of one whole-K problem (as decode_wk_kernel takes them).
template <typename ST, typename YT>
struct WkProb {
  const bf16_t* X;
  int M;
  int64_t K;
  const uint32_t* W;
  int64_t N;
  const f16_t* pre;
  const ST* post;
  YT* Y;
  bf16_t* T3;
  const bf16_t* gin;
  float* gsum;
  const ST* gscale;
  void* gout;
  int gout_bf16;
};

// Two problems of one kernel instance in one launch (the backward's two
// contractions): blocks [0, nb0) take p0, the others p1.  A workgroup's
// result does not depend on which launch it belongs to.
template <int XM, typename ST, typename YT, int CPW, int PER, bool NT, bool MS>
__global__ __launch_bounds__(64 * wk_waves(XM, PER, CPW)) void decode_wk_pair_kernel(WkProb<ST, YT> p0,
                                                                                    WkProb<ST, YT> p1,
                                                                                    unsigned nb0) {
  extern __shared__ u32x4 wk_lds[];
  if (blockIdx.x < nb0)
    decode_wk_body<XM, ST, YT, CPW, PER, NT, MS>(wk_lds, blockIdx.x, p0.X, p0.M, p0.K, p0.W, p0.N, p0.pre, p0.post,
                                                 p0.Y, p0.T3, p0.gin, p0.gsum, p0.gscale, p0.gout, p0.gout_bf16);
  else
    decode_wk_body<XM, ST, YT, CPW, PER, NT, MS>(wk_lds, blockIdx.x - nb0, p1.X, p1.M, p1.K, p1.W, p1.N, p1.pre,
                                                 p1.post, p1.Y, p1.T3, p1.gin, p1.gsum, p1.gscale, p1.gout,
                                                 p1.gout_bf16);
}

template <int XM, typename ST, typename YT, int CPW, int PER, bool NT = true, bool MS = false>
hipError_t launch_wk(const LinearArgs& a) {
  if constexpr (XM == WK_B2 && NT) {
    if (a.gsum) return launch_wk<XM, ST, YT, CPW, PER, false>(a);   // the backward's contractions
  }
  if constexpr (!MS) {
    // More slices than waves: the instance with the per-slice compensated fold.
    if ((a.K / 32 + DEC_STEPS - 1) / DEC_STEPS > wk_waves(XM, PER, CPW)) return launch_wk<XM, ST, YT, CPW, PER, NT, true>(a);
  }
  const int64_t blocks = (a.N + 16 * CPW - 1) / (16 * CPW);
  if (blocks > 0x7fffffff || a.M > 4 * PER) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_wk_kernel<XM, ST, YT, CPW, PER, NT, MS>), dim3((unsigned)blocks),
                     dim3(64 * wk_waves(XM, PER, CPW)), wk_lds_bytes(XM, PER, CPW), a.stream,
                     static_cast<const bf16_t*>(a.X), (int)a.M, a.K, a.W, a.N, static_cast<const f16_t*>(a.pre),
                     static_cast<const ST*>(a.post), static_cast<YT*>(a.Y), static_cast<bf16_t*>(a.T3),
                     static_cast<const bf16_t*>(a.gin), a.gsum, static_cast<const ST*>(a.gscale), a.gout,
                     a.gout_dtype == DT_BF16 ? 1 : 0);
  return hipGetLastError();
}

template <int XM, typename ST, typename YT, int CPW>
hipError_t launch_wk_rows(const LinearArgs& a) {
  const int per = wk_per(a.M);
  if (per == 1) return launch_wk<XM, ST, YT, CPW, 1>(a);
  if (per == 2) return launch_wk<XM, ST, YT, CPW, 2>(a);
  if constexpr (XM == WK_B2) {
    if (per == 4) return launch_wk<XM, ST, YT, CPW, 4>(a);
    return launch_wk<XM, ST, YT, CPW, 8>(a);
  }
  return hipErrorInvalidValue;   // WK_T3 serves up to 8 rows
}

// Columns per wave of the whole-K variant, or 0 for the split kernel.  The
// test suite can force either (forced_kernels().decode).
int wk_columns_per_wave(const LinearArgs& a, const DeviceInfo& dev) {
  const int forced = forced_kernels().decode;
  if (forced == 1) return 0;
  int cpw = forced > 10 ? forced - 10 : 0;
  if (cpw == 0) {
    // Default: the fewest columns per wave that keep the grid within one
    // workgroup per CU (the 16-row staging takes most of a CU's LDS, so a
    // second round of workgroups pays the whole latency chain again).
    // Same-box timings, us per call, CPW = 1 / 2 / 4: 16 x 4096 x 4096
    // 6.4 / 8.0 / 11.4; 16 x 4096 x 14336 20.8 / 14.7 / 11.7; 16 x 4096 x
    // 11008 16.1 / 14.4 / 11.5 (the split kernel: 8.4, 16.7, 14.6).
    const int64_t cols = (a.N + 15) / 16;
    cpw = cols <= dev.num_cus ? 1 : (cols <= 2 * dev.num_cus ? 2 : 4);
  }
  return cpw;
}

// Operands the kernel DMAs 16-byte aligned, K % 128 == 0, byte ranges (and
// offsets, with one slice to spare) within 32 bits.  `terms`: X is [3][M][K].
bool wk_operands_ok(const LinearArgs& a, int terms) {
  const int64_t lim = (int64_t)0xFFFFF000u - 4096;
  return a.K % 128 == 0 && reinterpret_cast<uintptr_t>(a.X) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(a.W) % 16 == 0 && terms * a.M * a.K * 2 <= lim && a.N * (a.K / 32) * 4 <= lim;
}

// Mode B2 with b 16-byte aligned too.
bool wk_eligible(const LinearArgs& a, bool b2) {
  return b2 && reinterpret_cast<uintptr_t>(a.pre) % 16 == 0 && wk_operands_ok(a, 1);
}

template <int XM, typename ST, typename YT>
hipError_t launch_wk_any(const LinearArgs& a, int cpw) {
  if (cpw == 4) return launch_wk_rows<XM, ST, YT, 4>(a);
  if (cpw == 2) return launch_wk_rows<XM, ST, YT, 2>(a);
  return launch_wk_rows<XM, ST, YT, 1>(a);
}

// K-slices of the split kernel.
int64_t split_slices(const LinearArgs& a) { return (a.K / 32 + DEC_STEPS - 1) / DEC_STEPS; }

// The backward's pair in one launch: mode B2, fp16 scales, fp32 outputs, plain
// sign loads (NT = false, as launch_wk picks for a gradient epilogue).
template <int CPW, int PER, bool MS>
hipError_t launch_pair_t(const LinearArgs& t, const LinearArgs& u, int64_t nb0, int64_t nb1) {
  auto prob = [](const LinearArgs& a) {
    return WkProb<f16_t, float>{static_cast<const bf16_t*>(a.X), (int)a.M, a.K, a.W, a.N,
                                static_cast<const f16_t*>(a.pre), static_cast<const f16_t*>(a.post),
                                static_cast<float*>(a.Y), static_cast<bf16_t*>(a.T3),
                                static_cast<const bf16_t*>(a.gin), a.gsum, static_cast<const f16_t*>(a.gscale),
                                a.gout, a.gout_dtype == DT_BF16 ? 1 : 0};
  };
  hipLaunchKernelGGL((decode_wk_pair_kernel<WK_B2, f16_t, float, CPW, PER, false, MS>), dim3((unsigned)(nb0 + nb1)),
                     dim3(64 * wk_waves(WK_B2, PER, CPW)), wk_lds_bytes(WK_B2, PER, CPW), t.stream, prob(t), prob(u),
                     (unsigned)nb0);
  return hipGetLastError();
}

template <int CPW, int PER>
hipError_t launch_pair_ms(const LinearArgs& t, const LinearArgs& u, int64_t nb0, int64_t nb1, bool ms) {
  return ms ? launch_pair_t<CPW, PER, true>(t, u, nb0, nb1) : launch_pair_t<CPW, PER, false>(t, u, nb0, nb1);
}

template <int CPW>
hipError_t launch_pair_per(const LinearArgs& t, const LinearArgs& u, int64_t nb0, int64_t nb1, int per, bool ms) {
  if (per == 1) return launch_pair_ms<CPW, 1>(t, u, nb0, nb1, ms);
  if (per == 2) return launch_pair_ms<CPW, 2>(t, u, nb0, nb1, ms);
  if (per == 4) return launch_pair_ms<CPW, 4>(t, u, nb0, nb1, ms);
  return launch_pair_ms<CPW, 8>(t, u, nb0, nb1, ms);
}

template <int MODE, typename XT, typename ST, typename YT, bool PRE>
hipError_t launch_t(const LinearArgs& a, const DeviceInfo& dev) {
  const int64_t kw = a.K / 32;
  const int64_t tiles = (a.N + DEC_BN - 1) / DEC_BN;
  const int64_t nslices = split_slices(a);
  float* partials = nullptr;
  if (nslices > 1) {
    partials = a.sx ? a.sx->get(0, (size_t)(nslices * a.M * a.N)) : nullptr;
    if (!partials) return hipErrorInvalidValue;
  }
  const bool fast = (kw % 4 == 0) && (reinterpret_cast<uintptr_t>(a.W) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(a.X) % 16 == 0);
  const int64_t blocks = tiles * nslices;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  auto X = static_cast<const XT*>(a.X);
  auto pre = static_cast<const ST*>(a.pre);
  auto post = static_cast<const ST*>(a.post);
  auto Y = static_cast<YT*>(a.Y);
  if (fast)
    hipLaunchKernelGGL((decode_mfma_kernel<MODE, XT, ST, YT, PRE, true>), dim3((unsigned)blocks),
                       dim3(DEC_THREADS), 0, a.stream, X, (int)a.M, a.K, a.W, a.N, pre, post, Y,
                       (int)nslices, partials);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<MODE, XT, ST, YT, PRE, false>), dim3((unsigned)blocks),
                       dim3(DEC_THREADS), 0, a.stream, X, (int)a.M, a.K, a.W, a.N, pre, post, Y,
                       (int)nslices, partials);
  if (nslices > 1) {
    const int64_t MN = a.M * a.N;
    hipLaunchKernelGGL((splitk_reduce_kernel<ST, YT>), dim3((unsigned)((MN + 255) / 256)), dim3(256), 0,
                       a.stream, partials, (int)nslices, MN, a.N, post, Y);
  }
  return hipGetLastError();
}

// Whether the call runs on the whole-K kernel in mode B2 (bf16 x with an fp16
// input-side scale, aligned; every public entry point passes an input-side
// scale, so only this mode reaches it), and with how many column groups per
// wave; 0 for the split kernel.
int wk_b2_columns(const LinearArgs& a, const DeviceInfo& dev) {
  const bool b2 = a.x_dtype == DT_BF16 && a.pre && a.scale_dtype == DT_F16;
  if (!wk_eligible(a, b2)) return 0;
  const int cpw = wk_columns_per_wave(a, dev);
  return (cpw > 0 && (!a.T3 || a.y_dtype == DT_F32)) ? cpw : 0;
}

template <typename ST, typename YT>
hipError_t launch_mode(const LinearArgs& a, const DeviceInfo& dev) {
  // bf16 x: A is x itself (any alignment: the staging copies it to LDS).
  const bool raw = a.x_dtype == DT_BF16;
  const bool b1 = raw && !a.pre, b2 = raw && a.pre && a.scale_dtype == DT_F16;
  if (a.x_dtype == DT_BF16X3) {
    // Exact bf16 terms of an fp32 input (DBF stage 2): the whole-K kernel only.
    const int cpw = wk_columns_per_wave(a, dev);
    if (a.pre || a.T3 || a.M > 8 || cpw == 0 || !wk_operands_ok(a, 3)) return hipErrorInvalidValue;
    return launch_wk_any<WK_T3, ST, YT>(a, cpw);
  }
  if constexpr (std::is_same<ST, f16_t>::value) {
    const int cpw = wk_b2_columns(a, dev);
    if (cpw > 0) return launch_wk_any<WK_B2, ST, YT>(a, cpw);
  }
  if (a.T3 || a.gsum || a.gout) return hipErrorInvalidValue;   // epilogues of the whole-K kernel only
  if (a.M > kDecodeMaxM) return hipErrorInvalidValue;   // the split kernel stages 16 rows
  if (b1) return launch_t<MODE_B1, bf16_t, ST, YT, false>(a, dev);
  if (b2) return launch_t<MODE_B2, bf16_t, ST, YT, true>(a, dev);
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
  if (a.M < 1 || a.M > kDecodeWideMaxM || (a.M > kDecodeMaxM && !decode_wide_ok(a))) return hipErrorInvalidValue;
  return a.scale_dtype == DT_F32 ? launch_y<float>(a, dev) : launch_y<f16_t>(a, dev);
}

// 17..32 rows by default: on the whole-K kernel (one launch, fp32
// contraction) while each of its 4 waves has at most 4 slices; the prefill
// GEMM otherwise.  Same-box timings, us per call, GEMM vs whole-K: K = 4096
// and N = 4096 11.3 / 8.3 (M = 17) and 12.7 / 8.4 (M = 32); N = 11008
// 22.1 / 13.6 and 23.3 / 14.1; N = 14336 22.8 / 13.7 and 24.0 / 14.3; K = 11008,
// N = 4096, M = 32 20.1 / 19.4; K = 14336, N = 4096, M = 24 22.6 / 23.0.
bool decode_wide_preferred(const LinearArgs& a) {
  return a.M > kDecodeMaxM && a.K <= 8192 && decode_wide_ok(a);
}

bool decode_terms_ok(const LinearArgs& s1, const LinearArgs& s2) {
  if (!decode_wide_ok(s1) || s1.M > 8 || s1.y_dtype != DT_F32 || s2.pre) return false;
  LinearArgs t = s2;
  t.X = s2.W;   // the terms go to 256-byte aligned library scratch: only sizes and W are checked
  return wk_operands_ok(t, 3);
}

hipError_t launch_decode_pair(const LinearArgs& t, const LinearArgs& u, const DeviceInfo& dev) {
  const auto plain = [](const LinearArgs& a) {
    return a.x_dtype == DT_BF16 && a.scale_dtype == DT_F16 && a.y_dtype == DT_F32 && a.gsum && !a.T3 && !a.Y2 &&
           decode_wide_ok(a);
  };
  if (t.M != u.M || t.stream != u.stream || !plain(t) || !plain(u)) return hipErrorNotSupported;
  // Columns per wave: a forced whole-K variant for both, else the fewest that
  // keep the two grids together within one workgroup per CU.
  const int forced = forced_kernels().decode;
  int cpw = forced > 10 ? forced - 10 : 0;
  const int64_t ct = (t.N + 15) / 16, cu = (u.N + 15) / 16;
  if (cpw == 0) {
    cpw = 4;
    for (int c = 1; c <= 2; c *= 2)
      if ((ct + c - 1) / c + (cu + c - 1) / c <= dev.num_cus) {
        cpw = c;
        break;
      }
  }
  if (cpw != 1 && cpw != 2 && cpw != 4) return hipErrorNotSupported;
  const int per = wk_per(t.M);
  const int waves = wk_waves(WK_B2, per, cpw);
  // One instance for both: the same choice of the compensated per-slice fold.
  const bool ms_t = (t.K / 32 + DEC_STEPS - 1) / DEC_STEPS > waves;
  const bool ms_u = (u.K / 32 + DEC_STEPS - 1) / DEC_STEPS > waves;
  if (ms_t != ms_u || t.M > 4 * per) return hipErrorNotSupported;
  const int64_t nb0 = (t.N + 16 * cpw - 1) / (16 * cpw), nb1 = (u.N + 16 * cpw - 1) / (16 * cpw);
  if (nb0 + nb1 > 0x7fffffff) return hipErrorNotSupported;
  if (cpw == 1) return launch_pair_per<1>(t, u, nb0, nb1, per, ms_t);
  if (cpw == 2) return launch_pair_per<2>(t, u, nb0, nb1, per, ms_t);
  return launch_pair_per<4>(t, u, nb0, nb1, per, ms_t);
}

bool decode_wide_ok(const LinearArgs& a) {
  const bool b2 = a.x_dtype == DT_BF16 && a.pre && a.scale_dtype == DT_F16;
  // (Y2, the bf16 copy of the output for a DBF prefill stage, is written by
  // the prefill GEMM only.)
  return a.M >= 1 && a.M <= kDecodeWideMaxM && !a.Y2 && wk_eligible(a, b2) && forced_kernels().decode != 1;
}

void decode_scratch(const LinearArgs& a, const DeviceInfo& dev, ScratchNeed* need) {
  if (a.x_dtype == DT_BF16X3 || wk_b2_columns(a, dev) > 0) return;   // the whole-K kernel: none
  const int64_t nslices = split_slices(a);
  if (nslices > 1) need->need(0, (size_t)(nslices * a.M * a.N));
}

}  // namespace obl
