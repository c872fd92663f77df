// Decode GEMV for M <= 2 rows: Y = ((X ⊙ b) W_sign^T) ⊙ a in fp32.
//
// OneBit page ("1bit量化"), proposition 1: the contraction with W_sign only
// adds or subtracts x_k b_k; a is applied once per output.  The DBF page
// ("Methodologie") makes the same point: the binary matrices turn the
// multiplications into additions.
//
// Design (bandwidth-bound at M = 1; every sign bit is read once from HBM):
//  * The sign additions are regrouped four k at a time.  For a group of four
//    inputs x'_4g..x'_4g+3 (x' = x ⊙ b in fp32) a table holds all 16 signed
//    sums  T[n] = Σ_i (bit i of n ? -x'_i : x'_i).  One nibble of a packed
//    sign word then selects the sum of its four signed terms: one bit-field
//    extract, one LDS read and one fp32 add replace four conditional adds.
//  * The table (one per input row) is built by the block in LDS from X and b
//    for a 4096-k slab: 1024 groups x 16 entries.  Group (c, q) -- chunk c of
//    128 k, nibble q of that chunk -- sits so that the 32 lanes of a
//    half-wave (c = 0..31, same q) hit 32 different banks whatever nibbles
//    they read.  Two rows (M = 2): dword column 33c + q of each 16-entry row.
//    One row: the paired layout (entry strides 256 and 4096 bytes for even
//    and odd q), where one shift of a sign word puts two nibbles at bits
//    8..15 and each lookup address is a single v_and_or: 19 VALU ops per 8
//    lookups instead of 24, and the table is stored with ds_write2st64 (half
//    the store instructions).  Same entries, same order of adds: results are
//    bitwise those of the padded layout.  Measured 3.78 -> 3.69 us per launch
//    (1 x 4096 x 11008); the lookups are then bound by VALU issue and LDS
//    reads about equally (~0.6 us per launch: a build that skips them takes
//    3.05 us).
//  * Lane l of a half-wave owns chunk c = l % 32 (4 sign words per row); a
//    half-wave walks whole rows.  All loads are issued up front, table inputs
//    first: every wave issues its X/b loads, a bare barrier, then the 128-bit
//    sign loads, so the small L2-resident inputs are not queued behind the HBM
//    stream in the CU's memory pipeline; the table barrier waits only for LDS,
//    so the sign loads stay in flight while the table is built.
//  * Per-lane partial sums are reduced across the 32 lanes with DPP
//    (quad_perm, half-mirror, mirror) plus one swizzle, in a fixed order, so
//    results are bitwise reproducible.  No atomics.
#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

constexpr int LUT_THREADS = 1024;
constexpr int LUT_HALFWAVES = LUT_THREADS / 32;  // 32
constexpr int LUT_SLAB_K = 4096;                 // 32 chunks x 128 k
constexpr int LUT_COLS = 33 * 32;                // padded columns per nibble row
// Paired layout (one input row), in dwords: group (chunk c, nibble position
// q), entry n at
//   q even:  1024 (q / 2) + 64 n + c + q            (entry stride 256 bytes)
//   q odd:   LUT_ODD_DW + 1024 n + 64 (q / 2) + c + q  (entry stride 4096 bytes)
// Both strides are multiples of the 32 banks, so a lookup's bank is
// (c + q) mod 32 whatever the nibble: the 32 lanes of a half-wave (c = 0..31)
// never collide.  Entry offsets 256 n and 4096 n are a nibble moved to bits
// 8..11 or 12..15.
constexpr int LUT_ODD_DW = 16384;
constexpr int LUT_PAIRED_DW = 2 * LUT_ODD_DW;     // 128 KiB

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over the 32 lanes of each half-wave; every lane receives the total.
__device__ __forceinline__ float halfwave_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror: combine the two quads of each 8
  v += dpp_mov<0x140>(v);  // row_mirror: combine the two 8-lane halves of each row
  v += __shfl_xor(v, 16);  // combine the two 16-lane rows of the half-wave
  return v;
}

// Four consecutive elements (8 or 16 bytes, aligned) as fp32.
__device__ __forceinline__ void load4(const bf16_t* p, float (&o)[4]) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xFFFF0000u);
  o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xFFFF0000u);
}
__device__ __forceinline__ void load4(const f16_t* p, float (&o)[4]) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  o[0] = to_f32(f16_t{uint16_t(v.x)}); o[1] = to_f32(f16_t{uint16_t(v.x >> 16)});
  o[2] = to_f32(f16_t{uint16_t(v.y)}); o[3] = to_f32(f16_t{uint16_t(v.y >> 16)});
}
__device__ __forceinline__ void load4(const float* p, float (&o)[4]) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}

// VEC4: K % 128 == 0 and W, X, b aligned for 16-byte sign loads and 4-element
// X / b loads (one load per thread and input instead of four: fewer requests
// queued ahead of the sign stream).
template <int MR, int RPH, bool MULTI, typename XT, typename ST, typename YT, bool PRE, bool VEC4>
__global__ __launch_bounds__(LUT_THREADS) void gemv_lut_kernel(
    const XT* __restrict__ X, int64_t K, const uint32_t* __restrict__ W, int64_t N,
    const ST* __restrict__ pre, const ST* __restrict__ post, YT* __restrict__ Y,
    int rows_per_block, uint64_t* __restrict__ span) {
  // Start of this wave in constant-clock ticks; stored at the end only when
  // a span record was asked for (the read is issued unconditionally: no
  // branch, and its wait falls on the first LDS wait below).
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  // One 16-entry table per group and row.  MR = 2: lut[(nib * LUT_COLS + col)
  // * MR + m].  MR = 1: the paired layout (see lut_dw below).
  constexpr bool PAIRED = MR == 1;
  __shared__ float lut[PAIRED ? LUT_PAIRED_DW : 16 * LUT_COLS * MR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int hw = tid >> 5;
  const int c = lane & 31;
  const int64_t row0 = (int64_t)blockIdx.x * rows_per_block;
  const int nrows = (int)min((int64_t)rows_per_block, N - row0);
  const int64_t kw = K >> 5;

  float acc[RPH][MR];
  float post_r[RPH];  // output scales of this half-wave's rows, fetched up front
#pragma unroll
  for (int r = 0; r < RPH; ++r) {
    const int row = hw + LUT_HALFWAVES * r;
    post_r[r] = scale_or_one(post, row0 + (row < nrows ? row : nrows - 1), W);   // W: >= 4N bytes
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[r][m] = 0.f;
  }

  // K > 4096 (MULTI): each slab's lookups start a fresh per-lane sum, and the
  // slab sums are added with compensated (Kahan) summation, so a lane's error
  // stays that of one slab's 32 adds plus about two roundings whatever K is.
  float ktot[RPH][MR], kcomp[RPH][MR];
#pragma unroll
  for (int r = 0; r < RPH; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) ktot[r][m] = kcomp[r][m] = 0.f;

  // K <= 4096 (MULTI = false) runs the slab body once, with no loop: a loop
  // header would drain vmcnt and wait for the output-scale loads above.
  const int64_t nslab = MULTI ? K : 1;
  for (int64_t s0 = 0; s0 < nslab; s0 += LUT_SLAB_K) {
    if constexpr (MULTI) {
#pragma unroll
      for (int r = 0; r < RPH; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[r][m] = 0.f;
    }
    // This thread's table group g (k = s0 + 4g .. +3), i.e. chunk g / 32,
    // nibble position g % 32.  Paired layout: wave w builds nibble positions
    // of parity w % 2 in chunks 4(w / 2) .. +3, so a wave's writes share one
    // stride and a half-wave's 32 writes fall in 32 banks.
    const int g = PAIRED ? 32 * (4 * (tid >> 7) + ((tid & 63) >> 4)) + 2 * (tid & 15) + ((tid >> 6) & 1) : tid;
    const int64_t k = s0 + 4 * g;
    const bool kval = k < K;                 // K % 32 == 0: a group is all in or all out
    const int64_t kk = kval ? k : 0;

    // Sign words of this lane's chunk for each of its rows.  Rows past the
    // block's last row read a clamped row and are never looked up; words past
    // K read a clamped address and meet zero table entries, so they add nothing.
    const int64_t w0 = (s0 >> 5) + 4 * c;
    u32x4 wv[RPH];
    auto load_signs = [&]() {
#pragma unroll
      for (int r = 0; r < RPH; ++r) {
        const int row = hw + LUT_HALFWAVES * r;
        const uint32_t* src = W + (row0 + (row < nrows ? row : nrows - 1)) * kw;
        if constexpr (VEC4) {
          wv[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (w0 < kw ? w0 : kw - 4)));
        } else {
          uint32_t t[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) t[i] = src[w0 + i < kw ? w0 + i : kw - 1];
          wv[r] = u32x4{t[0], t[1], t[2], t[3]};
        }
      }
    };

    float xr[MR][4], pr[4];
    {
      // Table inputs first, from every wave, then a barrier (no memory wait),
      // then the sign words: the CU's memory pipeline serves requests in issue
      // order, so the small, L2-resident table inputs are not queued behind the
      // HBM-bound sign stream.  Loads are unconditional (clamped addresses).
      if constexpr (VEC4) {
#pragma unroll
        for (int m = 0; m < MR; ++m) load4(X + m * K + kk, xr[m]);
        if constexpr (PRE) load4(pre + kk, pr);
        else pr[0] = pr[1] = pr[2] = pr[3] = 1.f;
      } else {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) xr[m][i] = to_f32(X[m * K + kk + i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (PRE) pr[i] = to_f32(pre[kk + i]);
          else pr[i] = 1.f;
        }
      }
      // Barrier without a wait for global loads: every wave has issued its
      // table inputs before any wave issues sign loads.  For later slabs it
      // also orders every wave's reads of the previous table before the
      // writes of this one: each wave's LDS reads complete (release fence on
      // LDS: lgkmcnt(0)) before it arrives.  Neither waits for the X/b loads
      // just issued.
      if (MULTI && s0 > 0) {
        lds_barrier();
      } else {
        __builtin_amdgcn_s_barrier();
      }
      load_signs();
    }

    // Table for this slab.  Thread tid owns group g (k = s0 + 4g .. +3).
    {
      const int col = 33 * (g >> 5) + (g & 31);
      const int gq = g & 31, gc = g >> 5;
      // Nibble parity, the same for the whole wave (held in a scalar register,
      // so the store loops below get one stride and immediate offsets each).
      const int odd = __builtin_amdgcn_readfirstlane((tid >> 6) & 1);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = kval ? xr[m][i] * pr[i] : 0.f;
        // bit i of the nibble set -> -x_i.  p indexed by bits (0,1), q by bits (2,3).
        const float p0 = x[0] + x[1], p2 = x[0] - x[1];
        const float q0 = x[2] + x[3], q2 = x[2] - x[3];
        const float p[4] = {p0, -p2, p2, -p0};
        const float q[4] = {q0, -q2, q2, -q0};
        if constexpr (PAIRED) {
          if (odd) {
            // Base held opaque, as for the odd lookups: 64 KiB folded into
            // the offsets would not fit the offset field.
            uint32_t eb = 4u * (LUT_ODD_DW + 64 * (gq >> 1) + gc + gq);
            asm volatile("" : "+v"(eb));
            char* e = reinterpret_cast<char*>(lut) + eb;
#pragma unroll
            for (int n = 0; n < 16; ++n) *reinterpret_cast<float*>(e + 4096 * n) = p[n & 3] + q[n >> 2];
          } else {
            float* e = &lut[1024 * (gq >> 1) + gc + gq];
#pragma unroll
            for (int n = 0; n < 16; ++n) e[64 * n] = p[n & 3] + q[n >> 2];
          }
        } else {
#pragma unroll
          for (int n = 0; n < 16; ++n) lut[(n * LUT_COLS + col) * MR + m] = p[n & 3] + q[n >> 2];
        }
      }
    }
    lds_barrier();  // table visible; sign loads may still be in flight

    // Lookups: one nibble -> one signed 4-term sum per input row.  Each row's
    // sign load is pinned (an empty asm that takes the register) just before
    // its own lookups and outside their condition: the pin stops the compiler
    // from sinking the load into the conditional block (i.e. after the table
    // build), and the wait for row r's data lands only there, so a wave starts
    // on its first row while its later rows are still arriving (the CU returns
    // loads in issue order, staggered across waves).
    const int cbase = 33 * c;
#pragma unroll
    for (int r = 0; r < RPH; ++r) {
      asm volatile("" : "+v"(wv[r]));
      if (PAIRED && hw + LUT_HALFWAVES * r < nrows) {
        // Nibbles q (even) and q + 1 of a word, moved to bits 8..11 and 12..15
        // by one shift, are the table's byte offsets 256 nib and 4096 nib: one
        // v_and_or per address, the rest in the LDS offset field.  Adds in q
        // order, as below.
        const uint32_t words[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
        const char* lb = reinterpret_cast<const char*>(lut);
        // The odd-entry base (64 KiB + 4c) held opaque: folded into the
        // constant offset it would exceed the 16-bit offset field and cost an
        // extra add per lookup.
        uint32_t bo = 4u * (LUT_ODD_DW + c);
        asm volatile("" : "+v"(bo));
#pragma unroll
        for (int q = 0; q < 32; q += 2) {
          const uint32_t wd = words[q >> 3];
          const int sh = 4 * (q & 7) - 8;
          const uint32_t ws = sh < 0 ? wd << 8 : wd >> sh;
          const uint32_t ea = (ws & 0x0F00u) | (4u * c);
          const uint32_t oa = (ws & 0xF000u) | bo;
          acc[r][0] += *reinterpret_cast<const float*>(lb + ea + 4 * (1024 * (q >> 1) + q));
          acc[r][0] += *reinterpret_cast<const float*>(lb + oa + 4 * (64 * (q >> 1) + q + 1));
        }
      } else if (!PAIRED && hw + LUT_HALFWAVES * r < nrows) {
        const uint32_t words[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
#pragma unroll
        for (int q = 0; q < 32; ++q) {
          const uint32_t nib = (words[q >> 3] >> ((q & 7) * 4)) & 15u;
          const float* e = &lut[(nib * LUT_COLS + cbase + q) * MR];
#pragma unroll
          for (int m = 0; m < MR; ++m) acc[r][m] += e[m];
        }
      }
    }
    if constexpr (MULTI) {
#pragma unroll
      for (int r = 0; r < RPH; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const float y = acc[r][m] - kcomp[r][m];
          const float t = ktot[r][m] + y;
          kcomp[r][m] = (t - ktot[r][m]) - y;
          ktot[r][m] = t;
        }
    }
  }
  if constexpr (MULTI) {
#pragma unroll
    for (int r = 0; r < RPH; ++r)
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[r][m] = ktot[r][m];
  }

  // Reduce across the half-wave and write the scaled outputs.  A row index is
  // uniform within a half-wave; the reduction runs while any half of the wave
  // still has a row (DPP reads stay inside each half).
#pragma unroll
  for (int r = 0; r < RPH; ++r) {
    const int row = hw + LUT_HALFWAVES * r;
    if ((hw & ~1) + LUT_HALFWAVES * r >= nrows) break;   // neither half of this wave has row r
    float tot[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) tot[m] = halfwave_sum(acc[r][m]);
    if (c == 0 && row < nrows) {
      const int64_t n = row0 + row;
#pragma unroll
      for (int m = 0; m < MR; ++m) Store<YT>::put(&Y[m * N + n], tot[m] * post_r[r]);
    }
  }
  if (span) {   // uniform: the block's start (wave 0) and end (after every wave's stores)
    __syncthreads();
    if (tid == 0) {
      const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
      *reinterpret_cast<u32x4*>(span + 2 * blockIdx.x) =
          u32x4{(uint32_t)t_start, (uint32_t)(t_start >> 32), (uint32_t)t_end, (uint32_t)(t_end >> 32)};
    }
  }
}

template <int MR, int RPH, typename XT, typename ST, typename YT, bool PRE>
hipError_t launch_rph(const LinearArgs& a, int64_t blocks, int rpb) {
  const bool vec4 = (a.K % 128 == 0) && (reinterpret_cast<uintptr_t>(a.W) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(a.X) % (4 * sizeof(XT)) == 0) &&
                    (!a.pre || reinterpret_cast<uintptr_t>(a.pre) % (4 * sizeof(ST)) == 0);
  auto X = static_cast<const XT*>(a.X);
  auto pre = static_cast<const ST*>(a.pre);
  auto post = static_cast<const ST*>(a.post);
  auto Y = static_cast<YT*>(a.Y);
  const dim3 grid((unsigned)blocks), block(LUT_THREADS);
  const bool multi = a.K > LUT_SLAB_K;
  if (vec4 && !multi)
    hipLaunchKernelGGL((gemv_lut_kernel<MR, RPH, false, XT, ST, YT, PRE, true>), grid, block, 0, a.stream, X, a.K, a.W, a.N, pre, post, Y, rpb, a.span);
  else if (vec4)
    hipLaunchKernelGGL((gemv_lut_kernel<MR, RPH, true, XT, ST, YT, PRE, true>), grid, block, 0, a.stream, X, a.K, a.W, a.N, pre, post, Y, rpb, a.span);
  else
    hipLaunchKernelGGL((gemv_lut_kernel<MR, RPH, true, XT, ST, YT, PRE, false>), grid, block, 0, a.stream, X, a.K, a.W, a.N, pre, post, Y, rpb, a.span);
  return hipGetLastError();
}

// Rows per block: N spread over a whole number of blocks per CU (the fewest
// that respects the row cap), at least 16 rows to amortise the table build,
// at most 32 x RPH.  LDS: the tables take 67.5 KB per input row, so M = 2
// fits too; rows per half-wave go up to four (M = 1) and one (M = 2, register
// budget of the two accumulators per row).  At M = 2 and N = 11008 this gives
// 22 rows in two blocks per CU, measured faster than 32-row blocks spread
// unevenly (344 blocks on 256 CUs): 6.08 vs 6.36 us.
template <int MR, typename XT, typename ST, typename YT, bool PRE>
hipError_t launch_t(const LinearArgs& a, const DeviceInfo& dev) {
  constexpr int64_t max_rows = (MR == 1 ? 4 : 1) * LUT_HALFWAVES;
  const int64_t per_cu = (a.N + dev.num_cus * max_rows - 1) / (dev.num_cus * max_rows);   // >= 1
  int64_t rpb = (a.N + per_cu * dev.num_cus - 1) / (per_cu * dev.num_cus);
  if (rpb < 16) rpb = a.N < 16 ? a.N : 16;
  if (rpb > max_rows) rpb = max_rows;
  const int64_t blocks = (a.N + rpb - 1) / rpb;
  if constexpr (MR == 2) {
    return launch_rph<MR, 1, XT, ST, YT, PRE>(a, blocks, (int)rpb);
  } else {
    if (rpb <= 2 * LUT_HALFWAVES) return launch_rph<MR, 2, XT, ST, YT, PRE>(a, blocks, (int)rpb);
    return launch_rph<MR, 4, XT, ST, YT, PRE>(a, blocks, (int)rpb);
  }
}

template <int MR, typename XT, typename ST, typename YT>
hipError_t launch_pre(const LinearArgs& a, const DeviceInfo& dev) {
  return a.pre ? launch_t<MR, XT, ST, YT, true>(a, dev) : launch_t<MR, XT, ST, YT, false>(a, dev);
}

template <int MR, typename XT, typename ST>
hipError_t launch_y(const LinearArgs& a, const DeviceInfo& dev) {
  return a.y_dtype == DT_F32 ? launch_pre<MR, XT, ST, float>(a, dev)
                             : launch_pre<MR, XT, ST, bf16_t>(a, dev);
}

template <int MR, typename XT>
hipError_t launch_s(const LinearArgs& a, const DeviceInfo& dev) {
  return a.scale_dtype == DT_F32 ? launch_y<MR, XT, float>(a, dev) : launch_y<MR, XT, f16_t>(a, dev);
}

template <int MR>
hipError_t launch_x(const LinearArgs& a, const DeviceInfo& dev) {
  return a.x_dtype == DT_F32 ? launch_s<MR, float>(a, dev) : launch_s<MR, bf16_t>(a, dev);
}

}  // namespace

hipError_t launch_gemv_lut(const LinearArgs& a, const DeviceInfo& dev) {
  if (a.M == 1) return launch_x<1>(a, dev);
  if (a.M == 2) return launch_x<2>(a, dev);
  return hipErrorInvalidValue;
}

}  // namespace obl
