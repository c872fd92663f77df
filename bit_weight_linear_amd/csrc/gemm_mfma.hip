// Prefill contraction for M > 16 on bf16 matrix cores:
// Y = ((X ⊙ b) W_sign^T) ⊙ a with fp32 accumulation.
//
// OneBit page ("1bit量化"), proposition 1; for M > 16 this is a dense
// contraction (2·M·N·K flops), so it runs on v_mfma_f32_16x16x32_bf16.
//
// Operands per 32-k step, in pair order (obl_common.hpp):
//  * B (weights) is never stored as bf16 anywhere: each wave reads packed sign
//    words from LDS and expands them in registers -- one shift and one
//    v_bitop3 per two weights -- into +-m_k, where m_k is bf16(b_k) when the
//    input-side scale is folded into B ("raw" A mode) or 1.0 otherwise.
//  * A (activations) is staged in LDS already in pair order, one 16-byte
//    fragment per lane, so each A fragment is a single ds_read_b128.
//      raw mode     (X bf16):  A = x exactly; b is folded into B as bf16(b).
//      convert mode (X fp32, or no b):  A = bf16(x·b) (or bf16(x)), B = +-1.
//    Either way each product carries one bf16 rounding of one input-side
//    factor (relative error <= 2^-8), products are exact in fp32 and the
//    accumulation is fp32.
//  * Epilogue: acc·a in fp32, one cast to the output dtype.
//
// Tiling: 256 x 224 block tile, 8 waves as 4 (M) x 2 (N), 64 x 112 per wave
// (4 x 7 fragments, 112 fp32 accumulators per lane), K staged 64 at a time in
// double-buffered LDS.  For M = 2048, N = 14336 this gives 8 x 64 = 512 tiles,
// exactly two per CU on 256 CUs.  Workgroups are dispatched round-robin over
// the 8 XCDs, so the tile order puts all tiles of one block-row on one XCD:
// that XCD's L2 then holds the shared activation rows.
#include <type_traits>

#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

constexpr int GM_BM = 256;
constexpr int GM_BN = 224;
constexpr int GM_KT = 64;
constexpr int GM_STEPS = GM_KT / 32;
constexpr int GM_THREADS = 512;
constexpr int GM_FM = 4;   // A fragments per wave (64 rows)
constexpr int GM_FN = 7;   // B fragments per wave (112 columns)
constexpr int GM_SLOTS = GM_STEPS * (GM_BM / 16) * 64;  // A fragment slots per stage
constexpr int GM_SLOTS_PER_THREAD = GM_SLOTS / GM_THREADS;

enum AMode { A_RAW = 0, A_CONVERT = 1 };

struct GemmSmem {
  u32x4 a[2][GM_STEPS][GM_BM / 16][64];
  uint32_t bw[2][GM_BN][GM_STEPS];
  u32x4 mag[2][GM_STEPS][4];
};

// Two 4-element runs r0 = (v0..v3), r1 = (v16..v19) of bf16 -> pair order
// dwords (v_j, v_{16+j}).
__device__ __forceinline__ u32x4 interleave_pairs(u32x2 r0, u32x2 r1) {
  u32x4 o;
  o.x = __builtin_amdgcn_perm(r1.x, r0.x, 0x05040100u);
  o.y = __builtin_amdgcn_perm(r1.x, r0.x, 0x07060302u);
  o.z = __builtin_amdgcn_perm(r1.y, r0.y, 0x05040100u);
  o.w = __builtin_amdgcn_perm(r1.y, r0.y, 0x07060302u);
  return o;
}

// One pipeline stage of global data held in registers between its loads and
// its LDS store.  Loads are issued without branches (an invalid element reads a
// clamped, valid address and is zeroed at store time), so a stage costs one
// memory round trip and overlaps the MFMA work of the previous stage.  In raw
// mode the registers hold the loaded bits untouched and the pair-order
// interleave happens at store time; convert mode (fp32 or misaligned X) does
// its arithmetic at load time.
template <int AMODE, typename XT, typename ST, bool PRE>
struct Stager {
  static constexpr bool kRaw = AMODE == A_RAW;
  static constexpr bool kMag = kRaw && PRE;
  u32x2 r0[GM_SLOTS_PER_THREAD], r1[GM_SLOTS_PER_THREAD];  // raw mode
  u32x4 cv[GM_SLOTS_PER_THREAD];                           // convert mode
  uint32_t valid;                                          // bit i: slot i in range
  uint32_t bw;
  u32x2 p0, p1;                                            // raw fp16/f32 b words (mag)

  __device__ __forceinline__ void load(const XT* __restrict__ X, int64_t M, int64_t K,
                                       const uint32_t* __restrict__ W, int64_t N,
                                       const ST* __restrict__ pre, int64_t m0, int64_t n0,
                                       int64_t kt, int tid) {
    const int64_t kw = K >> 5;
    valid = 0;
#pragma unroll
    for (int i = 0; i < GM_SLOTS_PER_THREAD; ++i) {
      const int slot = tid + GM_THREADS * i;
      const int g = slot & 3;
      const int row = (slot >> 2) & (GM_BM - 1);
      const int t = slot >> 10;
      const int64_t gr = m0 + row;
      const int64_t step = kt * GM_STEPS + t;
      const bool ok = gr < M && step < kw;
      valid |= uint32_t(ok) << i;
      const int64_t kb = step * 32 + 4 * g;
      const XT* xr = X + (ok ? gr * K + kb : 0);
      if constexpr (kRaw) {
        r0[i] = *reinterpret_cast<const u32x2*>(xr);
        r1[i] = *reinterpret_cast<const u32x2*>(xr + 16);
      } else {
        float lo[4], hi[4], plo[4], phi[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo[j] = to_f32(xr[j]);
          hi[j] = to_f32(xr[j + 16]);
          plo[j] = 1.f;
          phi[j] = 1.f;
          if constexpr (PRE) {
            const ST* pr = pre + (ok ? kb : 0);
            plo[j] = to_f32(pr[j]);
            phi[j] = to_f32(pr[j + 16]);
          }
        }
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = ok ? pack_bf16_pair(lo[j] * plo[j], hi[j] * phi[j]) : 0u;
        cv[i] = u32x4{d[0], d[1], d[2], d[3]};
      }
    }
    // Sign words: thread -> (column, step).
    {
      const int c = tid >> 1, t = tid & 1;
      const int64_t n = n0 + c, step = kt * GM_STEPS + t;
      const bool ok = tid < GM_BN * GM_STEPS && n < N && step < kw;
      bw = W[ok ? n * kw + step : 0];   // masked at store time
      valid |= uint32_t(ok) << 8;
    }
    // Raw b for the magnitudes of B in raw mode: bf16(b) pairs per (step, group).
    if constexpr (kMag) {
      const int r = tid - GM_BN * GM_STEPS;
      const int t = (r >> 2) & 1, g = r & 3;
      const int64_t step = kt * GM_STEPS + t;
      const bool ok = r >= 0 && r < GM_STEPS * 4 && step < kw;
      valid |= uint32_t(ok) << 9;
      const ST* pr = pre + (ok ? step * 32 + 4 * g : 0);
      if constexpr (sizeof(ST) == 2) {
        p0 = *reinterpret_cast<const u32x2*>(pr);
        p1 = *reinterpret_cast<const u32x2*>(pr + 16);
      } else {
        // fp32 b: round to bf16 here (small: 8 threads, 8 values each).
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = pack_bf16_pair(to_f32(pr[j]), to_f32(pr[j + 16]));
        p0 = u32x2{d[0], d[1]};
        p1 = u32x2{d[2], d[3]};
      }
    }
  }

  __device__ __forceinline__ void store(GemmSmem& sm, int buf, int tid) const {
    // Every thread consumes every staged register here, including the ones
    // only some threads write to LDS: otherwise the next stage's loads into
    // the same registers would wait for this stage's loads to land.
    if constexpr (kMag) asm volatile("" ::"v"(bw), "v"(p0), "v"(p1));
    else asm volatile("" ::"v"(bw));
#pragma unroll
    for (int i = 0; i < GM_SLOTS_PER_THREAD; ++i) {
      const int slot = tid + GM_THREADS * i;
      const int g = slot & 3;
      const int row = (slot >> 2) & (GM_BM - 1);
      const int t = slot >> 10;
      u32x4 v;
      if constexpr (kRaw) v = interleave_pairs(r0[i], r1[i]);
      else v = cv[i];
      if (!((valid >> i) & 1u)) v = u32x4{0u, 0u, 0u, 0u};
      sm.a[buf][t][row >> 4][16 * g + (row & 15)] = v;
    }
    if (tid < GM_BN * GM_STEPS) sm.bw[buf][tid >> 1][tid & 1] = ((valid >> 8) & 1u) ? bw : 0u;
    if constexpr (kMag) {
      const int r = tid - GM_BN * GM_STEPS;
      if (r >= 0 && r < GM_STEPS * 4) {
        u32x4 m;
        if constexpr (sizeof(ST) == 2) {
          // fp16 (b_j, b_{j+16}) -> bf16 pairs in pair order.
          const uint32_t lo[2] = {p0.x, p0.y}, hi[2] = {p1.x, p1.y};
          uint32_t d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint16_t bl = uint16_t(lo[j >> 1] >> (16 * (j & 1)));
            const uint16_t bh = uint16_t(hi[j >> 1] >> (16 * (j & 1)));
            d[j] = pack_bf16_pair(to_f32(f16_t{bl}), to_f32(f16_t{bh}));
          }
          m = u32x4{d[0], d[1], d[2], d[3]};
        } else {
          m = u32x4{p0.x, p0.y, p1.x, p1.y};
        }
        if (!((valid >> 9) & 1u)) m = u32x4{0u, 0u, 0u, 0u};
        sm.mag[buf][r >> 2][r & 3] = m;
      }
    }
  }
};

template <int AMODE, typename XT, typename ST, typename YT, bool PRE>
__global__ __launch_bounds__(GM_THREADS) void gemm_mfma_kernel(
    const XT* __restrict__ X, int64_t M, int64_t K, const uint32_t* __restrict__ W, int64_t N,
    const ST* __restrict__ pre, const ST* __restrict__ post, YT* __restrict__ Y, int mt, int nt,
    int xcd_groups) {
  __shared__ GemmSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4;

  // Tile order: with xcd_groups = 8, XCD x (= blockIdx % 8) gets the
  // contiguous tile range [x·T/8, (x+1)·T/8), row-major over (tm, tn).
  int lin = blockIdx.x;
  if (xcd_groups > 1) {
    const int per = (mt * nt) / xcd_groups;
    lin = (blockIdx.x % xcd_groups) * per + blockIdx.x / xcd_groups;
  }
  const int tm = lin / nt, tn = lin - (lin / nt) * nt;
  const int64_t m0 = (int64_t)tm * GM_BM, n0 = (int64_t)tn * GM_BN;
  const int64_t kw = K >> 5;
  const int64_t nk = (kw + GM_STEPS - 1) / GM_STEPS;

  f32x4 acc[GM_FM][GM_FN];
#pragma unroll
  for (int i = 0; i < GM_FM; ++i)
#pragma unroll
    for (int j = 0; j < GM_FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Output scales of this lane's columns, fetched before the main loop.
  float post_c[GM_FN];
#pragma unroll
  for (int j = 0; j < GM_FN; ++j) {
    const int64_t n = n0 + wn * (GM_FN * 16) + j * 16 + (lane & 15);
    post_c[j] = scale_or_one(post, n < N ? n : N - 1, W);   // W: >= 4N bytes
  }

  Stager<AMODE, XT, ST, PRE> st;
  st.load(X, M, K, W, N, pre, m0, n0, 0, tid);
  st.store(sm, 0, tid);
  __syncthreads();

  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nk) st.load(X, M, K, W, N, pre, m0, n0, kt + 1, tid);
#pragma unroll
    for (int t = 0; t < GM_STEPS; ++t) {
      u32x4 af[GM_FM];
#pragma unroll
      for (int i = 0; i < GM_FM; ++i) af[i] = sm.a[buf][t][wm * GM_FM + i][lane];
      const u32x4 mag = (AMODE == A_RAW && PRE) ? sm.mag[buf][t][g] : ones;
#pragma unroll
      for (int j = 0; j < GM_FN; ++j) {
        const uint32_t w = sm.bw[buf][wn * (GM_FN * 16) + j * 16 + (lane & 15)][t];
        const u32x4 bf = expand_signs_scaled(w >> (4 * g), mag);
#pragma unroll
        for (int i = 0; i < GM_FM; ++i) acc[i][j] = mfma16x16x32(af[i], bf, acc[i][j]);
      }
    }
    if (kt + 1 < nk) st.store(sm, buf ^ 1, tid);
    __syncthreads();
  }

  // Epilogue: lane holds rows 4g..4g+3 of column (lane & 15) of each fragment.
#pragma unroll
  for (int j = 0; j < GM_FN; ++j) {
    const int64_t n = n0 + wn * (GM_FN * 16) + j * 16 + (lane & 15);
    if (n >= N) continue;
    const float s = post_c[j];
#pragma unroll
    for (int i = 0; i < GM_FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * (GM_FM * 16) + i * 16 + 4 * g + r;
        if (m < M) Store<YT>::put(&Y[m * N + n], acc[i][j][r] * s);
      }
    }
  }
}

// ===========================================================================
// Main prefill kernel (bf16 activations, 16-byte aligned): 4 waves, one per
// SIMD, each owning a 128 (rows) x 112 (columns) output tile.
//
// The VALU cost of expanding signs is fixed per 16 x 32 sign fragment, and a
// fragment feeds one MFMA per 16 rows of the wave tile, so the VALU/MFMA ratio
// falls as the wave's row extent grows: 128 rows give 8 MFMAs per expansion.
// The 224 fp32 accumulators per lane live in AGPRs (one wave per SIMD leaves
// the whole 512-entry register file to it).
//  * Activations go global -> LDS by DMA (global_load_lds_dwordx4, no VGPRs),
//    in natural k order into an XOR-swizzled tile (16-byte chunk c of row r at
//    slot c ^ (r & 7)), so each operand fragment is one conflict-free
//    ds_read_b128.  Two stage buffers are distinct LDS objects and the K loop
//    is unrolled by two, so each access names its buffer statically and the
//    waits on the DMA are explicit s_waitcnt vmcnt(n).
//  * Sign words are unzipped once at staging (bit 2i -> i, 2i+1 -> 16+i): the
//    adjacent-k pairs of the natural order are then 16 bits apart, exactly
//    what the one-shift expansion produces.  b, when present, is folded into
//    the sign operand as bf16(b) (magnitudes, natural order).
//  * Operands are swapped (signs = MFMA A, activations = MFMA B), so a lane's
//    four accumulator values are four consecutive output columns of one row.
//  * Rows past M and columns past N read clamped (valid) addresses and are not
//    stored; k past K (last stage only) is zeroed in LDS after the DMA lands.
// ===========================================================================
constexpr int G2_BM = 256;
constexpr int G2_BN = 224;
constexpr int G2_KT = 128;
constexpr int G2_STEPS = G2_KT / 32;                       // 4
constexpr int G2_THREADS = 256;
constexpr int G2_FM = 8;                                   // 16-row fragments per wave
constexpr int G2_FN = 7;                                   // 16-column fragments per wave
constexpr int G2_CPR = G2_KT / 8;                          // 16-byte chunks per row per stage (16)
constexpr int G2_DMA = G2_BM * G2_CPR / G2_THREADS;        // DMA instructions per thread per stage (16)

template <typename ST, typename YT, bool PRE>
struct Gemm2 {
  const bf16_t* __restrict__ X;
  int64_t M, K;
  const uint32_t* __restrict__ W;
  int64_t N;
  const ST* __restrict__ pre;
  int64_t m0, n0, kw, nk;
  int tid, wave, lane;
  bool full_m;
  uint32_t loff[2];     // per-lane element offset of its DMA chunk, for even / odd instructions
  u32x4 wr;             // raw sign words of the next stage (column tid, 4 steps)
  u32x4 br;             // raw b of the next stage (mag threads)

  // Activation DMA of stage s into buffer `dst` (a [256][16] u32x4 LDS tile).
  // Instruction i of wave w fills rows 4(16w + i) .. +3; lane l takes row
  // + l/16 and LDS slot l % 16, i.e. global chunk (l % 16) ^ (row & 7).
  __device__ __forceinline__ void dma(u32x4 (*dst)[G2_CPR], int64_t s) const {
    const int64_t k0 = min(s, nk - 1) * G2_KT;
    if (full_m) {
#pragma unroll
      for (int i = 0; i < G2_DMA; ++i) {
        const int rbase = 4 * (16 * wave + i);
        load_lds16(X + (m0 + rbase) * K + k0 + loff[i & 1], &dst[rbase][0]);
      }
    } else {
      // Last row tile: rows past M re-read row M - 1 (never stored).
#pragma unroll
      for (int i = 0; i < G2_DMA; ++i) {
        const int rbase = 4 * (16 * wave + i);
        const int rr = lane >> 4;
        const int64_t row = min(m0 + rbase + rr, M - 1);
        load_lds16(X + row * K + k0 + (loff[i & 1] - (uint32_t)(rr * K)), &dst[rbase][0]);
      }
    }
  }

  // Exactly two vector loads (one without b), whatever the stage: the DMA
  // waits below count on it.
  __device__ __forceinline__ void load_side(int64_t s) {
    const int64_t st = min(s, nk - 1) * G2_STEPS;
    const int64_t n = min(n0 + min(tid, G2_BN - 1), N - 1);
    wr = *reinterpret_cast<const u32x4*>(W + n * kw + st);
    if constexpr (PRE) {
      const int r = min(max(tid - G2_BN, 0), 15);
      br = *reinterpret_cast<const u32x4*>(pre + st * 32 + 32 * (r >> 2) + 8 * (r & 3));
    }
  }

  __device__ __forceinline__ void store_side(uint32_t (*w)[G2_BN], u32x4 (*mag)[4]) const {
    if (tid < G2_BN) {
      w[0][tid] = unzip_bits(wr.x);
      w[1][tid] = unzip_bits(wr.y);
      w[2][tid] = unzip_bits(wr.z);
      w[3][tid] = unzip_bits(wr.w);
    } else {
      asm volatile("" ::"v"(wr));
    }
    if constexpr (PRE) {
      const int r = tid - G2_BN;
      if (r >= 0 && r < 16) {
        const uint32_t h[4] = {br.x, br.y, br.z, br.w};   // 8 fp16 values
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          d[j] = pack_bf16_pair(to_f32(f16_t{uint16_t(h[j] & 0xFFFFu)}), to_f32(f16_t{uint16_t(h[j] >> 16)}));
        mag[r >> 2][r & 3] = u32x4{d[0], d[1], d[2], d[3]};
      } else {
        asm volatile("" ::"v"(br));
      }
    }
  }

};

// vmcnt(n) with expcnt / lgkmcnt left alone (gfx9 encoding, n < 64).
#define OBL_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

template <typename ST, typename YT, bool PRE>
__global__ __launch_bounds__(G2_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const bf16_t* __restrict__ X, int64_t M, int64_t K, const uint32_t* __restrict__ W,
                      int64_t N, const ST* __restrict__ pre, const ST* __restrict__ post,
                      YT* __restrict__ Y, int mt, int nt, int xcd_groups) {
  __shared__ u32x4 xa[G2_BM][G2_CPR];
  __shared__ u32x4 xb[G2_BM][G2_CPR];
  __shared__ uint32_t wsa[G2_STEPS][G2_BN];
  __shared__ uint32_t wsb[G2_STEPS][G2_BN];
  __shared__ u32x4 maga[G2_STEPS][4];
  __shared__ u32x4 magb[G2_STEPS][4];
  __shared__ float post_s[G2_BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4;
  const int l16 = lane & 15;

  int lin = blockIdx.x;
  if (xcd_groups > 1) {
    const int per = (mt * nt) / xcd_groups;
    lin = (blockIdx.x % xcd_groups) * per + blockIdx.x / xcd_groups;
  }
  const int tm = lin / nt, tn = lin - (lin / nt) * nt;

  Gemm2<ST, YT, PRE> G;
  G.X = X; G.M = M; G.K = K; G.W = W; G.N = N; G.pre = pre;
  G.m0 = (int64_t)tm * G2_BM;
  G.n0 = (int64_t)tn * G2_BN;
  G.kw = K >> 5;
  G.nk = G.kw / G2_STEPS;               // K % 128 == 0 on this path
  G.tid = tid; G.wave = wave; G.lane = lane;
  G.full_m = G.m0 + G2_BM <= M;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int rr = lane >> 4;
    G.loff[p] = (uint32_t)(rr * K + 8 * ((lane & 15) ^ ((4 * p + rr) & 7)));
  }

  // Prologue: side data of stage 0, output scales, DMA of stage 0.
  G.load_side(0);
  if (tid < G2_BN) post_s[tid] = scale_or_one(post, min(G.n0 + tid, N - 1), W);   // W: >= 4N bytes
  G.store_side(wsa, maga);
  G.dma(xa, 0);

  f32x4 acc[G2_FN][G2_FM];
#pragma unroll
  for (int j = 0; j < G2_FN; ++j)
#pragma unroll
    for (int i = 0; i < G2_FM; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const int xrow0 = wm * (G2_FM * 16) + l16;
  const int wcol0 = wn * (G2_FN * 16) + l16;
  constexpr int kIssued = G2_DMA + 1 + (PRE ? 1 : 0);   // vector memory ops issued per prefetch (exact)

  auto compute = [&](u32x4 (*xs)[G2_CPR], uint32_t (*ws)[G2_BN], u32x4 (*mg)[4]) {
    // One k-step (56 independent MFMAs) per iteration; not unrolled across
    // steps, which would let the scheduler hoist later steps' operand reads
    // and exhaust the VGPRs.
#pragma unroll 1
    for (int t = 0; t < G2_STEPS; ++t) {
      u32x4 xf[G2_FM];
#pragma unroll
      for (int i = 0; i < G2_FM; ++i) xf[i] = xs[xrow0 + 16 * i][(4 * t + g) ^ (l16 & 7)];
      const u32x4 mag = PRE ? mg[t][g] : ones;
#pragma unroll
      for (int j = 0; j < G2_FN; ++j) {
        const u32x4 sf = expand_signs_scaled(ws[t][wcol0 + 16 * j] >> (4 * g), mag);
#pragma unroll
        for (int i = 0; i < G2_FM; ++i) acc[j][i] = mfma16x16x32(sf, xf[i], acc[j][i]);
      }
    }
  };

  // Stages in pairs: A (even) then B (odd).  Each half first issues the next
  // stage's loads (two side loads, then 16 DMAs), then waits until only those
  // are outstanding, i.e. until its own stage's DMA has landed.  The second
  // half always prefetches stage kt+2 (clamped): for an odd stage count that
  // is the final stage, computed after the loop; otherwise it is unused.
  int64_t kt = 0;
  for (; kt + 1 < G.nk; kt += 2) {
    G.load_side(kt + 1);
    G.dma(xb, kt + 1);
    OBL_WAIT_VMCNT(kIssued);
    lds_barrier();                      // stage kt visible to all
    compute(xa, wsa, maga);
    G.store_side(wsb, magb);
    lds_barrier();                      // everyone is done with A and side A
    G.load_side(kt + 2);
    G.dma(xa, kt + 2);
    OBL_WAIT_VMCNT(kIssued);
    lds_barrier();
    compute(xb, wsb, magb);
    G.store_side(wsa, maga);
    lds_barrier();
  }
  if (kt < G.nk) {                      // odd number of stages: the last one is in A
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    compute(xa, wsa, maga);
  }
  __builtin_amdgcn_s_waitcnt(0);        // no DMA may still target LDS when the block ends

  // Epilogue: acc[j][i][r] = Y[row m0 + xrow0 + 16 i][col n0 + 112 wn + 16 j + 4 g + r].
#pragma unroll
  for (int i = 0; i < G2_FM; ++i) {
    const int64_t m = G.m0 + xrow0 + 16 * i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < G2_FN; ++j) {
      const int cl = wn * (G2_FN * 16) + j * 16 + 4 * g;   // column within the tile
      const int64_t n = G.n0 + cl;
      YT* yp = Y + m * N + n;
      const float v0 = acc[j][i][0] * post_s[cl + 0], v1 = acc[j][i][1] * post_s[cl + 1];
      const float v2 = acc[j][i][2] * post_s[cl + 2], v3 = acc[j][i][3] * post_s[cl + 3];
      if (n + 3 < N && (reinterpret_cast<uintptr_t>(yp) & (4 * sizeof(YT) - 1)) == 0) {
        if constexpr (sizeof(YT) == 2) {
          *reinterpret_cast<u32x2*>(yp) = u32x2{pack_bf16_pair(v0, v1), pack_bf16_pair(v2, v3)};
        } else {
          *reinterpret_cast<f32x4*>(yp) = f32x4{v0, v1, v2, v3};
        }
      } else {
        if (n + 0 < N) Store<YT>::put(yp + 0, v0);
        if (n + 1 < N) Store<YT>::put(yp + 1, v1);
        if (n + 2 < N) Store<YT>::put(yp + 2, v2);
        if (n + 3 < N) Store<YT>::put(yp + 3, v3);
      }
    }
  }
}

template <typename ST, typename YT, bool PRE>
hipError_t launch_bf16(const LinearArgs& a) {
  const int64_t mt = (a.M + G2_BM - 1) / G2_BM;
  const int64_t nt = (a.N + G2_BN - 1) / G2_BN;
  const int64_t tiles = mt * nt;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const int xcd = (tiles % 8 == 0) ? 8 : 1;
  hipLaunchKernelGGL((gemm_bf16_kernel<ST, YT, PRE>), dim3((unsigned)tiles), dim3(G2_THREADS), 0, a.stream,
                     static_cast<const bf16_t*>(a.X), a.M, a.K, a.W, a.N, static_cast<const ST*>(a.pre),
                     static_cast<const ST*>(a.post), static_cast<YT*>(a.Y), (int)mt, (int)nt, xcd);
  return hipGetLastError();
}

template <int AMODE, typename XT, typename ST, typename YT, bool PRE>
hipError_t launch_t(const LinearArgs& a, const DeviceInfo&) {
  const int64_t mt = (a.M + GM_BM - 1) / GM_BM;
  const int64_t nt = (a.N + GM_BN - 1) / GM_BN;
  const int64_t tiles = mt * nt;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const int xcd = (tiles % 8 == 0) ? 8 : 1;
  hipLaunchKernelGGL((gemm_mfma_kernel<AMODE, XT, ST, YT, PRE>), dim3((unsigned)tiles),
                     dim3(GM_THREADS), 0, a.stream, static_cast<const XT*>(a.X), a.M, a.K, a.W, a.N,
                     static_cast<const ST*>(a.pre), static_cast<const ST*>(a.post),
                     static_cast<YT*>(a.Y), (int)mt, (int)nt, xcd);
  return hipGetLastError();
}

// The test suite can force the 8-wave or the LDS-staged kernel
// (forced_kernels().gemm 1 / 2) to compare them with the default choice.
int gemm_forced() {
  const int f = forced_kernels().gemm;
  return (f == 1 || f == 2) ? f : 0;
}

template <typename ST, typename YT>
hipError_t launch_mode(const LinearArgs& a, const DeviceInfo& dev) {
  // bf16 activations (8-byte aligned rows): A = x exactly, and the input-side
  // scale, if any, is folded into B as bf16(b).  Otherwise A is converted once
  // per staged element: bf16(x·b) or bf16(x).
  // Main kernel: bf16 x and packed words 16-byte aligned, K % 128 == 0, b
  // absent or fp16 and 16-byte aligned.  Everything else runs the 8-wave kernel.
  const bool v2 = a.x_dtype == DT_BF16 && (reinterpret_cast<uintptr_t>(a.X) % 16 == 0) &&
                  (reinterpret_cast<uintptr_t>(a.W) % 16 == 0) && a.K % G2_KT == 0 &&
                  (!a.pre || (a.scale_dtype == DT_F16 && reinterpret_cast<uintptr_t>(a.pre) % 16 == 0));
  const int forced = gemm_forced();
  if (forced == 0 && gemm_wide_eligible(a)) return launch_gemm_wide(a, dev);
  if (forced == 0 && gemm_wide_prescale_eligible(a)) return launch_gemm_wide_prescaled(a, dev);
  if (a.Y2) return hipErrorInvalidValue;   // only the wide kernel writes the bf16 copy
  if (v2 && forced != 1) {
    if constexpr (std::is_same<ST, f16_t>::value) {
      if (a.pre) return launch_bf16<ST, YT, true>(a);
    }
    if (!a.pre) return launch_bf16<ST, YT, false>(a);
  }
  const bool raw = a.x_dtype == DT_BF16 && (reinterpret_cast<uintptr_t>(a.X) % 8 == 0);
  if (raw) return a.pre ? launch_t<A_RAW, bf16_t, ST, YT, true>(a, dev)
                        : launch_t<A_RAW, bf16_t, ST, YT, false>(a, dev);
  if (a.x_dtype == DT_BF16) return a.pre ? launch_t<A_CONVERT, bf16_t, ST, YT, true>(a, dev)
                                         : launch_t<A_CONVERT, bf16_t, ST, YT, false>(a, dev);
  return a.pre ? launch_t<A_CONVERT, float, ST, YT, true>(a, dev)
               : launch_t<A_CONVERT, float, ST, YT, false>(a, dev);
}
template <typename ST>
hipError_t launch_y(const LinearArgs& a, const DeviceInfo& dev) {
  return a.y_dtype == DT_F32 ? launch_mode<ST, float>(a, dev) : launch_mode<ST, bf16_t>(a, dev);
}

}  // namespace

void gemm_scratch(const LinearArgs& a, const DeviceInfo& dev, ScratchNeed* need) {
  // The same order of choices as launch_mode: only the main kernel (split K)
  // and its prescaled route use scratch.
  if (gemm_forced() != 0) return;
  if (gemm_wide_eligible(a)) gemm_wide_scratch(a, dev, need);
  else if (gemm_wide_prescale_eligible(a)) gemm_wide_prescaled_scratch(a, dev, need);
}

hipError_t launch_gemm_mfma(const LinearArgs& a, const DeviceInfo& dev) {
  return a.scale_dtype == DT_F32 ? launch_y<float>(a, dev) : launch_y<f16_t>(a, dev);
}

}  // namespace obl
