// Main prefill kernel for M > 16 with bf16 activations:
// Y = ((X ⊙ b) W_sign^T) ⊙ a on v_mfma_f32_32x32x16_bf16, fp32 accumulation.
//
// OneBit page ("1bit量化"), proposition 1: for M > 16 the sign-binarised layer
// is a dense contraction (2·M·N·K flops), so it belongs on the matrix cores.
//
// Why 32x32x16 and one wave per SIMD.  On gfx950 a single wave issuing
// independent 16x16x32 MFMAs keeps the matrix pipe only ~60% busy, while
// 32x32x16 MFMAs (32 cycles each) reach ~90% from one wave and tolerate about
// four VALU ops per MFMA at ~80%.  One wave per SIMD leaves the whole
// 512-entry register file to it: 224 fp32 accumulators in AGPRs plus the
// operand stages in VGPRs.
//
// Tiling: 4 waves as 2 (rows) x 2 (columns), 64 x 224 outputs per wave
// (2 x 7 fragments of 32 x 32), so a workgroup owns 128 x 448 outputs.  For
// M = 2048, N = 14336 that is 16 x 32 = 512 tiles: exactly two per CU on 256
// CUs.  Tiles are ordered so each XCD (blockIdx % 8) takes a contiguous range
// that walks all column tiles of two row tiles: its L2 then serves one
// 128-row activation block to 32 workgroups at a time.
//
// Operands, per 16-k step (MFMA A = signs, B = activations):
//  * Activations: each 128-k stage of the workgroup's 128 rows is copied
//    global -> LDS by DMA (buffer_load_dwordx4 ... lds, 1 KiB per
//    instruction, fully coalesced), XOR-swizzled so that the MFMA-layout
//    reads -- lane (row r = lane % 32, half g = lane / 32) takes
//    x[r][16s + 8g .. 16s + 8g + 7], natural k order -- are one conflict-free
//    ds_read_b128 each.  Loading straight into registers in MFMA layout
//    touches 32 rows per instruction and costs the texture path ~4x more.
//  * Signs: the stage's 4 packed words (16 bytes) per column also arrive by
//    DMA; each wave reads its 7 columns' words once per stage.  A dword of
//    the operand holds the pair (k, k+1); its two sign bits sit side by side
//    in one 16-bit half of a word.  One packed 16-bit shift
//    (v_pk_lshlrev_b16, both result halves fed from the same source half)
//    moves bit k to bit 15 and bit k+1 to bit 31, and one v_bitop3 masks them
//    and applies them to the magnitudes: two VALU ops per two weights, with
//    no bit shuffling of the packed words.
//  * Magnitudes: bf16(b_k) pairs (or 1.0 without b), converted once per
//    workgroup into an LDS table at kernel start, one ds_read_b128 per step.
//  * Three stage buffers, one barrier per stage: stages t + 1 and t + 2 are
//    in flight while stage t is computed (two stages of latency cover the
//    misses of the streamed sign words, one line per column per 8 stages).
//  * The sign operands of k-step s + 1 are expanded between the MFMAs of
//    step s, into registers of their own, and the barrier sits inside the
//    last k-step of a stage, so the next stage's step-0 operands are
//    expanded under that step's MFMAs.  With one operand register set reused
//    for all columns (the compiler's choice) expansion and MFMAs ran one
//    after the other: 2048 x 4096 x 14336 took 210 us, 192-197 us now.  The
//    expansion is still ~13 % of the kernel's time (measured by removing
//    it); the clock then runs at ~1.5 GHz, power-limited.
//  * Out-of-range rows / columns re-read the last valid one and are not
//    stored; every load is unconditional.
//  * Epilogue: acc·a in fp32 (a staged in LDS), one cast to the output dtype.
//    A lane holds four consecutive output columns per register quad, written
//    as one 16-byte (fp32) or 8-byte (bf16) store.
//  * Small grids first take smaller tiles (64 x 128 when that grid fits the
//    CUs once: M = 512, N = 3072 is 192 tiles, whole K each), and a grid
//    still at most half as many tiles as CUs splits K: tiles x slices fill
//    the CUs once, each slice writes fp32 partial sums and a second kernel
//    adds the slices in order (fixed order: reproducible; accumulation stays
//    fp32).  Measured on 512 x 4096 x 3072 with the 448-wide tile (28 tiles):
//    8 slices of 4 stages, ~31 us for the split kernel and ~11 us for the
//    reduction, against ~99 us unsplit.  The split kernel's fixed cost is the
//    burst of partial sums written when every workgroup ends together and
//    the reduction reading them back; more slices of fewer stages stop
//    paying at about 8.
#include <algorithm>
#include <type_traits>

#include "obl_common.hpp"
#include "obl_internal.hpp"

namespace obl {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int GW_THREADS = 256;
constexpr int GW_WM = 64;         // wave rows
constexpr int GW_FM = GW_WM / 32; // 2 activation fragments
constexpr int GW_KT = 128;        // k per stage
constexpr int GW_S = GW_KT / 16;  // MFMA k-steps per stage

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Sign operand of one k-step from the 16-bit half `h` of a packed word:
// dword j covers the pair (2j + 8g, 2j + 8g + 1) of that half, whose sign
// bits go to bits 15 and 31 by the per-lane shift pair sh[j].  The four
// shifts are pinned (empty asm, registers only) ahead of the four masks:
// issued shift, mask, shift, mask the compiler put an s_nop between each
// dependent pair (914 in the 448-wide kernel, 275 this way); 2048 x 4096 x
// 14336 192.2 -> 188.1 us on the same box.
__device__ __forceinline__ u32x4 expand_half(uint32_t h, const u16x2* sh, u32x4 mag) {
  const u16x2 d = u16x2{(unsigned short)h, (unsigned short)h};
  uint32_t t0 = __builtin_bit_cast(uint32_t, d << sh[0]);
  uint32_t t1 = __builtin_bit_cast(uint32_t, d << sh[1]);
  uint32_t t2 = __builtin_bit_cast(uint32_t, d << sh[2]);
  uint32_t t3 = __builtin_bit_cast(uint32_t, d << sh[3]);
  asm volatile("" : "+v"(t0), "+v"(t1), "+v"(t2), "+v"(t3));
  u32x4 r;
  r.x = (t0 & 0x80008000u) ^ mag.x;
  r.y = (t1 & 0x80008000u) ^ mag.y;
  r.z = (t2 & 0x80008000u) ^ mag.z;
  r.w = (t3 & 0x80008000u) ^ mag.w;
  return r;
}

constexpr int GW_BTAB_BATCH = 8 * GW_THREADS;             // bf16(b) pairs per table-fill batch
constexpr double GW_EFF4 = 1.08;                          // per-column cost of the 256-wide tile vs the 448-wide

// Tiling.  Every wave owns 64 rows (two 32-row activation fragments) and FN
// sign fragments of 32 columns; the four waves stand WR = 2 (rows) x 2
// (columns) or WR = 1 x 4.  FN = 7, WR = 2: 64 x 224 wave tiles, 128 x 448
// workgroup tile; FN = 4: 128 x 256; FN = 2: 128 x 128; FN = 1, WR = 1: 64 x
// 32 wave tiles side by side, a 64 x 128 workgroup tile (for grids that the
// 128-row tiles leave short of the CUs).  Sign columns are staged in whole
// 256-column DMA rounds (one 16-byte DMA per lane per round; the 128-wide
// tiles use half of it).
template <int FN, int WR = 2> struct GwTile {
  static constexpr int WN = 32 * FN;                      // wave columns
  static constexpr int BM = 64 * WR;                      // workgroup rows
  static constexpr int BN = WN * (4 / WR);                // workgroup columns
  static constexpr int WCOLS = (BN + 255) / 256 * 256;    // sign columns staged
  static constexpr int WDMA = WCOLS / 256;                // sign DMAs per wave per stage
  static constexpr int XDMA = BM * (GW_KT / 8) / 64 / 4;  // activation DMAs per wave per stage
  static_assert(WR == 1 || WR == 2, "wave rows");
  static_assert(BN <= 2 * GW_THREADS, "two output scales per thread");
};

// Entries of the bf16(b) pair table: K / 2 rounded up to whole fill batches.
inline int64_t gw_btab_entries(int64_t K) {
  return (K / 2 + GW_BTAB_BATCH - 1) / GW_BTAB_BATCH * GW_BTAB_BATCH;
}

// SPLIT: block b takes tile b / nsplit and the 128-k stages
// [s·per, min((s + 1)·per, K/128)) of slice s = b % nsplit, and writes its raw
// fp32 sums (no output scale) to part[s][M][N]; gemm_split_reduce_kernel adds
// the slices in order.
template <typename ST, typename YT, bool PRE, bool SPLIT, int FN, int WR>
__global__ __launch_bounds__(GW_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_wide_kernel(const bf16_t* __restrict__ X, int64_t M, int64_t K, const uint32_t* __restrict__ W,
                      int64_t N, const ST* __restrict__ pre, const ST* __restrict__ post,
                      YT* __restrict__ Y, bf16_t* __restrict__ Y2, int mt, int nt, int xcd_groups,
                      int nsplit, int per, float* __restrict__ part) {
  using TL = GwTile<FN, WR>;
  constexpr int GW_WN = TL::WN, GW_BN = TL::BN, GW_FN = FN, GW_BM = TL::BM;
  constexpr int GW_WCOLS = TL::WCOLS, GW_WDMA = TL::WDMA, GW_XDMA = TL::XDMA;
  // Three stage buffers as distinct LDS objects: the K loop is unrolled by
  // three so every access names its buffer, and the compiler can tell a DMA
  // into one buffer from reads of another.
  __shared__ u32x4 xa[GW_BM][GW_KT / 8];     // activations: row, 16-byte slot (swizzled)
  __shared__ u32x4 xb[GW_BM][GW_KT / 8];
  __shared__ u32x4 xc[GW_BM][GW_KT / 8];
  __shared__ u32x4 wa[GW_WCOLS];             // 4 packed words (128 k) per column
  __shared__ u32x4 wb[GW_WCOLS];
  __shared__ u32x4 wc[GW_WCOLS];
  __shared__ float post_s[2 * GW_THREADS];   // GW_BN used
  extern __shared__ uint32_t btab[];         // [gw_btab_entries(K)] bf16(b) pairs (with b only)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS DMA bases stay scalar
  const int wm = WR == 2 ? (wave & 1) : 0, wn = WR == 2 ? (wave >> 1) : wave;
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const int64_t kw = K >> 5;
  const int nk_all = (int)(K / GW_KT);
  const int tiles = mt * nt;
  const int slice = SPLIT ? (int)(blockIdx.x % (unsigned)nsplit) : 0;
  const int t0 = SPLIT ? slice * per : 0;                  // first stage of this block
  const int nk = SPLIT ? min(per, nk_all - t0) : nk_all;   // stages of this block (>= 1)
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)(M * K * 2));
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W, (uint32_t)(N * kw * 4));


  // Shift pairs: dword j of half-group g takes bits 8g + 2j (-> 15) and
  // 8g + 2j + 1 (-> 31) of a 16-bit half.
  u16x2 sh[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    sh[j] = u16x2{(unsigned short)(15 - 8 * g - 2 * j), (unsigned short)(14 - 8 * g - 2 * j)};
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const u32x4* bt4 = reinterpret_cast<const u32x4*>(btab);
  const int xrow = wm * GW_WM + l32;       // + 32 i
  const int wcol = wn * GW_WN + l32;       // + 32 c

  // XCD x (= blockIdx % 8) takes tiles [x·T/8, (x+1)·T/8), column index fastest.
  int lin = SPLIT ? (int)(blockIdx.x / (unsigned)nsplit) : (int)blockIdx.x;
  if (!SPLIT && xcd_groups > 1) {
    const int per = tiles / xcd_groups;
    lin = (blockIdx.x % xcd_groups) * per + blockIdx.x / xcd_groups;
  }
  const int tm = lin / nt, tn = lin - (lin / nt) * nt;
  const int64_t bm0 = (int64_t)tm * GW_BM, bn0 = (int64_t)tn * GW_BN;

  // DMA offsets (bytes, < 2^32: checked by the launcher), fixed across stages.
  // Activation DMA i of wave w fills rows 4(8w + i) .. +3 of the tile; lane l
  // takes row + l/16 and LDS slot l % 16, i.e. global 16-byte chunk
  // (l % 16) ^ (row % 16): chunk c of row r sits at slot c ^ (r % 16), so the
  // 16 rows read by a half-wave fall on 16 different slots.  Rows past M
  // re-read row M - 1, columns past N column N - 1 (never stored).
  uint32_t xo[GW_XDMA], wo[GW_WDMA];
#pragma unroll
  for (int i = 0; i < GW_XDMA; ++i) {
    const int row = 4 * (GW_XDMA * wave + i) + (lane >> 4);
    const int64_t r = min(bm0 + row, M - 1);
    xo[i] = (uint32_t)((r * K + 8 * ((lane & 15) ^ (row & 15))) * 2);
  }
#pragma unroll
  for (int j = 0; j < GW_WDMA; ++j) {
    const int64_t n = min(bn0 + 64 * (GW_WDMA * wave + j) + lane, N - 1);
    wo[j] = (uint32_t)(n * kw * 4);
  }
  auto dma = [&](u32x4 (*xs)[GW_KT / 8], u32x4* ws, int t) {
#pragma unroll
    for (int i = 0; i < GW_XDMA; ++i)
      dma16(xr, &xs[4 * (GW_XDMA * wave + i)][0], xo[i], (uint32_t)(t0 + t) * (GW_KT * 2));
#pragma unroll
    for (int j = 0; j < GW_WDMA; ++j) dma16(wr, &ws[64 * (GW_WDMA * wave + j)], wo[j], (uint32_t)(t0 + t) * 16);
  };

  dma(xa, wa, 0);
  dma(xb, wb, min(1, nk - 1));

  // Output scales of this tile (loads issued now, stored below), then the
  // bf16(b) table, all while stages 0 and 1 are in flight.
  float ps0 = 1.f, ps1 = 1.f;
  if constexpr (!SPLIT) {
    ps0 = scale_or_one(post, min(bn0 + tid, N - 1), W);
    ps1 = scale_or_one(post, min(bn0 + tid + GW_THREADS, N - 1), W);
  }

  // The table is filled after the stage DMAs are issued: the CU returns
  // loads in issue order, so waiting for its inputs also covers the two
  // stages (one round trip for both).  All loads of a batch are issued before
  // any is used, and the stores are unconditional (the table is padded to
  // whole batches, see gw_btab_entries): a store under a branch takes its
  // load into the branch, where it is waited for at once.
  if constexpr (PRE) {
    const int64_t npair = K / 2;
    for (int64_t p0 = 0; p0 < npair; p0 += GW_BTAB_BATCH) {
      float lo[8], hi[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t pc = min(p0 + u * GW_THREADS + tid, npair - 1);
        lo[u] = to_f32(pre[2 * pc]);
        hi[u] = to_f32(pre[2 * pc + 1]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) btab[p0 + u * GW_THREADS + tid] = pack_bf16_pair(lo[u], hi[u]);
    }
  }

  if constexpr (!SPLIT) {                  // padded: GW_BN <= 2 * GW_THREADS
    post_s[tid] = ps0;
    post_s[tid + GW_THREADS] = ps1;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): stages 0 and 1 landed
  __syncthreads();

  f32x16 acc[GW_FN][GW_FM];
#pragma unroll
  for (int c = 0; c < GW_FN; ++c)
#pragma unroll
    for (int i = 0; i < GW_FM; ++i) acc[c][i] = f32x16{};

  // Operand registers.  wv: the current stage's packed sign words (128 k per
  // column); mr: bf16(b) pair quads of two k-steps (by step parity); xf:
  // activation fragments of two k-steps; av: sign operands of two k-steps.
  // Operands of step s + 1 are formed while the MFMAs of step s run, into
  // registers of their own: the expansion of a k-step then costs no
  // matrix-core time.
  u32x4 wv[GW_FN], mr[2], xf[2][GW_FM], av[2][GW_FN];
  auto half = [&](int c, int s) -> uint32_t {
    const uint32_t word = wv[c][s >> 1];
    return (s & 1) ? (word >> 16) : (word & 0xFFFFu);
  };
  // Magnitudes of k-step s (possibly past the stage's last) of stage t.  The
  // table is static, so they are read two k-steps ahead of their use; the
  // stage is clamped to the block's last.
  auto mag = [&](int t, int s) -> u32x4 {
    if constexpr (!PRE) return ones;
    const int ts = min(t + s / GW_S, nk - 1);
    return bt4[((t0 + ts) * GW_KT + 16 * (s % GW_S) + 8 * g) >> 3];
  };
  // The MFMAs of column fragment c at k-step s (operand set b), with the
  // expansion of another operand (column cn of step sn, into set bn, with the
  // magnitudes mr[sn & 1]) between the first and the second.
  auto group = [&](int b, int c, bool expand, int bn, int cn, int sn) {
    acc[c][0] = mfma32(av[b][c], xf[b][0], acc[c][0]);
    if (expand) av[bn][cn] = expand_half(half(cn, sn), sh, mr[sn & 1]);
#pragma unroll
    for (int i = 1; i < GW_FM; ++i) acc[c][i] = mfma32(av[b][c], xf[b][i], acc[c][i]);
  };
  // Issue order of a k-step: MFMA, 4 VALU, MFMA, 4 VALU per column fragment.
  auto interleave = [&](int groups) {
#pragma unroll
    for (int c = 0; c < groups; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, GW_FM - 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
  };

  // One stage: k-steps 0..6 read the activations of the next step and the
  // magnitudes of the step after, issue their share of the DMAs of stage
  // t + 2 (into the buffer stage t - 1 used) and run their MFMAs with the
  // next step's sign operands expanded in between.  Step 7 waits for this
  // wave's DMAs of stage t + 1 (all but the GW_XDMA + GW_WDMA most recent
  // transfers) and for its LDS reads, issues the first column's MFMAs, meets
  // the other waves at the barrier (which publishes stage t + 1 and retires
  // stage t's buffer), then reads stage t + 1's sign words and first
  // activations and expands its step-0 signs under the remaining MFMAs.
  // Prefetch indices are clamped: a redundant reload of the last stage into
  // an idle buffer is harmless, and so is reading it.
  auto step = [&](u32x4 (*xs)[GW_KT / 8], u32x4 (*xn)[GW_KT / 8], const u32x4* wn_, u32x4 (*xp)[GW_KT / 8],
                  u32x4* wp, int t) {
    const uint32_t tn = (uint32_t)(t0 + min(t + 2, nk - 1));
#pragma unroll
    for (int s = 0; s + 1 < GW_S; ++s) {
      const int b = s & 1;
#pragma unroll
      for (int i = 0; i < GW_FM; ++i) xf[b ^ 1][i] = xs[xrow + 32 * i][(2 * (s + 1) + g) ^ (lane & 15)];
      mr[b] = mag(t, s + 2);
      __builtin_amdgcn_sched_barrier(0);
      // This step's DMAs: activation transfers s, s + 7, ..., then sign
      // transfer s.  Transfer d goes with column group d % GW_FN, in a
      // scheduling region of its own, so the ~40 cycles a DMA holds the wave
      // overlap that group's MFMAs rather than stacking up in front of one.
      const int nx = s < GW_XDMA ? (GW_XDMA - 1 - s) / (GW_S - 1) + 1 : 0;
      const int nd = nx + (s < GW_WDMA ? 1 : 0);
#pragma unroll
      for (int c = 0; c < GW_FN; ++c) {
        group(b, c, true, b ^ 1, c, s + 1);
#pragma unroll
        for (int d = c; d < nd; d += GW_FN) {
          if (d < nx) dma16(xr, &xp[4 * (GW_XDMA * wave + s + (GW_S - 1) * d)][0], xo[s + (GW_S - 1) * d],
                            tn * (GW_KT * 2));
          else dma16(wr, &wp[64 * (GW_WDMA * wave + s)], wo[s], tn * 16);
        }
        interleave(1);
        if (c < nd) __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    constexpr int bl = (GW_S - 1) & 1;
    __builtin_amdgcn_s_waitcnt(0x0070 | (GW_XDMA + GW_WDMA));   // vmcnt(n) lgkmcnt(0)
    group(bl, 0, false, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < GW_FN; ++c) wv[c] = wn_[wcol + 32 * c];
#pragma unroll
    for (int i = 0; i < GW_FM; ++i) xf[0][i] = xn[xrow + 32 * i][g ^ (lane & 15)];
    mr[1] = mag(t, GW_S + 1);
#pragma unroll
    for (int c = 1; c < GW_FN; ++c) group(bl, c, true, 0, c - 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, GW_FN + GW_FM + 1, 0);
    interleave(GW_FN - 1);
    __builtin_amdgcn_sched_barrier(0);
    av[0][GW_FN - 1] = expand_half(half(GW_FN - 1, 0), sh, mr[0]);
    __builtin_amdgcn_sched_barrier(0);
  };
  static_assert(GW_XDMA + GW_WDMA < 16, "vmcnt immediate");
  static_assert(GW_WDMA <= GW_S - 1, "every sign DMA of a stage has a k-step to go with");

#pragma unroll
  for (int c = 0; c < GW_FN; ++c) wv[c] = wa[wcol + 32 * c];
#pragma unroll
  for (int i = 0; i < GW_FM; ++i) xf[0][i] = xa[xrow + 32 * i][g ^ (lane & 15)];
  mr[0] = mag(0, 0);
  mr[1] = mag(0, 1);
#pragma unroll
  for (int c = 0; c < GW_FN; ++c) av[0][c] = expand_half(half(c, 0), sh, mr[0]);
  int t = 0;
  for (; t + 3 <= nk; t += 3) {
    step(xa, xb, wb, xc, wc, t);
    step(xb, xc, wc, xa, wa, t + 1);
    step(xc, xa, wa, xb, wb, t + 2);
  }
  if (t < nk) step(xa, xb, wb, xc, wc, t);
  if (t + 1 < nk) step(xb, xc, wc, xa, wa, t + 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);     // no DMA may still target LDS when the block ends

  // Epilogue.  acc[c][i][4q + e] = D[row n = 8q + 4g + e][col m = l32] of the
  // (c, i) fragment, i.e. Y[m0 + 32i + l32][n0 + 32c + 8q + 4g + e].
  const int64_t m0 = bm0 + wm * GW_WM;
  if constexpr (SPLIT) {
    float* pp = part + (int64_t)slice * M * N;
#pragma unroll
    for (int i = 0; i < GW_FM; ++i) {
      const int64_t m = m0 + 32 * i + l32;
      if (m >= M) continue;
#pragma unroll
      for (int c = 0; c < GW_FN; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = bn0 + wn * GW_WN + 32 * c + 8 * q + 4 * g;
          float* yp = pp + m * N + n;
          const float v[4] = {acc[c][i][4 * q], acc[c][i][4 * q + 1], acc[c][i][4 * q + 2], acc[c][i][4 * q + 3]};
          if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<f32x4*>(yp) = f32x4{v[0], v[1], v[2], v[3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) yp[e] = v[e];
          }
        }
    }
    return;
  }
  // bf16 output (the prefill case) through LDS: written straight from the
  // accumulators, a wave instruction covers 32 rows with 16 bytes each, and
  // the store requests of every workgroup ending together measured ~10 % of
  // the kernel (2048 x 4096 x 14336).  Each wave instead stages one 32-row
  // fragment of its tile at a time in its own part of the idle stage buffers
  // and stores whole row segments, consecutive lanes on consecutive 16 bytes.
  if constexpr (std::is_same<YT, bf16_t>::value) {
    if (!Y2 && (N & 7) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0) {
      constexpr int RB = GW_WN * 2 + 16;           // bytes per staged row (16 bytes of padding)
      constexpr int C16 = GW_WN / 8;               // 16-byte chunks per row
      static_assert(2 * 32 * RB <= (int)sizeof(xa), "two waves' fragments fit one stage buffer");
      __syncthreads();                             // every wave is done with the stage buffers
      unsigned char* tile = reinterpret_cast<unsigned char*>(wave < 2 ? &xa[0][0] : &xb[0][0]) + (wave & 1) * 32 * RB;
#pragma unroll
      for (int i = 0; i < GW_FM; ++i) {
#pragma unroll
        for (int c = 0; c < GW_FN; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cl = wn * GW_WN + 32 * c + 8 * q + 4 * g;
            const f32x4 ps = *reinterpret_cast<const f32x4*>(post_s + cl);
            *reinterpret_cast<u32x2*>(tile + l32 * RB + (32 * c + 8 * q + 4 * g) * 2) =
                u32x2{pack_bf16_pair(acc[c][i][4 * q] * ps.x, acc[c][i][4 * q + 1] * ps.y),
                      pack_bf16_pair(acc[c][i][4 * q + 2] * ps.z, acc[c][i][4 * q + 3] * ps.w)};
          }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < 32 * C16 / 64; ++k) {
          const int ch = lane + 64 * k;
          const int row = ch / C16, c16 = ch - (ch / C16) * C16;
          const u32x4 v = *reinterpret_cast<const u32x4*>(tile + row * RB + c16 * 16);
          const int64_t m = m0 + 32 * i + row, n = bn0 + wn * GW_WN + 8 * c16;
          if (m < M && n < N) *reinterpret_cast<u32x4*>(Y + m * N + n) = v;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < GW_FM; ++i) {
    const int64_t m = m0 + 32 * i + l32;
    if (m >= M) continue;
#pragma unroll
    for (int c = 0; c < GW_FN; ++c) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = wn * GW_WN + 32 * c + 8 * q + 4 * g;      // column within the workgroup tile
        const int64_t n = bn0 + cl;
        const f32x4 ps = *reinterpret_cast<const f32x4*>(post_s + cl);
        const float v0 = acc[c][i][4 * q + 0] * ps.x, v1 = acc[c][i][4 * q + 1] * ps.y;
        const float v2 = acc[c][i][4 * q + 2] * ps.z, v3 = acc[c][i][4 * q + 3] * ps.w;
        YT* yp = Y + m * N + n;
        if (Y2) {
          // bf16 copy of the same fp32 results (the next DBF stage's operand).
          bf16_t* y2 = Y2 + m * N + n;
          if (n + 3 < N && (reinterpret_cast<uintptr_t>(y2) & 7) == 0) {
            *reinterpret_cast<u32x2*>(y2) = u32x2{pack_bf16_pair(v0, v1), pack_bf16_pair(v2, v3)};
          } else {
            if (n + 0 < N) Store<bf16_t>::put(y2 + 0, v0);
            if (n + 1 < N) Store<bf16_t>::put(y2 + 1, v1);
            if (n + 2 < N) Store<bf16_t>::put(y2 + 2, v2);
            if (n + 3 < N) Store<bf16_t>::put(y2 + 3, v3);
          }
        }
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
}

// Y[m][n] = (Σ_s part[s][m][n]) · post[n] with the slices added in order,
// plus the optional bf16 copy Y2.  Four consecutive outputs per thread when
// N % 4 == 0, else one.
template <typename ST, typename YT, int V>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(const float* __restrict__ part, int nsplit,
                                                                int64_t MN, int64_t N, const ST* __restrict__ post,
                                                                YT* __restrict__ Y, bf16_t* __restrict__ Y2) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
  if (e0 >= MN) return;
  const int64_t n0 = e0 % N;
  float sc[V], acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    sc[e] = scale_or_one(post, n0 + e, part);   // part: >= MN floats; issued before the partial loads
    acc[e] = 0.f;
  }
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float p[8][V];
    bool ok[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      ok[r] = s0 + r < nsplit;
      const float* src = part + (int64_t)(ok[r] ? s0 + r : 0) * MN + e0;
      if constexpr (V == 4) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(src);
        p[r][0] = t.x; p[r][1] = t.y; p[r][2] = t.z; p[r][3] = t.w;
      } else {
        p[r][0] = src[0];
      }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += ok[r] ? p[r][e] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const float y = acc[e] * sc[e];
    Store<YT>::put(&Y[e0 + e], y);
    if (Y2) Store<bf16_t>::put(&Y2[e0 + e], y);
  }
}

// Split count: small grids (fewer tiles than CUs; the kernel runs one
// workgroup per CU) split K so that tiles · nsplit fills the CUs once, with at
// least 4 stages per slice so the three-buffer pipeline still overlaps.
int split_count(int64_t tiles, int64_t nk, int num_cus) {
  if (tiles * 2 > num_cus) return 1;
  int64_t s = num_cus / tiles;
  s = std::min<int64_t>(s, nk / 4);
  s = std::min<int64_t>(s, 16);
  return (int)std::max<int64_t>(s, 1);
}

// K-slices of a grid of `tiles` tiles (1: no split) and k-stages per slice.
int split_plan(int64_t tiles, int64_t nk, int num_cus, int* per) {
  int nsplit = split_count(tiles, nk, num_cus);
  *per = (int)((nk + nsplit - 1) / nsplit);
  return (int)((nk + *per - 1) / *per);                     // every slice non-empty
}

template <typename ST, typename YT, bool PRE, int FN, int WR>
hipError_t launch_fn(const LinearArgs& a, const DeviceInfo& dev) {
  constexpr int BN = GwTile<FN, WR>::BN, BM = GwTile<FN, WR>::BM;
  const int64_t mt = (a.M + BM - 1) / BM;
  const int64_t nt = (a.N + BN - 1) / BN;
  const int64_t tiles = mt * nt;
  const int64_t nk = a.K / GW_KT;
  const size_t lds = (PRE ? gw_btab_entries(a.K) : 0) * sizeof(uint32_t);
  int per = 0;
  const int nsplit = split_plan(tiles, nk, dev.num_cus, &per);
  if (nsplit > 1) {
    float* part = a.sx ? a.sx->get(1, (size_t)nsplit * (size_t)(a.M * a.N)) : nullptr;
    if (!part) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_wide_kernel<ST, float, PRE, true, FN, WR>), dim3((unsigned)(tiles * nsplit)),
                       dim3(GW_THREADS), lds, a.stream, static_cast<const bf16_t*>(a.X), a.M, a.K, a.W, a.N,
                       static_cast<const ST*>(a.pre), static_cast<const ST*>(a.post), nullptr, nullptr, (int)mt,
                       (int)nt, 1, nsplit, per, part);
    const int64_t MN = a.M * a.N;
    if (a.N % 4 == 0)
      hipLaunchKernelGGL((gemm_split_reduce_kernel<ST, YT, 4>), dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256),
                         0, a.stream, part, nsplit, MN, a.N, static_cast<const ST*>(a.post), static_cast<YT*>(a.Y),
                         static_cast<bf16_t*>(a.Y2));
    else
      hipLaunchKernelGGL((gemm_split_reduce_kernel<ST, YT, 1>), dim3((unsigned)((MN + 255) / 256)), dim3(256), 0,
                         a.stream, part, nsplit, MN, a.N, static_cast<const ST*>(a.post), static_cast<YT*>(a.Y),
                         static_cast<bf16_t*>(a.Y2));
    return hipGetLastError();
  }
  const int xcd = (tiles % 8 == 0) ? 8 : 1;
  hipLaunchKernelGGL((gemm_wide_kernel<ST, YT, PRE, false, FN, WR>), dim3((unsigned)tiles), dim3(GW_THREADS), lds,
                     a.stream, static_cast<const bf16_t*>(a.X), a.M, a.K, a.W, a.N,
                     static_cast<const ST*>(a.pre), static_cast<const ST*>(a.post),
                     static_cast<YT*>(a.Y), static_cast<bf16_t*>(a.Y2), (int)mt, (int)nt, xcd, 1, 0, nullptr);
  return hipGetLastError();
}

// Tile.  A grid that would split K with the 128 x 256 tile takes the 64 x 128
// tile when that grid fits one workgroup per CU (no split at all at M = 512,
// N = 3072 or 4096), else the 128 x 128 tile (twice the tiles of the 256-wide
// one, half the slices: half the partial-sum traffic).  Same-box timings,
// 64 x 128 / 128 x 128 / 128 x 256, us: 512x4096x3072 21.7 / 29.6 / 31.2,
// 512x3072x4096 19.9 / 30.3 / 33.6, 512x4096x4096 24.3 / 33.0 / 36.4,
// 256x4096x4096 21.7 / 26.0 / 32.2, 128x4096x4096 16.4 / 21.8 / 25.0,
// 64x4096x14336 21.3 / 26.5 / 28.8, the DBF prefill 512x4096->3072->4096
// 43.3 / 59.3 / 65.3; 1024x4096x4096 (512 of the small tiles: two rounds)
// 45.1 / 39.3 / 48.0.  Otherwise the estimated time is the number of rounds of one
// workgroup per CU times the tile width, with `GW_EFF4` the relative
// per-column cost of the 256-wide tile against the 448-wide one.  Measured at
// M = 2048, K = 4096: N = 14336 keeps 448 (217 vs 245 us), N = 11008 and
// N = 4096 take 256 (182 vs 198 us, 67 vs 96 us; the 128-wide tile 77 us).
// The test suite can force a tile (forced_kernels().gemm 11 / 12 / 14 / 17).
int64_t rounds(int64_t M, int64_t N, int bn, int cus) {
  const int64_t tiles = ((M + 127) / 128) * ((N + bn - 1) / bn);
  return (tiles + cus - 1) / cus;
}

// Returns FN for the 128-row tiles, or 1 for the 64 x 128 tile (WR = 1).
int pick_fn(int64_t M, int64_t N, int cus) {
  const int forced = forced_kernels().gemm;
  if (forced == 11 || forced == 12 || forced == 14 || forced == 17) return forced - 10;
  const int64_t tiles4 = ((M + 127) / 128) * ((N + GwTile<4>::BN - 1) / GwTile<4>::BN);
  if (tiles4 * 2 <= cus) {
    const int64_t tiles1 = ((M + 63) / 64) * ((N + GwTile<1, 1>::BN - 1) / GwTile<1, 1>::BN);
    return tiles1 <= cus ? 1 : 2;
  }
  const double u4 = (double)rounds(M, N, GwTile<4>::BN, cus) * GwTile<4>::BN * GW_EFF4;
  const double u7 = (double)rounds(M, N, GwTile<7>::BN, cus) * GwTile<7>::BN;
  return u4 < u7 ? 4 : 7;
}

template <typename ST, typename YT, bool PRE>
hipError_t launch(const LinearArgs& a, const DeviceInfo& dev) {
  const int fn = pick_fn(a.M, a.N, dev.num_cus);
  if (fn == 1) return launch_fn<ST, YT, PRE, 1, 1>(a, dev);
  if (fn == 2) return launch_fn<ST, YT, PRE, 2, 2>(a, dev);
  return fn == 4 ? launch_fn<ST, YT, PRE, 4, 2>(a, dev) : launch_fn<ST, YT, PRE, 7, 2>(a, dev);
}

template <typename ST>
hipError_t launch_y(const LinearArgs& a, const DeviceInfo& dev) {
  if (a.y_dtype == DT_F32) return a.pre ? launch<ST, float, true>(a, dev) : launch<ST, float, false>(a, dev);
  return a.pre ? launch<ST, bf16_t, true>(a, dev) : launch<ST, bf16_t, false>(a, dev);
}

// X'[m][k] = bf16(x_mk · b_k) (or bf16(x_mk) without b): the activations of
// the prescaled route, one rounding of the input-side product as the fp32
// staging of the other kernels does.  Eight consecutive elements per thread
// (K % 128 == 0 keeps them inside one row), 16-byte stores; VEC loads where X
// allows them.  The grid covers the matrix once for the usual sizes; the
// stride loop only serves larger ones.
template <typename XT, typename ST, bool PRE, bool VEC>
__global__ __launch_bounds__(256) void prescale_kernel(const XT* __restrict__ X, int64_t total, int64_t K,
                                                       const ST* __restrict__ pre, bf16_t* __restrict__ Xp) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 8;
  for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; e < total; e += stride) {
    float x[8], b[8];
    if constexpr (VEC && sizeof(XT) == 4) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(X + e);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(X + e + 4);
      x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
      x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
    } else if constexpr (VEC) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(X + e);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = to_f32(X[e + i]);
    }
    if constexpr (PRE) {
      const int64_t k = e % K;
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = to_f32(pre[k + i]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = 1.f;
    }
    *reinterpret_cast<u32x4*>(Xp + e) = u32x4{pack_bf16_pair(x[0] * b[0], x[1] * b[1]),
                                              pack_bf16_pair(x[2] * b[2], x[3] * b[3]),
                                              pack_bf16_pair(x[4] * b[4], x[5] * b[5]),
                                              pack_bf16_pair(x[6] * b[6], x[7] * b[7])};
  }
}

template <typename XT, typename ST, bool PRE>
void launch_prescale(const LinearArgs& a, bf16_t* Xp) {
  const int64_t total = a.M * a.K;
  const int64_t blocks = std::min<int64_t>((total / 8 + 255) / 256, 65536);
  const bool vec = reinterpret_cast<uintptr_t>(a.X) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((prescale_kernel<XT, ST, PRE, true>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                       static_cast<const XT*>(a.X), total, a.K, static_cast<const ST*>(a.pre), Xp);
  else
    hipLaunchKernelGGL((prescale_kernel<XT, ST, PRE, false>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                       static_cast<const XT*>(a.X), total, a.K, static_cast<const ST*>(a.pre), Xp);
}

template <typename XT, typename ST>
void launch_prescale_p(const LinearArgs& a, bf16_t* Xp) {
  if (a.pre) launch_prescale<XT, ST, true>(a, Xp);
  else launch_prescale<XT, ST, false>(a, Xp);
}

}  // namespace

bool gemm_wide_prescale_eligible(const LinearArgs& a) {
  if (a.Y2) return false;
  // The prescaled activations live in 256-byte aligned scratch: only K, N, W
  // and the sizes matter (no input-side table).
  return gemm_wide_shape_ok(a.M, a.K, a.N, false, a.W, a.W);
}

// Floats of slot 0 holding the prescaled bf16 activations.
size_t prescaled_floats(const LinearArgs& a) { return (size_t)((a.M * a.K + 1) / 2 + 64); }

void gemm_wide_scratch(const LinearArgs& a, const DeviceInfo& dev, ScratchNeed* need) {
  const int fn = pick_fn(a.M, a.N, dev.num_cus);
  const int bm = fn == 1 ? GwTile<1, 1>::BM : GwTile<2>::BM;
  const int bn = fn == 1 ? GwTile<1, 1>::BN : (fn == 2 ? GwTile<2>::BN : (fn == 4 ? GwTile<4>::BN : GwTile<7>::BN));
  const int64_t tiles = ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
  int per = 0;
  const int nsplit = split_plan(tiles, a.K / GW_KT, dev.num_cus, &per);
  if (nsplit > 1) need->need(1, (size_t)nsplit * (size_t)(a.M * a.N));
}

void gemm_wide_prescaled_scratch(const LinearArgs& a, const DeviceInfo& dev, ScratchNeed* need) {
  need->need(0, prescaled_floats(a));
  gemm_wide_scratch(a, dev, need);
}

hipError_t launch_gemm_wide_prescaled(const LinearArgs& a, const DeviceInfo& dev) {
  float* buf = a.sx ? a.sx->get(0, prescaled_floats(a)) : nullptr;
  if (!buf) return hipErrorInvalidValue;
  bf16_t* Xp = reinterpret_cast<bf16_t*>(buf);
  if (a.x_dtype == DT_F32) {
    if (a.scale_dtype == DT_F32) launch_prescale_p<float, float>(a, Xp);
    else launch_prescale_p<float, f16_t>(a, Xp);
  } else {
    if (a.scale_dtype == DT_F32) launch_prescale_p<bf16_t, float>(a, Xp);
    else launch_prescale_p<bf16_t, f16_t>(a, Xp);
  }
  LinearArgs b = a;
  b.X = Xp;
  b.x_dtype = DT_BF16;
  b.pre = nullptr;
  return launch_gemm_wide(b, dev);
}

bool gemm_wide_eligible(const LinearArgs& a) {
  if (a.x_dtype != DT_BF16) return false;
  return gemm_wide_shape_ok(a.M, a.K, a.N, a.pre != nullptr, a.X, a.W);
}

bool gemm_wide_shape_ok(int64_t M, int64_t K, int64_t N, bool has_pre, const void* X, const void* W) {
  LinearArgs a{};
  a.M = M; a.K = K; a.N = N; a.pre = has_pre ? X : nullptr;
  if (a.K % GW_KT != 0) return false;
  if (reinterpret_cast<uintptr_t>(X) % 16 != 0 || reinterpret_cast<uintptr_t>(W) % 16 != 0) return false;
  // Buffer byte ranges and offsets must fit in 32 bits (with room for the
  // out-of-range sentinel), and the grid in an int.
  const int64_t lim = (int64_t)0xFFFFF000u;
  if (a.M * a.K * 2 > lim || a.N * (a.K / 32) * 4 > lim) return false;
  const int64_t tiles = ((a.M + 63) / 64) * ((a.N + GwTile<1, 1>::BN - 1) / GwTile<1, 1>::BN);
  if (tiles > 0x7fffffff) return false;
  // LDS: the bf16(b) table (2K bytes rounded up to 8 KiB batches, dynamic)
  // next to ~124 KiB of static stage buffers.
  return !a.pre || a.K <= 16384;
}

hipError_t launch_gemm_wide(const LinearArgs& a, const DeviceInfo& dev) {
  return a.scale_dtype == DT_F32 ? launch_y<float>(a, dev) : launch_y<f16_t>(a, dev);
}

}  // namespace obl
