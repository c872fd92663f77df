// Internal launcher interface between the C ABI (obl_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace obl {

// Internal x_dtype: three bf16 arrays [3][rows][cols] whose sum hi + mid + lo
// is an fp32 value exactly (public dtype codes stay below 16).
constexpr int kDtBf16x3 = 16;
constexpr int DT_BF16X3 = kDtBf16x3;

// One sign-binarised contraction Y = ((X ⊙ pre) · W^T) ⊙ post.
struct LinearArgs {
  const void* X;      // [M][K], x_dtype
  int x_dtype;        // DT_F32 or DT_BF16 (internally also DT_BF16X3: DBF stage 2 on the decode path)
  int64_t M, K;
  const uint32_t* W;  // [N][K/32] packed signs
  int64_t N;
  const void* pre;    // [K] or nullptr (= all ones)
  const void* post;   // [N], or nullptr (= all ones; internal calls only)
  int scale_dtype;    // DT_F32 or DT_F16
  void* Y;            // [M][N]
  int y_dtype;        // DT_F32 or DT_BF16
  hipStream_t stream;
  const struct ScratchCtx* sx = nullptr;  // library scratch reserved for this call (see ScratchCtx)
  void* Y2 = nullptr; // optional bf16 copy of Y (prefill GEMM only; see gemm_wide_eligible)
  // Optional span record (LUT GEMV only; the bench's kernel-time measurement):
  // block b writes its first wave's start and its end, in s_memrealtime
  // ticks, to span[2b], span[2b + 1].
  uint64_t* span = nullptr;
  void* T3 = nullptr; // optional exact bf16 terms of an fp32 Y, [3][M][N] (decode whole-K kernel only)
  // Optional gradient epilogue (decode whole-K kernel only; the layer's
  // backward): gsum[n] = Σ_m gin[m][n] · Y[m][n] (gin in x_dtype, gsum fp32),
  // and gout[m][n] = Y[m][n] · gscale[n] (gscale in scale_dtype, gout in
  // gout_dtype) when gout is set.
  const void* gin = nullptr;
  float* gsum = nullptr;
  const void* gscale = nullptr;
  void* gout = nullptr;
  int gout_dtype = 0;
};

struct DeviceInfo {
  int device;
  int num_cus;
};

// Library scratch: device memory a call uses beyond its inputs and outputs,
// in two slots.  Slot 0 holds the split decode kernel's partial sums, the
// prescaled bf16 activations of the prefill route, the SVID vectors and (DBF)
// the copy of T1 that stage 2 reads; slot 1 holds the prefill GEMM's split-K
// partial sums.  A call first adds up what its launches will take
// (ScratchNeed, from the same decisions the launchers make), the entry point
// reserves it -- from the per-stream pool, or from the fixed array of the
// allocation-free entry point -- and the launchers then only carve it.
enum { kScratchSlots = 2 };
struct ScratchNeed {
  size_t floats[kScratchSlots] = {0, 0};
  void need(int slot, size_t n) {
    if (n > floats[slot]) floats[slot] = n;
  }
};
struct ScratchCtx {
  float* base[kScratchSlots] = {nullptr, nullptr};
  size_t cap[kScratchSlots] = {0, 0};    // floats
  size_t taken[kScratchSlots] = {0, 0};  // floats held by the entry point itself (DBF's T1 copy)
  // `floats` floats of slot `slot` past the entry point's own region, 256-byte
  // aligned, or nullptr when they were not reserved (a planning mistake: the
  // launcher then fails with an error instead of writing past the buffer).
  float* get(int slot, size_t floats) const {
    if (!base[slot] || taken[slot] + floats > cap[slot]) return nullptr;
    return base[slot] + taken[slot];
  }
};
// Floats of a region rounded up to 256 bytes, so the next region stays aligned.
inline size_t scratch_round(size_t floats) { return (floats + 63) & ~size_t(63); }

hipError_t device_info(DeviceInfo* out);

hipError_t launch_pack_signs(const void* S, int s_dtype, int64_t rows, int64_t K, uint32_t* P,
                             hipStream_t stream);
hipError_t launch_gemv_lut(const LinearArgs& a, const DeviceInfo& dev);
size_t svid_workspace_floats(int64_t N, int64_t K);
hipError_t launch_svid(const void* W, int w_dtype, int64_t N, int64_t K, int iters, void* a, void* b,
                       int scale_dtype, float* ws, hipStream_t st);
hipError_t launch_transpose_signs(const uint32_t* P, int64_t rows, int64_t K, uint32_t* PT, hipStream_t st);
hipError_t launch_backward_grads(int x_dtype, int scale_dtype, int dx_dtype, const void* dY, const void* X,
                                 const float* T, const float* U, const void* b, int64_t M, int64_t K,
                                 int64_t N, void* dX, float* da, float* db, hipStream_t st);
hipError_t launch_layernorm_rows(const void* Y, int y_dtype, int64_t M, int64_t N, float eps, const void* gamma,
                                 const void* beta, int g_dtype, void* Z, int z_dtype, hipStream_t st);
hipError_t launch_decode_mfma(const LinearArgs& a, const DeviceInfo& dev);
// Scratch the decode path's launch of this call takes (the split kernel's
// partial sums when K spans several slices).
void decode_scratch(const LinearArgs& a, const DeviceInfo& dev, ScratchNeed* need);
// The decode path's whole-K kernel takes this call (bf16 x, fp16 scales,
// aligned operands, K % 128 == 0, M <= kDecodeWideMaxM; not forced off).
bool decode_wide_ok(const LinearArgs& a);
// ... and is the faster choice for 17..32 rows (the automatic path).
bool decode_wide_preferred(const LinearArgs& a);
// A DBF decode can run both stages on the whole-K kernel: stage 1 writes the
// exact bf16 terms of T1 (s1.T3), stage 2 reads them (x_dtype DT_BF16X3).
bool decode_terms_ok(const LinearArgs& s1, const LinearArgs& s2);
// Two whole-K contractions with gradient epilogues (the layer's backward: bf16
// x, fp16 scales, fp32 outputs, same M and stream) as one launch; returns
// hipErrorNotSupported, with nothing launched, when they do not take one
// kernel instance.
hipError_t launch_decode_pair(const LinearArgs& t, const LinearArgs& u, const DeviceInfo& dev);
hipError_t launch_gemm_mfma(const LinearArgs& a, const DeviceInfo& dev);
// Scratch the prefill path's launch of this call takes (prescaled
// activations in slot 0, split-K partial sums in slot 1).
void gemm_scratch(const LinearArgs& a, const DeviceInfo& dev, ScratchNeed* need);
// Main prefill kernel (bf16 activations); launch_gemm_mfma dispatches to it.
bool gemm_wide_eligible(const LinearArgs& a);
// Shape/alignment test for a bf16-activation prefill call of the given sizes.
bool gemm_wide_shape_ok(int64_t M, int64_t K, int64_t N, bool has_pre, const void* X, const void* W);
hipError_t launch_gemm_wide(const LinearArgs& a, const DeviceInfo& dev);
// Prefill for activations the main kernel cannot take directly (fp32, or bf16
// that is misaligned or whose b exceeds the table): bf16(x ⊙ b) into library
// scratch (the first buffer), then the main kernel without b.
bool gemm_wide_prescale_eligible(const LinearArgs& a);
hipError_t launch_gemm_wide_prescaled(const LinearArgs& a, const DeviceInfo& dev);
void gemm_wide_scratch(const LinearArgs& a, const DeviceInfo& dev, ScratchNeed* need);
void gemm_wide_prescaled_scratch(const LinearArgs& a, const DeviceInfo& dev, ScratchNeed* need);

// Kernel choices forced by the test suite through obl_internal_force_kernels
// (an internal export, not part of obl.h; per calling thread, all zero unless
// a test sets them).  path: 0 auto, 1 LUT GEMV, 2 decode, 3 prefill GEMM.
// gemm: 0 auto, 1 / 2 the older 8-wave / LDS-staged kernels, 11 / 12 / 14 /
// 17 a tile of the main kernel (64 x 128, 128 x 128, 128 x 256, 128 x 448).
// decode: 0 auto, 1 the split kernel, 11 / 12 / 14 the whole-K kernel with
// 1 / 2 / 4 column groups per wave.  pair: 0 auto, 1 the backward's two
// contractions as two launches.
struct ForcedKernels {
  int path = 0, gemm = 0, decode = 0, pair = 0;
};
const ForcedKernels& forced_kernels();

// Largest M served by the LUT GEMV and by the decode kernels (the split
// kernel: 16; the whole-K kernel: 32).
constexpr int64_t kLutMaxM = 2;
constexpr int64_t kDecodeMaxM = 16;
constexpr int64_t kDecodeWideMaxM = 32;

}  // namespace obl
