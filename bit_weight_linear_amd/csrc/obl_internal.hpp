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
  void* Y2 = nullptr; // optional bf16 copy of Y (prefill GEMM only; see gemm_wide_eligible)
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

// Per-device scratch for split-K partial sums.
struct Scratch {
  float* partials;
  size_t partial_floats;
};

hipError_t device_info(DeviceInfo* out);
hipError_t scratch_reserve(int device, size_t partial_floats, Scratch* out);
// A second per-device buffer for the prefill GEMM's split-K partial sums (used
// while the first one may hold a DBF intermediate).  Same growth policy.
hipError_t split_reserve(int device, size_t floats, float** out);

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
// The decode path's whole-K kernel takes this call (bf16 x, fp16 scales,
// aligned operands, K % 128 == 0, M <= kDecodeWideMaxM; not forced off).
bool decode_wide_ok(const LinearArgs& a);
// ... and is the faster choice for 17..32 rows (the automatic path).
bool decode_wide_preferred(const LinearArgs& a);
// A DBF decode can run both stages on the whole-K kernel: stage 1 writes the
// exact bf16 terms of T1 (s1.T3), stage 2 reads them (x_dtype DT_BF16X3).
bool decode_terms_ok(const LinearArgs& s1, const LinearArgs& s2);
hipError_t launch_gemm_mfma(const LinearArgs& a, const DeviceInfo& dev);
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

// Largest M served by the LUT GEMV and by the decode kernels (the split
// kernel: 16; the whole-K kernel: 32).
constexpr int64_t kLutMaxM = 2;
constexpr int64_t kDecodeMaxM = 16;
constexpr int64_t kDecodeWideMaxM = 32;

}  // namespace obl
