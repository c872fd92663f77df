/*
 * obl.h -- C ABI of libobl, the MI355X (gfx950) library for sign-binarised
 * linear layers.
 *
 * Sources:
 *  - OneBit page, "1bit量化" (blog.zerodtree.com): proposition 1 and its proof
 *    (X W^T = [(X ⊙ b^T) W_sign^T] ⊙ a^T with W = W_sign ⊙ a b^T), and the
 *    layer block under "知识蒸馏" (Y = [(X ⊙ g) W_±1^T] ⊙ h, g = b^T, h = a^T).
 *  - DBF page, "Addition is almost all you need: Compressing large language
 *    models with double binary factorization" (gist.science summary),
 *    "Methodologie": W ≈ (a ⊙ A_±1 ⊙ m^T)(B_±1 ⊙ b^T), inference chain
 *    ((((X ⊙ b^T) B_±1^T) ⊙ m^T) A_±1^T) ⊙ a^T, scale vectors in FP16.
 *
 * Conventions shared by every call
 *  - All matrices are dense, row-major and contiguous.  X is [M][K]; a sign
 *    matrix is [rows][K] with rows = outputs (the OneBit page writes X W^T
 *    with W indexed [output][input]).
 *  - Packed signs: uint32 P[rows][K/32].  Bit j (LSB = 0) of P[r][w] holds the
 *    sign of column 32*w + j; 1 means -1 and 0 means +1.
 *  - Pointers to tensors are DEVICE pointers (HIP device memory of the current
 *    device).  `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Every call is asynchronous on `stream`: it returns once the work
 *    is enqueued, and buffers must stay alive until that work completes.
 *  - Ownership: the caller owns every buffer.  The library keeps no pointer
 *    to caller memory after a call returns.  Some calls also use library
 *    scratch (device memory beyond their arguments: the split decode
 *    kernel's partial sums, a copy of the DBF intermediate, the bf16(x ⊙ b)
 *    activations the prefill path stages for fp32 or misaligned X, the
 *    prefill kernel's split-K partial sums on small grids, the vectors of
 *    obl_svid).  It comes from a pool per device and per stream: calls on
 *    different streams never share it, and calls on one stream are ordered
 *    by the stream.  The pool grows with hipMalloc when a call needs more
 *    than it holds; a replaced buffer is never freed (work already enqueued,
 *    or recorded in a HIP graph, may still use it), so all pool memory is
 *    held until the process ends.  A call that would have to grow the pool
 *    while its stream is capturing returns OBL_ERR_CAPTURE before enqueuing
 *    anything, and the capture stays valid: make one call of the same shape
 *    on that stream before capturing.  A captured graph uses the scratch of
 *    the stream it was captured on, so replays of graphs captured on one
 *    stream must not overlap each other, or calls on that stream, in time.
 *    Each stream that has made a call needing scratch keeps its pool (at
 *    least 4 MiB per buffer in use) until the process ends, so a program
 *    that runs such calls on many short-lived streams holds memory for
 *    each of them.
 *  - Errors: every argument is validated BEFORE any HIP call; a failed check
 *    returns its status and enqueues nothing.  No call aborts or throws across
 *    the ABI.  HIP failures (including launch failures seen through
 *    hipGetLastError) return OBL_ERR_HIP.  Every call that can use library
 *    scratch (all but obl_pack_signs, obl_transpose_signs and obl_layernorm)
 *    can also return OBL_ERR_CAPTURE, before enqueuing anything.
 *  - M = 0 is a valid no-op.  N, K, Kmid, rows must be >= 1 and K, Kmid must
 *    be multiples of 32 (the packed word width); a call that violates this
 *    returns OBL_ERR_SHAPE.  Every dimension must be below 2^31 and keep every
 *    byte size below 2^62 (else OBL_ERR_SHAPE).
 */
#ifndef OBL_H_
#define OBL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums have int as their underlying type in C++ too, so that any
 * integer a C caller passes (an invalid dtype, an unknown status) is a valid
 * value to inspect and reject, not undefined behaviour. */
#ifdef __cplusplus
#define OBL_ENUM(tag) enum tag : int
#else
#define OBL_ENUM(tag) enum tag
#endif

typedef OBL_ENUM(obl_status_e) {
  OBL_OK = 0,
  OBL_ERR_NULL = 1,     /* a required pointer is NULL */
  OBL_ERR_SHAPE = 2,    /* a dimension is negative / zero where not allowed / not a multiple of 32 */
  OBL_ERR_DTYPE = 3,    /* unsupported dtype or dtype combination */
  OBL_ERR_ALIGN = 4,    /* a pointer is not aligned to its element size (packed words: 4 bytes) */
  OBL_ERR_ALIAS = 5,    /* an output overlaps an input or another output */
  OBL_ERR_HIP = 6,      /* the HIP runtime reported an error */
  OBL_ERR_INTERNAL = 7, /* unexpected internal failure */
  OBL_ERR_VALUE = 8,    /* a scalar argument is out of range (e.g. a negative epsilon) */
  OBL_ERR_CAPTURE = 9,  /* library scratch would have to grow while the call's stream is capturing */
  OBL_ERR_SCRATCH = 10  /* dbf_linear_noalloc: the call needs more than its fixed scratch */
} obl_status;

typedef OBL_ENUM(obl_dtype_e) {
  OBL_F32 = 0,
  OBL_F16 = 1,
  OBL_BF16 = 2,
  OBL_I8 = 3
} obl_dtype;

/*
 * obl_pack_signs -- W_sign = Sign(S) bit-packed along K.
 *   OneBit page, "rank-1 approximation" block: W = W_sign ⊙ |W| with
 *   W_sign = Sign(W).  Sign of zero is not given there; a value packs as -1
 *   exactly when it compares below zero (so 0, -0.0 and NaN pack as +1).
 *
 *   S       [rows][K] of s_dtype (OBL_I8, OBL_F32, OBL_F16 or OBL_BF16), device.
 *   packed  [rows][K/32] uint32, device, written.  Must not overlap S.
 *   Errors: OBL_ERR_NULL, OBL_ERR_SHAPE (rows < 1, K < 1 or K % 32 != 0),
 *           OBL_ERR_DTYPE, OBL_ERR_ALIGN (S not aligned to its element, packed
 *           not 4-byte aligned), OBL_ERR_ALIAS, OBL_ERR_HIP.
 */
obl_status obl_pack_signs(const void* S, obl_dtype s_dtype, int64_t rows, int64_t K,
                          uint32_t* packed, void* stream);

/*
 * obl_linear -- Y[M][N] = ((X[M][K] ⊙ b[K]) · W_sign[N][K]^T) ⊙ a[N].
 *   OneBit page, proposition 1 (right-hand side) and the layer block under
 *   "知识蒸馏" (b is the layer's g, a its h).
 *
 *   X         [M][K], x_dtype OBL_F32 or OBL_BF16.
 *   W_packed  [N][K/32] packed signs (format above).
 *   a         [N], b [K], both scale_dtype (OBL_F32 or OBL_F16).
 *   Y         [M][N], y_dtype OBL_F32 or OBL_BF16, written; must not overlap
 *             any input.
 *   Arithmetic: for M <= 16 (decode) x·b is formed in fp32 and the contraction
 *   keeps fp32 accuracy (|Y - Y_exact| <= 1e-5 · |a_j| Σ_k |x_ik b_k| before the
 *   final cast); for M > 16 (prefill) the contraction runs on bf16 matrix
 *   cores with one bf16 rounding of the input-side operand and fp32
 *   accumulation (<= 8e-3 on the same scale, including a bf16 output cast).
 *   Calls of 17..32 rows with bf16 X, fp16 scales, 16-byte aligned X, packed
 *   words and b and K % 128 == 0 run the decode path (fp32 accuracy) where it
 *   is the faster choice (K <= 8192).
 *   Errors: OBL_ERR_NULL, OBL_ERR_SHAPE, OBL_ERR_DTYPE, OBL_ERR_ALIGN,
 *           OBL_ERR_ALIAS, OBL_ERR_HIP.
 */
obl_status obl_linear(const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                      const uint32_t* W_packed, int64_t N,
                      const void* a, const void* b, obl_dtype scale_dtype,
                      void* Y, obl_dtype y_dtype, void* stream);

/*
 * dbf_linear -- Y[M][N] = ((((X ⊙ b) · S2[Kmid][K]^T) ⊙ m) · S1[N][Kmid]^T) ⊙ a.
 *   DBF page, "Methodologie": inference chain with S2 = B_±1, S1 = A_±1.
 *
 *   X          [M][K], x_dtype OBL_F32 or OBL_BF16.
 *   S2_packed  [Kmid][K/32], S1_packed [N][Kmid/32] packed signs.
 *   b [K], m [Kmid], a [N], all scale_dtype (OBL_F32 or OBL_F16).
 *   workspace  float32 [M][Kmid], caller-owned.  When the call's work has
 *              completed it holds T1 = ((X ⊙ b) S2^T) ⊙ m (stage 1, kept in
 *              fp32); stage 2 reads it, or (decode sizes up to 8 rows) the
 *              exact bf16 terms of T1 that stage 1 also writes into library
 *              scratch.  Must not overlap any other argument.
 *   Y          [M][N], y_dtype OBL_F32 or OBL_BF16.
 *   Arithmetic: each stage follows obl_linear's rules for the same M
 *   (stage 2 has no input-side scale; at prefill sizes it reads T1 rounded
 *   once to bf16).
 *   Errors: as obl_linear.
 */
obl_status dbf_linear(const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                      const uint32_t* S2_packed, int64_t Kmid,
                      const uint32_t* S1_packed, int64_t N,
                      const void* b, const void* m, const void* a, obl_dtype scale_dtype,
                      float* workspace, void* Y, obl_dtype y_dtype, void* stream);

/*
 * dbf_linear_noalloc -- dbf_linear for callers that cannot allocate device
 *   memory (code under HIP graph capture, tight serving loops, harnesses that
 *   forbid hipMalloc): the same arguments, arithmetic and results, but its
 *   scratch is a fixed 64 MiB device array (two 32 MiB slots: the copy of T1
 *   plus the stages' own scratch in one, split-K partial sums in the other)
 *   instead of the pool, and it calls no allocating routine.  Each GPU the
 *   library runs on holds that array until the process ends.  Every call on
 *   one GPU shares its array, and its contents persist from call to call
 *   (nothing there needs to start at zero: every value is written before it
 *   is read), so calls that overlap in time on one GPU -- on different
 *   streams, host threads, or replays of captured graphs -- race and must be
 *   serialised by the caller.  With bf16 X the limit is about
 *   3 M Kmid <= 2^25 at decode sizes (M <= 8) and M Kmid <= 2^26 at prefill
 *   sizes; a call that needs more returns OBL_ERR_SCRATCH before enqueuing
 *   anything.
 *   Errors: as dbf_linear, plus OBL_ERR_SCRATCH; never OBL_ERR_CAPTURE.
 */
obl_status dbf_linear_noalloc(const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                              const uint32_t* S2_packed, int64_t Kmid,
                              const uint32_t* S1_packed, int64_t N,
                              const void* b, const void* m, const void* a, obl_dtype scale_dtype,
                              float* workspace, void* Y, obl_dtype y_dtype, void* stream);

/*
 * obl_svid -- Sign-Value-Independent Decomposition of a dense weight:
 *   W ≈ W_sign ⊙ (a b^T).  OneBit page, "rank-1 approximation" block and
 *   proposition 2: W_sign = Sign(W) and a b^T is the rank-1 approximation of
 *   |W|: σ1 u1 v1^T of its leading singular triple, split as a = sqrt(σ1) u1,
 *   b = sqrt(σ1) v1 with the (nonnegative) singular vectors of |W|.
 *   W       [N][K] dense, w_dtype OBL_F32, OBL_F16 or OBL_BF16, device.
 *   iters   power-iteration steps, >= 1; each reads |W| once (K <= 4096 with
 *           16-bit W, K <= 2048 with fp32 W, W 16-byte aligned) or twice.
 *   packed  [N][K/32] Sign(W) (format above; 0 and -0 pack as +1), written.
 *   a [N], b [K] scale_dtype (OBL_F32 or OBL_F16), written.
 *   Uses the library's per-device scratch (see Ownership); sums are fp32 in a
 *   fixed order.  Errors: OBL_ERR_NULL, OBL_ERR_SHAPE (N, K < 1, K % 32 != 0,
 *   iters out of [1, 100000]), OBL_ERR_DTYPE, OBL_ERR_ALIGN, OBL_ERR_ALIAS,
 *   OBL_ERR_HIP.
 */
obl_status obl_svid(const void* W, obl_dtype w_dtype, int64_t N, int64_t K, int iters, uint32_t* packed,
                    void* a, void* b, obl_dtype scale_dtype, void* stream);

/*
 * obl_transpose_signs -- packed signs of the transposed sign matrix.
 *   packed    [rows][K/32] packed signs (format above).
 *   packed_t  [K][rows/32], written: bit j of packed_t[k][w] is the sign of
 *             row 32*w + j, column k (the same format, packed along rows).
 *   Needed once per weight by obl_linear_backward, whose input gradient
 *   contracts over the output dimension (OneBit page, knowledge-distillation
 *   block: the layer is trained through its gradients).
 *   Errors: OBL_ERR_NULL, OBL_ERR_SHAPE (rows or K < 1, or not multiples of
 *           32), OBL_ERR_ALIGN (4-byte), OBL_ERR_ALIAS, OBL_ERR_HIP.
 */
obl_status obl_transpose_signs(const uint32_t* packed, int64_t rows, int64_t K, uint32_t* packed_t,
                               void* stream);

/*
 * obl_linear_backward -- gradients of Y = ((X ⊙ b) W_sign^T) ⊙ a for an
 * upstream gradient dY [M][N] (OneBit page, knowledge-distillation block; the
 * formulas are the chain rule on proposition 1's right-hand side):
 *   dX = ((dY ⊙ a) · W_sign) ⊙ b          [M][K], dx_dtype (OBL_F32 / OBL_BF16)
 *   da_j = Σ_i dY_ij · T_ij,  T = (X ⊙ b) W_sign^T      [N] fp32
 *   db_k = Σ_i x_ik · U_ik,   U = (dY ⊙ a) W_sign       [K] fp32
 *   dY, X      x_dtype (OBL_F32 or OBL_BF16), row-major [M][N] and [M][K].
 *   W_packed   [N][K/32]; Wt_packed [K][N/32] from obl_transpose_signs.
 *   a [N], b [K] scale_dtype (OBL_F32 or OBL_F16).
 *   workspace  fp32 [M][N + K], caller-owned: after completion it holds T
 *              then U.  Must not overlap any other argument.
 *   Arithmetic: T and U follow obl_linear's rules for the same M (the decode
 *   paths keep fp32 accuracy, the prefill path rounds one input-side factor
 *   to bf16); the sums over M are fp32 in a fixed order (reproducible).
 *   M = 0 writes da = db = 0.
 *   Errors: as obl_linear; N must also be a multiple of 32.
 */
obl_status obl_linear_backward(const void* dY, const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                               const uint32_t* W_packed, const uint32_t* Wt_packed, int64_t N,
                               const void* a, const void* b, obl_dtype scale_dtype,
                               void* dX, obl_dtype dx_dtype, float* da, float* db,
                               float* workspace, void* stream);

/*
 * obl_layernorm -- Z = LayerNorm(Y) over each row of Y [M][N].
 *   OneBit page, knowledge-distillation block: the layer output is
 *   layer-normalised (Z = LayerNorm(Y)) before the distillation losses.  The
 *   page gives no epsilon or affine parameters; both are the caller's:
 *     μ_i = mean_j y_ij,  σ²_i = mean_j (y_ij - μ_i)²  (biased, two passes),
 *     z_ij = (y_ij - μ_i) / sqrt(σ²_i + eps) · gamma_j + beta_j.
 *   Y       [M][N], y_dtype OBL_F32 or OBL_BF16.
 *   eps     finite and >= 0 (eps = 0 turns a constant row into NaN, as the
 *           formula does); otherwise OBL_ERR_VALUE.
 *   gamma, beta  [N] of affine_dtype (OBL_F32 or OBL_F16); either may be NULL
 *           (gamma = 1, beta = 0).  affine_dtype is ignored when both are NULL.
 *   Z       [M][N], z_dtype OBL_F32 or OBL_BF16, written; must not overlap
 *           any input.
 *   Arithmetic: fp32 sums in a fixed order (bitwise reproducible); the error
 *   is a few fp32 ulps of (|y| + |μ|) / σ before the output cast.
 *   Errors: OBL_ERR_NULL, OBL_ERR_SHAPE (M < 0, N < 1), OBL_ERR_DTYPE,
 *           OBL_ERR_VALUE, OBL_ERR_ALIGN, OBL_ERR_ALIAS, OBL_ERR_HIP.
 */
obl_status obl_layernorm(const void* Y, obl_dtype y_dtype, int64_t M, int64_t N, float eps,
                         const void* gamma, const void* beta, obl_dtype affine_dtype,
                         void* Z, obl_dtype z_dtype, void* stream);

/*
 * obl_linear_layernorm -- Z = LayerNorm(((X ⊙ b) · W_sign^T) ⊙ a): the layer of
 *   obl_linear followed by obl_layernorm in one call (OneBit page,
 *   knowledge-distillation block: Y = [(X ⊙ g) W_±1^T] ⊙ h, then
 *   Z = LayerNorm(Y)).
 *   X, W_packed, a, b, scale_dtype: as obl_linear.
 *   eps, gamma, beta: as obl_layernorm, with gamma and beta of scale_dtype.
 *   workspace  float32 [M][N], caller-owned: after completion it holds Y in
 *              fp32.  Must not overlap any other argument.
 *   Z          [M][N], z_dtype OBL_F32 or OBL_BF16, written.
 *   Arithmetic: Y follows obl_linear's rules for the same M; LayerNorm as
 *   obl_layernorm on the fp32 Y.
 *   Errors: as obl_linear and obl_layernorm.
 */
obl_status obl_linear_layernorm(const void* X, obl_dtype x_dtype, int64_t M, int64_t K,
                                const uint32_t* W_packed, int64_t N,
                                const void* a, const void* b, obl_dtype scale_dtype,
                                float eps, const void* gamma, const void* beta,
                                float* workspace, void* Z, obl_dtype z_dtype, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* obl_status_string(obl_status status);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int obl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OBL_H_ */
