// Shared device helpers for the libobl kernels (gfx950 / CDNA4, wave64).
//
// Packed sign format: uint32 P[rows][K/32]; bit j of P[r][w] is the sign of
// column 32*w + j, 1 = -1.  A set bit is therefore exactly the IEEE sign bit
// that has to be applied to the matching input value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace obl {

enum Dtype : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Storage types.  bf16 and fp16 are carried as raw 16-bit patterns so that no
// host-side half/bfloat class is needed in kernel signatures.
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(uint32_t(v.bits) << 16); }
__device__ __forceinline__ float to_f32(f16_t v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, v.bits));
}

// fp32 -> bf16, round to nearest even (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf16_round(float f) {
  return __uint_as_float(bf16_bits_rne(f) << 16);
}

template <typename T> struct Store;
template <> struct Store<float> {
  static __device__ __forceinline__ void put(float* p, float v) { *p = v; }
};
template <> struct Store<bf16_t> {
  static __device__ __forceinline__ void put(bf16_t* p, float v) {
    p->bits = static_cast<uint16_t>(bf16_bits_rne(v));
  }
};
template <> struct Store<f16_t> {
  static __device__ __forceinline__ void put(f16_t* p, float v) {   // round to nearest even
    p->bits = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
  }
};

// Element i of an optional scale vector, or 1 when it is absent (p null).
// The load is issued unconditionally -- from `safe`, any buffer holding at
// least i + 1 elements' worth of bytes, when p is null -- and the result is
// selected: a load under a branch is waited for at the end of the branch,
// which would put a memory round trip in front of every later load.
template <typename ST>
__device__ __forceinline__ float scale_or_one(const ST* p, int64_t i, const void* safe) {
  const ST* q = p ? p : static_cast<const ST*>(safe);
  const float v = to_f32(q[i]);
  return p ? v : 1.f;
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds_wave_base + 16*l, where lds_wave_base must be
// the same for the whole wave.  Counted by vmcnt like any vector load.
__device__ __forceinline__ void load_lds16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Buffer resource for a raw byte range: loads past `bytes` return zeros
// instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// LDS DMA of 16 bytes per lane from a buffer resource at byte offset voff +
// soff (soff uniform): lane l's bytes land at lds_wave_base + 16 l
// (lds_wave_base uniform over the wave).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           (int)voff, (int)soff, 0, 0);
}

// The same, marked non-temporal (streamed data that no later access reuses:
// it does not displace cached operands).
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t voff,
                                         uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           (int)voff, (int)soff, 0, 2);
}

// Workgroup barrier that orders LDS accesses across the workgroup but does
// not wait for global loads in flight (__syncthreads() also drains vmcnt):
// workgroup-scope release and acquire fences on LDS only (they compile to
// lgkmcnt(0), and keep the compiler from moving LDS accesses across) around
// s_barrier.  s_waitcnt immediate: lgkmcnt = 0, vmcnt = 63, expcnt = 7.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One 16x16x32 bf16 MFMA step with fp32 accumulation.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Operand order inside one 32-wide k-step ("pair order").
//
// A lane of a 16x16x32 MFMA holds 8 bf16 values of one row (A) or one column
// (B), for lane group g = lane / 16.  Which eight of the 32 k-values a lane
// holds is free as long as A and B agree, so the kernels use the order that
// makes sign expansion cheapest: dword j (j = 0..3) of lane group g holds
//     low half  <- k = 4g + j
//     high half <- k = 4g + j + 16.
// Shifting the sign word right by 4g and then left by (15 - j) puts the sign
// bits of both k-values at bit 15 and bit 31, the sign bits of the two bf16
// halves -- one shift and one bitwise op per two weights.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 expand_signs_pm1(uint32_t w_shifted) {
  u32x4 r;
  r.x = ((w_shifted << 15) & 0x80008000u) ^ 0x3F803F80u;  // +-1.0 bf16 pairs
  r.y = ((w_shifted << 14) & 0x80008000u) ^ 0x3F803F80u;
  r.z = ((w_shifted << 13) & 0x80008000u) ^ 0x3F803F80u;
  r.w = ((w_shifted << 12) & 0x80008000u) ^ 0x3F803F80u;
  return r;
}

// Same, but the magnitudes come from `mag` (bf16 pairs in pair order): each
// half gets its sign flipped where the weight is -1 (v_bitop3: (x & m) ^ c).
__device__ __forceinline__ u32x4 expand_signs_scaled(uint32_t w_shifted, u32x4 mag) {
  u32x4 r;
  r.x = ((w_shifted << 15) & 0x80008000u) ^ mag.x;
  r.y = ((w_shifted << 14) & 0x80008000u) ^ mag.y;
  r.z = ((w_shifted << 13) & 0x80008000u) ^ mag.z;
  r.w = ((w_shifted << 12) & 0x80008000u) ^ mag.w;
  return r;
}

// Perfect outer unshuffle of a 32-bit sign word: bit 2i -> bit i and bit 2i+1
// -> bit 16+i (i < 16).  After it, the signs of the adjacent pair (k = 2i,
// 2i+1) sit 16 bits apart, which is the pair the expansion above serves, so
// operands stored in natural k order pair with the expanded signs.
__device__ __forceinline__ uint32_t unzip_bits(uint32_t x) {
  uint32_t t;
  t = (x ^ (x >> 1)) & 0x22222222u; x = x ^ t ^ (t << 1);
  t = (x ^ (x >> 2)) & 0x0C0C0C0Cu; x = x ^ t ^ (t << 2);
  t = (x ^ (x >> 4)) & 0x00F000F0u; x = x ^ t ^ (t << 4);
  return __builtin_amdgcn_perm(x, x, 0x07050604u) ;  // swap bytes 1 and 2
}

// Pack two fp32 values (already representable in bf16) into one dword.
__device__ __forceinline__ uint32_t pack_bf16_pair(float lo, float hi) {
  return bf16_bits_rne(lo) | (bf16_bits_rne(hi) << 16);
}

// Exact three-way split of an fp32 value into bf16 terms: v = hi + mid + lo
// whenever v has at most 24 significant bits and no term underflows.  Each
// remainder is exact in fp32 because it is the rounding error of the previous
// bf16 rounding.
struct Split3 { float hi, mid, lo; };
__device__ __forceinline__ Split3 split3(float v) {
  Split3 s;
  s.hi = bf16_round(v);
  float r = v - s.hi;
  s.mid = bf16_round(r);
  s.lo = bf16_round(r - s.mid);
  return s;
}

}  // namespace obl
