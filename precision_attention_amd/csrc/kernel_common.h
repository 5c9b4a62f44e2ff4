// Device helpers shared by the attention kernels (fwd.hip, decode.hip): operand types,
// the FP8 MFMA, exp2, the LDS swizzle and the LDS-DMA load. Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8attn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x16 mfma_e4m3(const i32x8& a, const i32x8& b, const f32x16& c) {
  // cbsz/blgp format 0 = E4M3 for both operands; zero scale operands select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// bf16 x bf16 -> fp32, 32x32 outputs, k = 16 (exact products, fp32 accumulation); the
// result layout is the one of mfma_e4m3.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x16 mfma_bf16(const i32x4& a, const i32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Two E4M3 codes (the low or the high 16-bit word of w) to two bf16 values, exactly (every
// E4M3 value is a bf16 value); one packed word.
template <bool HI>
__device__ __forceinline__ int e4m3x2_to_bf16x2(int w) {
  return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Four E4M3 codes (one dword) to four bf16 values (two dwords), in the same order.
__device__ __forceinline__ i32x2 e4m3x4_to_bf16x4(int w) {
  return i32x2{e4m3x2_to_bf16x2<false>(w), e4m3x2_to_bf16x2<true>(w)};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS row swizzle: 16-byte chunk c of row j lives at chunk c ^ swz(j). With
// swz(j) = (j ^ j>>3) & 7 the 128-bit K-operand reads (16 consecutive rows, one chunk,
// per cycle) hit distinct bank groups; the transposing V reads and the 128-bit staging
// writes stay conflict-free as with a plain (j & 7) swizzle (measured with the LDS bank
// conflict counters).
template <int SWZ>
__device__ __forceinline__ int swz_row(int j) { return (j ^ (j >> 3)) & SWZ; }

// One LDS-DMA instruction: every lane fetches 16 bytes at base + soff + voff (a raw buffer
// of `range` bytes, so an offset past it reads zeros) and the wave's 64 x 16 bytes land
// contiguously at lds_dst (lane L at byte 16 L). Completion is counted by vmcnt.
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ void lds_dma16(const uint8_t* base, int range, lds_u8* lds_dst,
                                          int voff, int soff) {
  constexpr int kRawBufferWord3 = 0x00020000;   // 32-bit data format, untyped access
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, range, kRawBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_dma16(const uint8_t* base, int range, uint8_t* lds_dst,
                                          int voff, int soff) {
  lds_dma16(base, range, (lds_u8*)lds_dst, voff, soff);
}

// The waves-per-SIMD floor is device code-generation information only. The host pass
// leaves it out: given a template-dependent waves_per_eu it emits no launch stub.
#ifdef __HIP_DEVICE_COMPILE__
#define FP8ATTN_BOUNDS(threads, waves) __launch_bounds__(threads, waves)
#else
#define FP8ATTN_BOUNDS(threads, waves) __launch_bounds__(threads)
#endif

}  // namespace
}  // namespace fp8attn
