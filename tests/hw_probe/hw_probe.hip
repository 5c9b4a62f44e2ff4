// Test-support kernels: one hardware instruction applied to caller data (hw_probe.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hw_probe.h"

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void cvt_kernel(const float* in, uint8_t* out, long n) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (2 * t + 1 < n) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(in[2 * t], in[2 * t + 1], 0, false);
    out[2 * t] = (uint8_t)(w & 0xff);
    out[2 * t + 1] = (uint8_t)((w >> 8) & 0xff);
  }
}

// One wave per problem t: lane (r, h) = (l % 32, l / 32) feeds row r, k-slots 32h..32h+31
// of each 64-wide chunk for both operands; the result layout is row 8(q/4)+4h+q%4, col l%32.
__global__ void mfma_kernel(const uint8_t* a, const uint8_t* b, float* raw, int kch) {
  const int t = blockIdx.x, l = threadIdx.x;
  const int K = 64 * kch;
  const int r = l & 31, h = l >> 5;
  f32x16 acc = {0};
  for (int m = 0; m < kch; ++m) {
    const uint8_t* pa = a + ((size_t)t * 32 + r) * K + 64 * m + 32 * h;
    const uint8_t* pb = b + ((size_t)t * 32 + r) * K + 64 * m + 32 * h;
    const i32x4 a0 = *(const i32x4*)pa, a1 = *(const i32x4*)(pa + 16);
    const i32x4 b0 = *(const i32x4*)pb, b1 = *(const i32x4*)(pb + 16);
    const i32x8 av = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const i32x8 bv = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
  }
  for (int q = 0; q < 16; ++q) {
    const int row = 8 * (q >> 2) + 4 * h + (q & 3);
    raw[((size_t)t * 32 + row) * 32 + r] = acc[q];
  }
}

}  // namespace

extern "C" int hw_probe_cvt_e4m3(const float* in, unsigned char* out, long n, void* stream) {
  if (!in || !out || n <= 0 || (n & 1)) return -1;
  const long pairs = n / 2;
  const unsigned blocks = (unsigned)((pairs + 255) / 256);
  hipLaunchKernelGGL(cvt_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, in, out, n);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int hw_probe_mfma_dots(const unsigned char* a, const unsigned char* b, float* raw, int T, int kch,
                                  void* stream) {
  if (!a || !b || !raw || T <= 0 || kch <= 0 || kch > 64) return -1;
  if ((((uintptr_t)a) | ((uintptr_t)b)) & 15) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(T), dim3(64), 0, (hipStream_t)stream, a, b, raw, kch);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
