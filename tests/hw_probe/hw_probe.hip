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

__global__ __launch_bounds__(512) void throughput_kernel(int kind, int iters, const int* seed, float* sink,
                                                         float* clock) {
  const int tid = threadIdx.x, wave = tid >> 6;
  i32x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = seed[(tid + i) & 255] & 0x3f3f3f3f;
    b[i] = seed[(tid + 3 * i) & 255] & 0x3f3f3f3f;
  }
  f32x16 acc[4];
  for (int u = 0; u < 4; ++u) acc[u] = f32x16{0};
  float x[32];
  for (int i = 0; i < 32; ++i) x[i] = (float)(seed[(tid + 7 * i) & 255] & 1023) * 1e-3f - 20.f;
  bool do_m = kind == 0 || kind == 2, do_e = kind == 1 || kind == 2;
  if (kind == 3) {
    do_m = wave < 4;
    do_e = wave >= 4;
  }
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if (do_m) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[u], 0, 0, 0, 0, 0, 0);
    }
    if (do_e) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) - 20.f;
    }
  }
  float s = 0.f;
  for (int u = 0; u < 4; ++u)
    for (int r = 0; r < 16; ++r) s += acc[u][r];
  for (int i = 0; i < 32; ++i) s += x[i];
  sink[(size_t)blockIdx.x * blockDim.x + tid] = s;
  if (tid == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clock[blockIdx.x] = r1 > r0 ? (float)((double)(t1 - t0) / (double)(r1 - r0)) : 0.f;
  }
}

}  // namespace

extern "C" int hw_probe_throughput(int kind, int blocks, int iters, const int* seed, float* sink, float* clock,
                                   void* stream) {
  if (kind < 0 || kind > 3 || blocks <= 0 || iters <= 0 || !seed || !sink || !clock) return -1;
  hipLaunchKernelGGL(throughput_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, kind, iters, seed,
                     sink, clock);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

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
