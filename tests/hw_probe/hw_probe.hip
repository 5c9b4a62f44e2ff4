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

// 16x16x128 form: one wave per problem t; lane l feeds row l % 16, k-slots 32(l / 16) ..
// +31 of each 128-wide chunk for both operands; the result layout is row 4(l / 16) + i,
// col l % 16.
__global__ void mfma16_kernel(const uint8_t* a, const uint8_t* b, float* raw, int kch) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int t = blockIdx.x, l = threadIdx.x;
  const int K = 128 * kch;
  const int r = l & 15, g = l >> 4;
  f32x4 acc = {0};
  for (int m = 0; m < kch; ++m) {
    const uint8_t* pa = a + ((size_t)t * 16 + r) * K + 128 * m + 32 * g;
    const uint8_t* pb = b + ((size_t)t * 16 + r) * K + 128 * m + 32 * g;
    const i32x4 a0 = *(const i32x4*)pa, a1 = *(const i32x4*)(pa + 16);
    const i32x4 b0 = *(const i32x4*)pb, b1 = *(const i32x4*)(pb + 16);
    const i32x8 av = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const i32x8 bv = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
  }
  for (int i = 0; i < 4; ++i) raw[((size_t)t * 16 + 4 * g + i) * 16 + r] = acc[i];
}

// bf16 form: one wave per problem t; a, b: [T][32][K] bf16 bits; k-slots 16m + 8h .. +7
// of instruction m for lane half h; same result layout as mfma_kernel.
__global__ void mfma_bf16_kernel(const uint16_t* a, const uint16_t* b, float* raw, int K) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  const int t = blockIdx.x, l = threadIdx.x;
  const int r = l & 31, h = l >> 5;
  f32x16 acc = {0};
  for (int m = 0; m < K / 16; ++m) {
    const i32x4 av = *(const i32x4*)(a + ((size_t)t * 32 + r) * K + 16 * m + 8 * h);
    const i32x4 bv = *(const i32x4*)(b + ((size_t)t * 32 + r) * K + 16 * m + 8 * h);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                  acc, 0, 0, 0);
  }
  for (int q = 0; q < 16; ++q) {
    const int row = 8 * (q >> 2) + 4 * h + (q & 3);
    raw[((size_t)t * 32 + row) * 32 + r] = acc[q];
  }
}

// The older FP8 forms (CDNA3 instructions, kept on gfx950): one wave per problem t.
// form 0: v_mfma_f32_32x32x16_fp8_fp8, lane l feeds row l % 32, k-slots 8(l / 32) .. +7 of
//         each 16-wide chunk; result layout as mfma_kernel.
// form 1: v_mfma_f32_16x16x32_fp8_fp8, lane l feeds row l % 16, k-slots 8(l / 16) .. +7 of
//         each 32-wide chunk; result layout as mfma16_kernel.
__global__ void mfma_fp8_legacy_kernel(int form, const uint8_t* a, const uint8_t* b, float* raw, int K) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int t = blockIdx.x, l = threadIdx.x;
  if (form == 0) {
    const int r = l & 31, h = l >> 5;
    f32x16 acc = {0};
    for (int m = 0; m < K / 16; ++m) {
      const long av = *(const long*)(a + ((size_t)t * 32 + r) * K + 16 * m + 8 * h);
      const long bv = *(const long*)(b + ((size_t)t * 32 + r) * K + 16 * m + 8 * h);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(av, bv, acc, 0, 0, 0);
    }
    for (int q = 0; q < 16; ++q) {
      const int row = 8 * (q >> 2) + 4 * h + (q & 3);
      raw[((size_t)t * 32 + row) * 32 + r] = acc[q];
    }
  } else {
    const int r = l & 15, g = l >> 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int m = 0; m < K / 32; ++m) {
      const long av = *(const long*)(a + ((size_t)t * 16 + r) * K + 32 * m + 8 * g);
      const long bv = *(const long*)(b + ((size_t)t * 16 + r) * K + 32 * m + 8 * g);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av, bv, acc, 0, 0, 0);
    }
    for (int i = 0; i < 4; ++i) raw[((size_t)t * 16 + 4 * g + i) * 16 + r] = acc[i];
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

// Vector-ALU issue rate against occupancy: every wave runs `iters` iterations of one
// pattern on 32 elements per lane; cycles[w] = shader-clock ticks (s_memtime) of wave w over
// the loop, ticks[w] = 100 MHz real-time ticks over the same loop.
template <int pattern>
__global__ __launch_bounds__(256, 8) void valu_rate_kernel(int iters, const int* seed, float* sink,
                                                        unsigned long long* cycles, unsigned long long* ticks,
                                                        float a, float b) {
  const int tid = threadIdx.x, lane = tid & 63;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = (float)(seed[(tid + 5 * i) & 255] & 1023) * 1e-4f;
  unsigned w[4] = {};
  float sum = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (pattern == 0) {          // 32 independent v_fma_f32
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = __builtin_fmaf(x[i], a, b);
    } else if constexpr (pattern == 1) {   // 32 independent v_exp_f32
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
    } else {                     // the softmax core: fma -> exp -> pairwise row sum, 16 E4M3 casts
      float s2 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * i], a, -b));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * i + 1], a, -b));
        s2 += p0 + p1;
        w[i & 3] = (i >> 2) & 1 ? __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, w[i & 3], true)
                                : __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, w[i & 3], false);
      }
      sum += s2;
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = x[i] + 1e-7f;
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float r = sum;
#pragma unroll
  for (int i = 0; i < 32; ++i) r += x[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) r += (float)w[i];
  sink[(size_t)blockIdx.x * blockDim.x + tid] = r;
  if (lane == 0) {
    const size_t wv = (size_t)blockIdx.x * (blockDim.x >> 6) + (tid >> 6);
    cycles[wv] = t1 - t0;
    ticks[wv] = r1 - r0;
  }
}

// Streaming read: thread t reads the 16-byte words t, t + S, t + 2S, ... (S = all threads)
// and XORs them, eight loads in flight per step; out[t] = the XOR of its four lanes.
__global__ __launch_bounds__(256) void stream_read_kernel(const i32x4* __restrict__ in, long n16, int* out) {
  const long stride = (long)gridDim.x * blockDim.x;
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  i32x4 acc = {0, 0, 0, 0};
  for (; i + 7 * stride < n16; i += 8 * stride) {
    i32x4 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = __builtin_nontemporal_load(in + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= w[u];
  }
  for (; i < n16; i += stride) acc ^= in[i];
  out[(long)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" int hw_probe_stream_read(const void* in, long bytes, int blocks, int* out, void* stream) {
  if (!in || !out || bytes <= 0 || bytes % 16 != 0 || blocks <= 0 || (reinterpret_cast<uintptr_t>(in) & 15) != 0)
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const i32x4*>(in), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int hw_probe_throughput(int kind, int blocks, int iters, const int* seed, float* sink, float* clock,
                                   void* stream) {
  if (kind < 0 || kind > 3 || blocks <= 0 || iters <= 0 || !seed || !sink || !clock) return -1;
  hipLaunchKernelGGL(throughput_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, kind, iters, seed,
                     sink, clock);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int hw_probe_valu_rate(int pattern, int waves_per_simd, int cus, int iters, const int* seed, float* sink,
                                  unsigned long long* cycles, unsigned long long* ticks, void* stream) {
  if (pattern < 0 || pattern > 2 || waves_per_simd <= 0 || waves_per_simd > 8 || cus <= 0 || iters <= 0 || !seed ||
      !sink || !cycles || !ticks)
    return -1;
  const dim3 grid(cus * waves_per_simd), block(256);
  if (pattern == 0)
    hipLaunchKernelGGL(valu_rate_kernel<0>, grid, block, 0, (hipStream_t)stream, iters, seed, sink, cycles, ticks,
                       0.5f, 0.25f);
  else if (pattern == 1)
    hipLaunchKernelGGL(valu_rate_kernel<1>, grid, block, 0, (hipStream_t)stream, iters, seed, sink, cycles, ticks,
                       0.5f, 0.25f);
  else
    hipLaunchKernelGGL(valu_rate_kernel<2>, grid, block, 0, (hipStream_t)stream, iters, seed, sink, cycles, ticks,
                       0.5f, 0.25f);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int hw_probe_mfma_fp8_legacy_dots(int form, const unsigned char* a, const unsigned char* b, float* raw,
                                            int T, int K, void* stream) {
  if ((form != 0 && form != 1) || !a || !b || !raw || T <= 0 || K <= 0 || K % 32 || K > 4096) return -1;
  if ((((uintptr_t)a) | ((uintptr_t)b)) & 7) return -1;
  hipLaunchKernelGGL(mfma_fp8_legacy_kernel, dim3(T), dim3(64), 0, (hipStream_t)stream, form, a, b, raw, K);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int hw_probe_mfma_bf16_dots(const unsigned short* a, const unsigned short* b, float* raw, int T, int K,
                                       void* stream) {
  if (!a || !b || !raw || T <= 0 || K <= 0 || K % 16 || K > 4096) return -1;
  if ((((uintptr_t)a) | ((uintptr_t)b)) & 15) return -1;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(T), dim3(64), 0, (hipStream_t)stream, a, b, raw, K);
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

extern "C" int hw_probe_mfma16_dots(const unsigned char* a, const unsigned char* b, float* raw, int T, int kch,
                                    void* stream) {
  if (!a || !b || !raw || T <= 0 || kch <= 0 || kch > 32) return -1;
  if ((((uintptr_t)a) | ((uintptr_t)b)) & 15) return -1;
  hipLaunchKernelGGL(mfma16_kernel, dim3(T), dim3(64), 0, (hipStream_t)stream, a, b, raw, kch);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
