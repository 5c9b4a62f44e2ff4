/*
 * hw_probe.h -- test-support C ABI that runs single gfx950 instructions on caller data,
 * so the test suite can pin the CPU oracle's E4M3 codec and its model of the FP8 matrix
 * core against the hardware. Not part of the attention library.
 *
 * All pointers are DEVICE pointers; calls are asynchronous on `stream` (a hipStream_t
 * passed as void*, NULL = default). Return 0 on success, -1 for invalid arguments
 * (checked before any HIP call), -3 if HIP reports a launch error.
 */
#ifndef FP8ATTN_HW_PROBE_H
#define FP8ATTN_HW_PROBE_H
#ifdef __cplusplus
extern "C" {
#endif

/* out[i] = E4M3 code of in[i] via v_cvt_pk_fp8_f32 (hardware rounding), i < n; n even. */
int hw_probe_cvt_e4m3(const float* in, unsigned char* out, long n, void* stream);

/* raw[t][i][j] = sum_c a[t][i][c] * b[t][j][c] over c < 64*kch, computed by kch chained
 * v_mfma_f32_32x32x64_f8f6f4 with the k-slots of each instruction taken as the 64
 * consecutive c values; a, b: [T][32][64*kch] E4M3 codes, raw: [T][32][32] fp32. */
int hw_probe_mfma_dots(const unsigned char* a, const unsigned char* b, float* raw, int T, int kch,
                       void* stream);

/* Throughput kernel for the roofline denominators. Each of `blocks` workgroups of 512
 * threads (8 waves, 2 per SIMD) runs `iters` iterations of
 *   kind 0: 8 v_mfma_f32_32x32x64_f8f6f4 on 4 independent accumulators (131072 FLOP each);
 *   kind 1: 32 v_exp_f32, each followed by one v_sub_f32 that keeps the chain bounded;
 *   kind 2: both in the same wave;
 *   kind 3: waves 0-3 the MFMA part, waves 4-7 the exp part (split across waves).
 * sink[blocks*512] receives one float per thread (so no work is dead code). clock[blocks]
 * receives, per workgroup, shader-clock ticks per 100 MHz real-time tick measured over the
 * loop by wave 0 (s_memtime / s_memrealtime); multiply by 1e8 for Hz. seed: 256 ints. */
int hw_probe_throughput(int kind, int blocks, int iters, const int* seed, float* sink, float* clock,
                        void* stream);

#ifdef __cplusplus
}
#endif
#endif
