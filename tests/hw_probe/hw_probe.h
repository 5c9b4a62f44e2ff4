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

/* raw[t][i][j] = sum_c a[t][i][c] * b[t][j][c] over c < 128*kch, computed by kch chained
 * v_mfma_f32_16x16x128_f8f6f4 with the k-slots of each instruction taken as the 128
 * consecutive c values; a, b: [T][16][128*kch] E4M3 codes, raw: [T][16][16] fp32. */
int hw_probe_mfma16_dots(const unsigned char* a, const unsigned char* b, float* raw, int T, int kch,
                         void* stream);

/* raw[t][i][j] = sum_c a[t][i][c] * b[t][j][c] over c < K (a multiple of 16), computed by
 * K/16 chained v_mfma_f32_32x32x16_bf16; a, b: [T][32][K] bf16 bit patterns (16-byte
 * aligned), raw: [T][32][32] fp32. */
int hw_probe_mfma_bf16_dots(const unsigned short* a, const unsigned short* b, float* raw, int T, int K,
                            void* stream);

/* The older FP8 forms: raw[t][i][j] = sum_c a[t][i][c] * b[t][j][c] over c < K (a multiple
 * of 32), computed by chained instructions with the k-slots of each instruction taken as
 * consecutive c values. form 0: v_mfma_f32_32x32x16_fp8_fp8 (a, b: [T][32][K] E4M3 codes,
 * raw: [T][32][32]); form 1: v_mfma_f32_16x16x32_fp8_fp8 (a, b: [T][16][K], raw:
 * [T][16][16]). a, b 8-byte aligned. */
int hw_probe_mfma_fp8_legacy_dots(int form, const unsigned char* a, const unsigned char* b, float* raw, int T,
                                  int K, void* stream);

/* Streaming read of `bytes` (a multiple of 16) at `in` (16-byte aligned): `blocks`
 * workgroups of 256 threads read the buffer once in 16-byte words at a grid stride, eight
 * loads in flight per thread, and out[blocks*256] receives each thread's XOR of its words
 * (so no load is dead code; the XOR of all of out is the XOR of the buffer's 32-bit words). */
int hw_probe_stream_read(const void* in, long bytes, int blocks, int* out, void* stream);

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

/* Vector-ALU issue rate against occupancy. cus * waves_per_simd workgroups of 256 threads
 * (one wave per SIMD each, so that on `cus` compute units every SIMD holds waves_per_simd
 * waves; 1 <= waves_per_simd <= 8) run `iters` iterations of
 *   pattern 0: 32 independent v_fma_f32;
 *   pattern 1: 32 independent v_exp_f32;
 *   pattern 2: the softmax core: 32 v_fma_f32 -> v_exp_f32, a pairwise row sum (32 v_add_f32)
 *              and 16 v_cvt_pk_fp8_f32, plus 32 v_add_f32 that move the inputs.
 * sink[blocks*256] receives one float per thread; cycles[w] and ticks[w] receive, for wave w
 * (blocks*4 waves), the shader-clock ticks (s_memtime) and the 100 MHz real-time ticks
 * (s_memrealtime) over its loop. seed: 256 ints. */
int hw_probe_valu_rate(int pattern, int waves_per_simd, int cus, int iters, const int* seed, float* sink,
                       unsigned long long* cycles, unsigned long long* ticks, void* stream);

#ifdef __cplusplus
}
#endif
#endif
