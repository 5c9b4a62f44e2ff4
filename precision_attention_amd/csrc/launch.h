// Internal interface between the C ABI layer (api.hip) and the kernels (fwd.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8attn {

// Everything a forward / count launch needs, passed by value as the kernel argument.
struct Params {
  const uint8_t* q;                 // [B][H][N][d] E4M3
  const uint8_t* k;                 // [B][Hkv][N][d] E4M3
  const uint8_t* kx;                // the same keys as bf16 (exact Q.K^T launches): per head and 64-key
                                    // block, d / 16 slices [64 rows][d 16m .. 16m + 15]
  const uint8_t* v;                 // [B][Hkv][N][d] E4M3 (unused by a count-only launch)
  float* o;                         // [B][H][N][d] fp32 (unused by a count-only launch)
  const float* q_descale;           // [B*H]
  const float* k_descale;           // [B*Hkv]
  const float* v_descale;           // [B*Hkv]
  unsigned long long* counts;       // [4] (launches that count)
  unsigned long long pairs;         // unmasked non-sink (query, key) pairs, all heads
  unsigned long long pairs_sink;    // of which in KV blocks holding a sink token
  int B, H, Hkv, N;
  int causal, reverse, n_sink;
  int sink_last;                    // reverse walk, block 0 as [n_sink, 64) then [0, n_sink)
  int qden;                         // row sum of the decoded cast operand (else of P~ S)
  int exact_qk;                     // Q.K^T on the bf16 matrix cores from kx (exact products)
  int head_major;                   // grid order within an XCD: all tiles of a head together
  float S;                          // static P scale
  float log2_S;                     // exact log2(S) when S is a power of two
  float log2e_rsqrt_d;              // log2(e)/sqrt(d), rounded once to fp32
};

// Each wave owns 32 query rows; a workgroup has 4 waves (128 rows), one per SIMD, which
// share every K/V block staged in LDS. Several workgroups share a CU (see the register
// budget below), so one workgroup's barrier stall is covered by the others.
constexpr int kRowsPerWave = 32;
constexpr int kKvBlock = 64;

constexpr int waves_for(int) { return 4; }
// waves per walk group of the two-group forward (64-row tiles)
constexpr int kPairWaves = 2;
// Register budget: at most 512 / n VGPRs per lane lets n waves share a SIMD.
constexpr int min_waves_per_simd(int d) { return d == 256 ? 2 : 3; }
constexpr int block_m_for(int d) { return kRowsPerWave * waves_for(d); }

inline int64_t num_workgroups(const Params& p, int d) {
  const int bm = block_m_for(d);
  const int64_t tiles = (p.N + bm - 1) / bm;
  return (int64_t)p.B * p.H * tiles;
}

// Split-KV decode: one query row per (batch, head), all N keys, n_split key ranges.
struct DecodeParams {
  const uint8_t* q;                 // [B][H][d] E4M3
  const uint8_t* k;                 // [B][Hkv][N][d] E4M3
  const uint8_t* v;                 // [B][Hkv][N][d] E4M3
  float* o;                         // [B][H][d] fp32
  float* ws;                        // [B][H][n_split] records of decode_record_floats(d)
  const float* q_descale;           // [B*H]
  const float* k_descale;           // [B*Hkv]
  const float* v_descale;           // [B*Hkv]
  int B, H, Hkv, N;
  int n_split;                      // key ranges (1 .. N / 64)
  int n_qgroups;                    // groups of up to 32 query heads per KV head
  int reverse;
  float S, log2_S, log2e_rsqrt_d;
};

// floats per (row, split) record of the decode workspace: acc[d], m, l, 2 unused (16 B aligned)
constexpr int decode_record_floats(int d) { return d + 4; }

hipError_t launch_fwd(const Params& p, int d, bool pow2_scale, hipStream_t stream);
// K [B][Hkv][N][d] E4M3 -> kx, the same values as bf16 (exact) in the slice layout of
// Params::kx, for the exact Q.K^T launches
hipError_t launch_keys_to_bf16(const uint8_t* k, uint8_t* kx, int64_t n_elements, int d, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int d, bool pow2_scale, hipStream_t stream);
hipError_t launch_count(const Params& p, int d, bool pow2_scale, hipStream_t stream);
hipError_t launch_fwd_count(const Params& p, int d, bool pow2_scale, hipStream_t stream);

}  // namespace fp8attn
