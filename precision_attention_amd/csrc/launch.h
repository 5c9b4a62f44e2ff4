// Internal interface between the C ABI layer (api.hip) and the kernels (fwd.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8attn {

// Everything a forward / count launch needs, passed by value as the kernel argument.
struct Params {
  const uint8_t* q;                 // [B][H][N][d] E4M3
  const uint8_t* k;                 // [B][Hkv][N][d] E4M3
  const uint8_t* v;                 // [B][Hkv][N][d] E4M3 (unused by a count-only launch)
  float* o;                         // [B][H][N][d] fp32 (unused by a count-only launch)
  const float* q_descale;           // [B*H]
  const float* k_descale;           // [B*Hkv]
  const float* v_descale;           // [B*Hkv]
  unsigned long long* counts;       // [4] (launches that count)
  int B, H, Hkv, N;
  int causal, reverse, n_sink;
  float S;                          // static P scale
  float log2_S;                     // exact log2(S) when S is a power of two
  float log2e_rsqrt_d;              // log2(e)/sqrt(d), rounded once to fp32
};

// Rows of queries per workgroup (4 waves x 32 rows).
constexpr int kRowsPerWave = 32;
constexpr int kWaves = 4;
constexpr int kBlockM = kRowsPerWave * kWaves;
constexpr int kKvBlock = 64;

inline int64_t num_workgroups(const Params& p) {
  const int64_t tiles = (p.N + kBlockM - 1) / kBlockM;
  return (int64_t)p.B * p.H * tiles;
}

hipError_t launch_fwd(const Params& p, int d, bool pow2_scale, hipStream_t stream);
hipError_t launch_count(const Params& p, int d, bool pow2_scale, hipStream_t stream);
hipError_t launch_fwd_count(const Params& p, int d, bool pow2_scale, hipStream_t stream);

}  // namespace fp8attn
