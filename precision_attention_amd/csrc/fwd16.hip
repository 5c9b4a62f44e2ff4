// FP8 (OCP E4M3) P-cast attention forward with 16 query rows per wave, d = 128, for small
// grids, where the 32-row kernel (fwd.hip) leaves compute units idle or, with causal
// masking, unevenly loaded (fwd_tile_rows has the rule). The computation is the one of
// fwd.hip ("P-Cast Precision in FP8 Attention", gist.science technical summary, section
// 1): online softmax per 64-key block, P~ S cast to E4M3 before the P.V product, S divided
// out at the end, blocks walked forward or reverse, the collapse count of
// fp8_attn_p_collapse_count.
//
// Layout of the work on the chip
// ------------------------------
// * One workgroup = 4 waves = 64 query rows of one (batch, head); each wave owns 16 rows.
//   The grid has twice the workgroups of the 32-row kernel, each with half the work, so a
//   small grid reaches more compute units and a causal one spreads its long tiles better.
//   Where two workgroups share a compute unit, each SIMD runs waves of different
//   workgroups, which the barrier of each step does not hold in phase. The 4 waves share
//   each 64-key K/V block staged in LDS (two DMA instructions each).
// * S^T = K . Q^T on v_mfma_f32_16x16x128_f8f6f4, one instruction per 16 keys (k = d =
//   128; it accumulates as two chained 64-slot halves, like the 32x32x64 form, so the
//   logits obey the same error bound). Lane l holds query col = l % 16 and, for
//   g = l / 16, keys 16t + 4g + i (t = 0..3, i = 0..3): 16 scores. The row max is
//   lane-local, then one v_permlane16_swap and one v_permlane32_swap across the four lane
//   groups that share a query.
// * The 16 probabilities are cast four per dword; the dwords of tiles 2c and 2c + 1 are
//   the B operand of O^T += V^T . P^T on v_mfma_f32_16x16x32_fp8_fp8 for key chunk c:
//   k-slot 8g + e holds key 32c + 16 (e / 4) + 4g + e % 4.
// * The A operand (16 output columns x 32 keys) comes from the V tile through
//   ds_read_b64_tr_b8: within a 16-lane group, lane 2e + b reads 8 bytes (columns
//   16u + 8b ..) of the key that k-slot 8g + e stands for, and the transpose hands each
//   lane the 8 keys of its own column. O^T holds one query per lane (column l % 16), so the
//   rescale by alpha stays lane-local.
// * LDS rows are XOR-swizzled at 16-byte granularity: K like fwd.hip ((j ^ j/8) % 8), which
//   keeps 16 consecutive rows read at one chunk on distinct banks; V with (j ^ j/16) % 8,
//   which does the same for the 16 rows two lane groups read per transposed load.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "launch.h"
#include "kernel_common.h"
#include "fwd_common.h"

namespace fp8attn {
namespace {

// 16 x 16 outputs from 16 x 128 E4M3 operands (format 0 for both, zero scales).
__device__ __forceinline__ f32x4 mfma16_k128(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// 16 x 16 outputs from 16 x 32 E4M3 operands (8 codes per lane each).
__device__ __forceinline__ f32x4 mfma16_k32(long a, long b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

constexpr int kWaves16 = 4;
constexpr int kRows16 = 16;

template <bool POW2, bool OUT, bool CNT>
__global__ FP8ATTN_BOUNDS(64 * kWaves16, 2) void fwd16_kernel(const Params p) {
  constexpr int D = 128;
  constexpr int kBlockM = kRows16 * kWaves16;   // 64 rows
  constexpr int TILE = kKvBlock * D;            // 8 KiB
  constexpr int DMA_PER_WAVE = TILE / 1024 / kWaves16;
  static_assert(DMA_PER_WAVE * kWaves16 * 1024 == TILE, "whole DMA instructions per wave and tile");
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[OUT ? TILE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[OUT ? TILE : 16];
  auto kbuf = [&](int i) __attribute__((always_inline)) { return i ? kb1 : kb0; };
  auto vbuf = [&](int i) __attribute__((always_inline)) { return i ? vb1 : vb0; };
  auto swzk = [](int j) { return (j ^ (j >> 3)) & 7; };
  auto swzv = [](int j) { return (j ^ (j >> 4)) & 7; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
  const int col = lane & 15;
  const int grp = lane >> 4;

  const int ntiles = (p.N + kBlockM - 1) / kBlockM;
  int b, h, hk, qt;
  map_tile(p, ntiles, b, h, hk, qt);

  const int i0 = qt * kBlockM;
  const int r0 = i0 + wave * kRows16;
  const bool wave_valid = r0 < p.N;             // N is a multiple of 64: all 16 rows or none
  const int nkb = p.N / kKvBlock;
  const int last_row = min(i0 + kBlockM, p.N) - 1;
  const int wg_nb = p.causal ? (last_row / kKvBlock + 1) : nkb;
  const int diag = r0 / kKvBlock;
  const int wave_nb = p.causal ? (diag + 1) : nkb;

  const size_t q_head = ((size_t)b * p.H + h) * (size_t)p.N * D;
  const size_t kv_head = ((size_t)b * p.Hkv + hk) * (size_t)p.N * D;
  const uint8_t* __restrict__ Kg = p.k + kv_head;
  const uint8_t* __restrict__ Vg = p.v + kv_head;

  // logits in log2 units: s' = raw . c with c = qd kd log2(e) / sqrt(d)
  const float c = p.q_descale[b * p.H + h] * p.k_descale[b * p.Hkv + hk] * p.log2e_rsqrt_d;

  // Q operand (B of S^T = K Q^T): lane (col, grp) holds q[r0 + col][32 grp .. + 32]
  i32x8 qop = {0, 0, 0, 0, 0, 0, 0, 0};
  if (wave_valid) {
    const uint8_t* qrow = p.q + q_head + (size_t)(r0 + col) * D + 32 * grp;
    const i32x4 lo = *(const i32x4*)qrow;
    const i32x4 hi = *(const i32x4*)(qrow + 16);
    qop = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }

  // ---- per-lane LDS byte offsets, computed once
  // K operand of key tile t: row 16t + col, 16-byte chunks 2 grp and 2 grp + 1
  int koff[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = 16 * t + col;
      koff[t][e] = j * D + (((2 * grp + e) ^ swzk(j)) << 4);
    }
  // V^T operand of output tile u, key chunk 0: lane (2e + hb) of its group reads the 8
  // bytes at columns 16u + 8 hb of key 16 (e / 4) + 4 grp + e % 4. Chunk 1 (keys + 32)
  // flips swizzle bit 1, so it reads like tile u ^ 2 of chunk 0, 32 rows further.
  int voff[8];
  {
    const int e = col >> 1, hb = col & 1;
    const int row = 16 * (e >> 2) + 4 * grp + (e & 3);
#pragma unroll
    for (int u = 0; u < 8; ++u) voff[u] = row * D + ((u ^ swzv(row)) << 4) + 8 * hb;
  }
  // DMA: instruction ii = wave + 4r of a tile covers LDS rows 8 ii .. + 7; lane L lands on
  // LDS bytes 16 L of that KiB (row 8 ii + L / 8, slot L % 8) and fetches the chunk stored there
  int goffk[DMA_PER_WAVE], goffv[DMA_PER_WAVE];
#pragma unroll
  for (int r = 0; r < DMA_PER_WAVE; ++r) {
    const int j = 8 * (wave + kWaves16 * r) + lane / 8, cs = lane % 8;
    goffk[r] = j * D + ((cs ^ swzk(j)) << 4);
    goffv[r] = j * D + ((cs ^ swzv(j)) << 4);
  }
  auto dma = [&](int blk, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < DMA_PER_WAVE; ++r) {
      const int dst = 1024 * (wave + kWaves16 * r);
      lds_dma16(Kg, p.N * D, kbuf(buf) + dst, goffk[r], blk * kKvBlock * D);
      if (OUT) lds_dma16(Vg, p.N * D, vbuf(buf) + dst, goffv[r], blk * kKvBlock * D);
    }
  };
  auto dma_wait_sync = []() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
  };
  auto block_of = [&](int n) { return p.reverse ? (wg_nb - 1 - n) : n; };
  auto active = [&](int n) { return wave_valid && block_of(n) < wave_nb; };

  // running max (log2 units), this lane's share of the row sum of P~ S, O^T
  float m_run = -1e30f;
  float l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  unsigned cnt_zero = 0, cnt_zero_sink = 0;
  const float bias_s = POW2 ? p.log2_S : 0.f;
  const int i_row = r0 + col;
  int pw[4] = {0, 0, 0, 0};   // E4M3 codes of P: word t holds keys 16t + 4 grp .. + 3

  // ---- S^T for the four 16-key tiles of the block in Ks; all operand reads first
  auto qk = [&](const uint8_t* Ks, f32x4 (&s)[4]) __attribute__((always_inline)) {
    i32x8 ko[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const i32x4 lo = *(const i32x4*)(Ks + koff[t][0]);
      const i32x4 hi = *(const i32x4*)(Ks + koff[t][1]);
      ko[t] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = mfma16_k128(ko[t], qop, f32x4{0.f, 0.f, 0.f, 0.f});
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // MFMA
  };

  // ---- online softmax of block blk: running max and sum, rescale of O, E4M3 cast, counts
  auto softmax = [&](f32x4 (&s)[4], int blk) __attribute__((always_inline)) {
    if (p.causal && blk >= diag) {
      // key offset 16t + 4 grp + i of the block against the query's own offset
      const int hi_rel = min(i_row - blk * kKvBlock, kKvBlock - 1) - 4 * grp;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * t + i > hi_rel) s[t][i] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = __builtin_elementwise_maximum(mx, s[t][i]);
    {
      // the four lane groups of a query trade maxima: a register swapped with itself
      // leaves the even 16-lane rows' values in every lane of [0] and the odd rows' in [1]
      // (permlane16), then the lower half's and the upper half's (permlane32)
      const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = __builtin_elementwise_maximum(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
      const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = __builtin_elementwise_maximum(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    }
    const float m_new = __builtin_elementwise_maximum(m_run, mx * c);
    const float alpha = fast_exp2(m_run - m_new);     // 0 on the first block
    m_run = m_new;
    const float bias = bias_s - m_new;

    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x0 = fast_exp2(fmaf(s[t][0], c, bias));
      float x1 = fast_exp2(fmaf(s[t][1], c, bias));
      float x2 = fast_exp2(fmaf(s[t][2], c, bias));
      float x3 = fast_exp2(fmaf(s[t][3], c, bias));
      if (!POW2) { x0 *= p.S; x1 *= p.S; x2 *= p.S; x3 *= p.S; }
      const float part = (x0 + x1) + (x2 + x3);
      lsum = t == 0 ? part : lsum + part;
      // the first cast writes the low half and keeps the rest (the previous block's
      // codes, dead by now); the second replaces it
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, pw[t], false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
      pw[t] = w;
    }
    l_run = alpha * l_run + lsum;

    if (CNT) {
      const int jb = blk * kKvBlock;
      const bool sink_block = jb < p.n_sink;
      unsigned z;
      if (__builtin_expect((p.causal && blk >= diag) || sink_block, 0)) {
        // only keys j in [n_sink, hi] count (hi = the query for causal attention); codes are
        // 0x00..0x7E, so byte + 0x7F leaves bit 7 clear exactly for a zero code
        const int hi = p.causal ? i_row : p.N - 1;
        const int n_hi = hi - jb - 4 * grp + 1, n_lo = p.n_sink - jb - 4 * grp;
        z = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const unsigned zero = ~((unsigned)pw[t] + 0x7F7F7F7Fu) & 0x80808080u;
          const unsigned live = bytes_below(n_hi - 16 * t) & ~bytes_below(n_lo - 16 * t);
          z += __builtin_popcount(zero & live);
        }
        cnt_zero_sink += z & (0u - (unsigned)sink_block);
      } else {
        // |b - 1| + |b - 127| is 126 for a code b in [1, 126] and 128 for b = 0
        unsigned sad = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          sad = __builtin_amdgcn_sad_u8((unsigned)pw[t], 0x01010101u, sad);
          sad = __builtin_amdgcn_sad_u8((unsigned)pw[t], 0x7F7F7F7Fu, sad);
        }
        z = (sad - 4u * 4u * 126u) >> 1;
      }
      cnt_zero += z;
    }
    if (OUT) {
      // alpha == 1 exactly when no row's max moved; a multiply by 1 changes nothing
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] *= alpha;
      }
    }
  };

  // ---- V^T operands of the block: all 16 read before the softmax, so that their LDS
  // latency is spent under it (tile u of key chunk c at index 8c + u)
  auto read_v = [&](const uint8_t* Vs, long (&vop)[16]) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2*)(Vs + voff[cc ? (u ^ 2) : u] + cc * 32 * D));
        vop[8 * cc + u] = __builtin_bit_cast(long, r);
      }
  };
  // ---- O^T += V^T . P^T, key chunk c from the codes of tiles 2c and 2c + 1
  auto pv = [&](const long (&vop)[16]) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const long pb = (long)(((unsigned long)(unsigned)pw[2 * cc + 1] << 32) | (unsigned)pw[2 * cc]);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = mfma16_k32(vop[8 * cc + u], pb, acc[u]);
    }
  };

  dma(block_of(0), 0);
  dma_wait_sync();
  // step n on buffers `cur` (a constant at each call site); block n + 1 lands in the other
  auto step = [&](int n, int cur) __attribute__((always_inline)) {
    if (n + 1 < wg_nb) dma(__builtin_amdgcn_readfirstlane(block_of(n + 1)), cur ^ 1);
    if (active(n)) {
      f32x4 s[4];
      qk(kbuf(cur), s);
      long vop[16];
      if (OUT) read_v(vbuf(cur), vop);
      softmax(s, block_of(n));
      if (OUT) pv(vop);
    }
    dma_wait_sync();
  };
  for (int n = 0; n < wg_nb; n += 2) {
    step(n, 0);
    if (n + 1 < wg_nb) step(n + 1, 1);
  }

  if (CNT) {
    if (!wave_valid) cnt_zero = cnt_zero_sink = 0;
    __shared__ unsigned red[2][kWaves16];
    unsigned v0 = cnt_zero, v1 = cnt_zero_sink;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      v0 += __shfl_xor(v0, off);
      v1 += __shfl_xor(v1, off);
    }
    if (lane == 0) {
      red[0][wave] = v0;
      red[1][wave] = v1;
    }
    __syncthreads();
    if (tid == 0) {
      unsigned long long zt = 0, zs = 0;
#pragma unroll
      for (int w = 0; w < kWaves16; ++w) {
        zt += red[0][w];
        zs += red[1][w];
      }
      if (zt) atomicAdd(p.counts + 0, zt);
      if (zs) atomicAdd(p.counts + 1, zs);
    }
  }
  if (!wave_valid) return;
  if (OUT) {
    // O = acc vd / (S l); the four lane groups of a query hold partial row sums
    const float l2 = l_run + __shfl_xor(l_run, 16);
    const float l_tot = l2 + __shfl_xor(l2, 32);
    const float scale = p.v_descale[b * p.Hkv + hk] / l_tot;
    float* orow = p.o + q_head + (size_t)i_row * D + 4 * grp;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const f32x4 val = {acc[u][0] * scale, acc[u][1] * scale, acc[u][2] * scale, acc[u][3] * scale};
      *(f32x4*)(orow + 16 * u) = val;
    }
  }
}

template <bool OUT, bool CNT>
void launch16(const Params& p, bool pow2, hipStream_t stream) {
  const int64_t tiles = (p.N + kRows16 * kWaves16 - 1) / (kRows16 * kWaves16);
  const dim3 grid((unsigned)((int64_t)p.B * p.H * tiles)), block(64 * kWaves16);
  if (pow2) hipLaunchKernelGGL((fwd16_kernel<true, OUT, CNT>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((fwd16_kernel<false, OUT, CNT>), grid, block, 0, stream, p);
}

}  // namespace

hipError_t launch_fwd16(const Params& p, bool pow2, bool out, bool count, hipStream_t stream) {
  if (out && count) launch16<true, true>(p, pow2, stream);
  else if (out) launch16<true, false>(p, pow2, stream);
  else if (count) launch16<false, true>(p, pow2, stream);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fp8attn
