// FP8 (OCP E4M3) P-cast attention forward for gfx950 (MI355X).
//
// Computation: "P-Cast Precision in FP8 Attention" (gist.science technical summary),
// section 1: Q.K^T and P.V on E4M3 operands with an online softmax (running max m
// updated per KV block), P~ multiplied by a static scale S and cast to E4M3 before the
// P.V product, S divided back out in the epilogue, KV blocks walked forward or reverse.
//
// Layout of the work on the chip
// ------------------------------
// * One workgroup = 4 waves = 128 query rows of one (batch, head); each wave owns 32
//   rows. K/V blocks of 64 keys stream through LDS (two stages, double-buffered). Small
//   d = 128 grids run fwd_pair_kernel instead: 64 rows per workgroup, whose KV walk two
//   groups of two waves split (fwd_body, NG = 2).
// * Both GEMMs use v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3 -> fp32). That instruction
//   truncates small products inside its adder tree; the exact-Q.K^T variant (QX) forms
//   S^T on v_mfma_f32_32x32x16_bf16 instead, from keys converted once to bf16 and queries
//   converted in registers (every E4M3 value is a bf16 value, the products are exact and
//   the sum is accumulated in fp32), with the same 32x32 result layout.
// * Q.K^T is computed transposed, S^T = K . Q^T (A = 32 keys of K, B = 32 query rows of
//   Q), so in the result each lane holds one query row: lane l has query col = l % 32
//   and, for half = l / 32, the keys 8*(r/4) + 4*half + (r%4), r = 0..15, of each
//   32-key tile. Row max and row sum are lane-local plus one exchange between the two
//   lane halves; the running state (m, l) lives in the lane.
// * P never leaves registers: the 32 fp32 probabilities of a lane are packed to E4M3
//   four per dword (v_cvt_pk_fp8_f32), and those 8 dwords are, as they stand, the B
//   operand of O^T = V^T . P^T (32 output columns x 32 query rows per MFMA).
// * V^T comes straight from the V tile in LDS with ds_read_b64_tr_b8: within each
//   16-lane group, lane t receives byte t%8 of the 8-byte rows supplied by lanes
//   2e + t/8 (e = 0..7), so each lane gets 8 consecutive LDS rows of one column. The V
//   tile is stored with its key rows' bits 2 and 3 exchanged, which makes those LDS rows
//   the keys whose P the cast left in the matching bytes of the lane.
// * LDS rows are XOR-swizzled at 16-byte granularity (chunk ^ ((row ^ row/8) % 8)) so
//   that the 128-bit K reads, the transposing V reads and the DMA writes hit distinct
//   banks.
// * The MFMA operand k-slot order is only required to agree between A and B, so the d
//   index of Q and K and the key index of P and V may be permuted consistently.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <atomic>
#include <type_traits>

#include "launch.h"
#include "kernel_common.h"
#include "fwd_common.h"

namespace fp8attn {
namespace {

// OUT: compute and store O. CNT: count collapsed P casts (see fp8_attn_p_collapse_count).
// EXT: the options of fp8_attn_fwd_ex (sink split of block 0, quantized row sum); the
// launches without them run the kernel compiled without their branches. QX: Q.K^T on the
// bf16 matrix cores from the bf16 keys p.kx (d <= 128; three waves per SIMD).
// NG: walk groups. NG = 1: 4 waves, 128 query rows, each wave walks all of its rows' KV
// blocks. NG = 2: 4 waves, 64 query rows, two walk groups of 2 waves over the same rows;
// group g visits the walk positions g, g + 2, g + 4, ... and the groups trade each block's
// row maxima through LDS, so every block sees the running maximum of the sequential walk
// (the block maxima of all earlier positions) while each wave's chain of dependent blocks
// halves. The two partial (m, l, acc) states are merged once at the end. The four waves sit
// on the four SIMDs, so a second workgroup on the compute unit supplies each SIMD's second
// wave, in its own phase.
template <int D, bool POW2, bool OUT, bool CNT, bool EXT, bool QX, int NG>
__device__ __forceinline__ void fwd_body(const Params p) {
  static_assert(NG == 1 || (NG == 2 && D == 128 && !EXT && !QX), "walk groups: d = 128, plain options");
  constexpr int kWaves = NG == 1 ? waves_for(D) : kPairWaves;   // waves per walk group
  constexpr int kBlockM = kRowsPerWave * kWaves;
  constexpr int DM = D / 64;             // QK^T MFMAs per 32-key tile (k = 64 of d each)
  constexpr int DU = D / 32;             // 32-column output tiles
  constexpr int CH = D / 16;             // 16-byte chunks per row
  constexpr int SWZ = (CH >= 8 ? 8 : CH) - 1;
  auto swz = [](int j) { return swz_row<SWZ>(j); };
  constexpr int TILE = kKvBlock * D;     // bytes of one K or V block
  // staging: one LDS-DMA instruction moves 64 lanes x 16 bytes = 1 KiB of a tile
  constexpr int INST_PER_TILE = TILE / 1024;
  constexpr int RPW = (INST_PER_TILE + kWaves - 1) / kWaves;    // per wave and tile (at most)
  // K rows: D bytes of E4M3, or 2 D bytes of bf16 (QX, laid out in slices: below), in CHK
  // 16-byte chunks
  static_assert(!QX || D <= 128, "the exact Q.K^T variant holds d <= 128");
  constexpr int KROW = QX ? 2 * D : D;
  constexpr int CHK = KROW / 16;
  constexpr int TILE_K = kKvBlock * KROW;
  constexpr int INST_PER_TILE_K = TILE_K / 1024;
  constexpr int RPWK = (INST_PER_TILE_K + kWaves - 1) / kWaves;
  // Double buffers for K and V, four separate arrays so that the compiler can tell a DMA
  // into one buffer from reads of another: K(n), V(n) are read while block n + 1 lands.
  // (one set per walk group)
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[NG * TILE_K];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[NG * TILE_K];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[OUT ? NG * TILE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[OUT ? NG * TILE : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_g = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
  const int grp = NG == 1 ? 0 : wave_g / kWaves;                 // walk group
  const int wave = NG == 1 ? wave_g : wave_g % kWaves;           // rows 32 wave .. of the tile
  auto kbuf = [&](int i) __attribute__((always_inline)) { return (i ? kb1 : kb0) + (NG == 1 ? 0 : grp * TILE_K); };
  auto vbuf = [&](int i) __attribute__((always_inline)) {
    return (i ? vb1 : vb0) + (NG == 1 || !OUT ? 0 : grp * TILE);
  };
  const int col = lane & 31;
  const int half = lane >> 5;

  const int ntiles = (p.N + kBlockM - 1) / kBlockM;
  int b, h, hk, qt;
  map_tile(p, ntiles, b, h, hk, qt);

  const int i0 = qt * kBlockM;
  const int r0 = i0 + wave * kRowsPerWave;
  const bool wave_valid = r0 < p.N;
  const int nkb = p.N / kKvBlock;
  const int last_row = min(i0 + kBlockM, p.N) - 1;
  const int wg_nb = p.causal ? (last_row / kKvBlock + 1) : nkb;
  const int diag = r0 / kKvBlock;
  const int wave_nb = p.causal ? (diag + 1) : nkb;

  const size_t q_head = ((size_t)b * p.H + h) * (size_t)p.N * D;
  const size_t kv_head = ((size_t)b * p.Hkv + hk) * (size_t)p.N * D;
  const uint8_t* __restrict__ Kg = QX ? p.kx + 2 * kv_head : p.k + kv_head;
  const uint8_t* __restrict__ Vg = p.v + kv_head;

  // logits in log2 units: s' = raw . c with c = qd kd log2(e) / sqrt(d)
  const float c = p.q_descale[b * p.H + h] * p.k_descale[b * p.Hkv + hk] * p.log2e_rsqrt_d;

  // Q operand (B of S^T = K Q^T): lane (col, half) holds q[r0+col][64m + 32 half .. +32];
  // QX: the bf16 operand of instruction m, q[r0+col][16m + 8 half .. +8] converted
  constexpr int MX = D / 16;
  i32x8 qop[QX ? 1 : DM];
  i32x4 qopx[QX ? MX : 1];
  if (wave_valid) {
    if constexpr (QX) {
      const uint8_t* qrow = p.q + q_head + (size_t)(r0 + col) * D + 8 * half;
#pragma unroll
      for (int m = 0; m < MX; ++m) {
        const i32x2 w = *(const i32x2*)(qrow + 16 * m);
        const i32x2 lo = e4m3x4_to_bf16x4(w.x), hi = e4m3x4_to_bf16x4(w.y);
        qopx[m] = i32x4{lo.x, lo.y, hi.x, hi.y};
      }
    } else {
      const uint8_t* qrow = p.q + q_head + (size_t)(r0 + col) * D + 32 * half;
#pragma unroll
      for (int m = 0; m < DM; ++m) {
        const i32x4 lo = *(const i32x4*)(qrow + 64 * m);
        const i32x4 hi = *(const i32x4*)(qrow + 64 * m + 16);
        qop[m] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
    }
  }

  // ---- per-lane byte offsets, computed once: the loop adds only constants (buffer base,
  // row offsets), which the LDS instructions take as immediates.
  // K operand of S^T = K.Q^T: key row 32t + col, 16-byte chunk (4m + 2 half + e) ^ swz(row).
  // Row 32t + col swizzles like row col with bit 2 flipped, i.e. m ^ 1 when SWZ has bit 2.
  constexpr int KT = (SWZ & 4) ? 1 : 0;
  int koff[DM][2];
#pragma unroll
  for (int m = 0; m < DM; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) koff[m][e] = col * D + (((4 * m + 2 * half + e) ^ swz(col)) << 4);
  auto kaddr = [&](int t, int m, int e) { return koff[m ^ (KT * t)][e] + 32 * t * D; };
  // QX: the bf16 keys of a block sit in MX slices of 2 KiB, slice m holding chunks 2m and
  // 2m + 1 (d = 16m .. 16m + 15) of the 64 rows, 32 bytes a row; within a row the two
  // chunks trade places on rows with bit 3 set. Sixteen lanes reading one chunk of 16
  // consecutive rows then cover the 64 banks once, and the operand of instruction m for
  // key row 32t + col is at a per-lane base plus the constant 2048 m + 1024 t.
  const int kxoff = col * 32 + ((half ^ ((col >> 3) & 1)) << 4);
  // V^T operand through the transpose read: within a 16-lane group g, lane sl supplies key
  // row 16 tw + 8 (g >> 1) + (sl >> 1) and 8 columns of output tile u. Adding 16 tw to the
  // row flips swizzle bits 2 tw, i.e. tile u reads like tile u ^ tw.
  int voff[DU];
  {
    const int g = lane >> 4, sl = lane & 15;
    const int j = 8 * (g >> 1) + (sl >> 1);
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int cc = 32 * u + 16 * (g & 1) + 8 * (sl & 1);
      voff[u] = j * D + (((cc >> 4) ^ swz(j)) << 4) + (cc & 15);
    }
  }
  auto vaddr = [&](int u, int tw) { return voff[u ^ (tw & (SWZ >> 1))] + 16 * tw * D; };
  // LDS (row j, 16-byte slot cs) holds global chunk cs ^ swz(j) of key row j for K, and of
  // key row j with bits 2 and 3 exchanged for V. Instruction ii of a tile covers LDS rows
  // (1024 / D) ii .. and lane L lands on LDS bytes 16 L of that KiB, so it fetches the
  // matching chunk.
  // The V row order makes the transposed V reads (LDS row 16w + 8h + e for MFMA k-index
  // 32h + 8w + e) meet P exactly where the E4M3 cast leaves it: lane half h holds, in
  // byte 16t + 4a + b of its P operand, key 32t + 8a + 4h + b, which is the V row stored
  // at LDS row 16(2t + a/2) + 8h + 4(a%2) + b. So P needs no exchange between lane halves.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  auto swap23 = [](int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); };
  int goff[RPWK], goffv[RPW];
#pragma unroll
  for (int r = 0; r < RPWK; ++r) {
    const int ii = wave + kWaves * r;
    if constexpr (QX) {
      goff[r] = 1024 * ii + 16 * (lane ^ ((lane >> 4) & 1));
    } else {
      const int j = (1024 / KROW) * ii + lane / CHK, cs = lane % CHK;
      goff[r] = j * KROW + ((cs ^ swz(j)) << 4);
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int ii = wave + kWaves * r;
    const int j = (1024 / D) * ii + lane / CH, cs = lane % CH;
    goffv[r] = swap23(j) * D + ((cs ^ swz(j)) << 4);
  }
  // one tile of rows of `row_bytes` bytes (INST instructions of 1 KiB, RPWT per wave)
  auto dma_rows = [&](const uint8_t* src, int row_bytes, int inst, auto rpwt, int blk, uint8_t* dst,
                      const int* off) __attribute__((always_inline)) {
    constexpr int R = decltype(rpwt)::value;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (inst % kWaves == 0 || wave_s + kWaves * r < inst)
        lds_dma16(src, p.N * row_bytes, dst + (wave_s + kWaves * r) * 1024, off[r], blk * kKvBlock * row_bytes);
  };
  auto dma_k = [&](int blk, uint8_t* dst) __attribute__((always_inline)) {
    dma_rows(Kg, KROW, INST_PER_TILE_K, std::integral_constant<int, RPWK>{}, blk, dst, goff);
  };
  auto dma_v = [&](int blk, uint8_t* dst) __attribute__((always_inline)) {
    dma_rows(Vg, D, INST_PER_TILE, std::integral_constant<int, RPW>{}, blk, dst, goffv);
  };
  // every wave waits for its own DMA, then the barrier publishes all of them
  auto dma_wait_sync = []() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
  };
  auto block_of = [&](int n) { return p.reverse ? (wg_nb - 1 - n) : n; };
  auto active = [&](int n) { return wave_valid && (NG == 1 || n < wg_nb) && block_of(n) < wave_nb; };

  // Running max (log2 units). It starts finite and far below any logit, so that a fully
  // masked block (max -inf) leaves it and the row unchanged; the first real block still
  // gets alpha = exp2(-1e30 - m) = 0.
  float m_run = -1e30f;
  float l_run = 0.f;         // this lane half's share of the row sum of P~ S
  f32x16 acc[DU];
#pragma unroll
  for (int u = 0; u < DU; ++u) acc[u] = f32x16{0};
  unsigned cnt_zero = 0, cnt_zero_sink = 0;
  const float bias_s = POW2 ? p.log2_S : 0.f;
  const int i_row = r0 + col;

  // ---- S^T = K . Q^T for the two 32-key tiles of the block in Ks. For d <= 128 all
  // operand reads are issued first (the registers are free at this point), so that one
  // LDS latency covers them all; d = 256 has no room for that and pairs each MFMA with
  // its two reads.
  auto qk = [&](const uint8_t* Ks, f32x16 (&s)[2]) __attribute__((always_inline)) {
    if constexpr (QX) {
      // 2 tiles x MX bf16 MFMAs; each operand read right before its MFMA
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = f32x16{0};
#pragma unroll
        for (int m = 0; m < MX; ++m)
          s[t] = mfma_bf16(*(const i32x4*)(Ks + kxoff + 2048 * m + 1024 * t), qopx[m], s[t]);
      }
      return;
    }
    auto kop = [&](int t, int m) __attribute__((always_inline)) {
      const i32x4 lo = *(const i32x4*)(Ks + kaddr(t, m, 0));
      const i32x4 hi = *(const i32x4*)(Ks + kaddr(t, m, 1));
      return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    if (DM <= 2) {
      i32x8 ko[2][DM];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int m = 0; m < DM; ++m) ko[t][m] = kop(t, m);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = f32x16{0};
#pragma unroll
        for (int m = 0; m < DM; ++m) s[t] = mfma_e4m3(ko[t][m], qop[m], s[t]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * DM, 0);   // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * DM, 0);   // MFMA
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = f32x16{0};
#pragma unroll
        for (int m = 0; m < DM; ++m) s[t] = mfma_e4m3(kop(t, m), qop[m], s[t]);
      }
    }
  };

  // ---- V^T operand u of O^T += V^T . P^T, read transposed from the row-major V tile
  auto read_v = [&](const uint8_t* Vs, int u) __attribute__((always_inline)) {
    i32x8 vop;
#pragma unroll
    for (int tw = 0; tw < 4; ++tw) {
      const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(Vs + vaddr(u, tw)));
      vop[2 * tw] = r.x;
      vop[2 * tw + 1] = r.y;
    }
    return vop;
  };
  // the first NVPRE V operands are read before the softmax, so that their LDS latency is
  // spent under it
  constexpr int NVPRE = (D == 256 || QX) ? 0 : 1;   // d = 256 and the bf16 Q.K^T have no registers to spare
  constexpr int NVARR = NVPRE > 0 ? NVPRE : 1;

  // ---- online softmax of block blk with scores s: running max and sum, the rescale of O,
  // the E4M3 cast of P (into pop, the B-operand layout of the P.V product) and the counts
  // part: 0 = the whole block; with the sink split of block 0, 1 = its non-sink keys
  // [n_sink, 64) and 2 = its sink keys [0, n_sink)
  auto block_max = [&](f32x16 (&s)[2], int blk, int part) __attribute__((always_inline)) {
    // Masking: causal (key j > query i) on the wave's diagonal block (blocks past it are
    // never visited; the test covers them too), and the key window of a split part.
    if ((p.causal && blk >= diag) || (EXT && part != 0)) {
      // keep key offsets lo..hi within the block; element (t, r) holds offset
      // 32t + 8(r / 4) + r % 4 + 4 half
      int hi = p.causal ? min(i_row - blk * kKvBlock, kKvBlock - 1) : kKvBlock - 1;
      if (EXT && part == 2) hi = min(hi, p.n_sink - 1);
      const int lo = EXT && part == 1 ? p.n_sink : 0;
      const int hi_rel = hi - 4 * half, lo_rel = lo - 4 * half;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k = 32 * t + 8 * (r >> 2) + (r & 3);
          if (k > hi_rel || k < lo_rel) s[t][r] = -INFINITY;
        }
    }

    // running max: raw maximum, scaled once (c > 0 keeps the order). The IEEE maximum
    // (v_maximum3_f32) needs no quieting of its inputs, unlike fmaxf, and passes NaN on.
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, s[t][r]);
    {
      // the two lane halves trade maxima with v_permlane32_swap (no LDS round trip):
      // swapping a register with itself leaves the lower half's values in every lane of
      // sw[0] and the upper half's in every lane of sw[1]
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    return mx;
  };
  // the rest of the step from the new running max m_new (log2 units, >= m_run)
  auto softmax_from = [&](f32x16 (&s)[2], int blk, i32x8& pop, int part, float m_new) __attribute__((always_inline)) {
    const float alpha = fast_exp2(m_run - m_new);     // 0 on the first block
    m_run = m_new;
    const float bias = bias_s - m_new;

    // P~ S (exp2 with log2 S folded in for S = 2^k), row sum, E4M3 cast. The first cast
    // of a dword writes its low half and keeps the rest, which the second cast replaces,
    // so the kept value is arbitrary: it is the previous block's P operand, dead by now,
    // whose registers the new codes then take over without copies
    int pw[8];   // E4M3 codes of P, four per dword
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float x0 = fast_exp2(fmaf(s[t][4 * a + 0], c, bias));
        float x1 = fast_exp2(fmaf(s[t][4 * a + 1], c, bias));
        float x2 = fast_exp2(fmaf(s[t][4 * a + 2], c, bias));
        float x3 = fast_exp2(fmaf(s[t][4 * a + 3], c, bias));
        if (!POW2) { x0 *= p.S; x1 *= p.S; x2 *= p.S; x3 *= p.S; }
        const float part = (x0 + x1) + (x2 + x3);
        lsum = (t == 0 && a == 0) ? part : lsum + part;
        // (the option-carrying variant keeps no P across blocks: it has no registers to
        // spare for it)
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, EXT ? __builtin_nondeterministic_value(0) : pop[4 * t + a], false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
        pw[4 * t + a] = w;
      }
    if (EXT && p.qden) {
      // row sum of the decoded cast operand: codes back to fp32 (exact), two per cvt
      lsum = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(pw[q], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(pw[q], true);
        lsum += (lo[0] + lo[1]) + (hi[0] + hi[1]);
      }
    }
    l_run = alpha * l_run + lsum;

    if (CNT && !(EXT && part == 2)) {   // the sink keys themselves are never counted
      const int jb = blk * kKvBlock;
      const bool sink_block = jb < p.n_sink;
      unsigned z;   // zero codes among this lane's counted keys of the block
      // (rare: the diagonal and sink blocks; marked so, the byte masks are not computed
      // ahead of the branch on every block)
      if (__builtin_expect((p.causal && blk >= diag) || sink_block, 0)) {
        // blocks with masked or sink keys: only keys j in [n_sink, hi] count, hi = i for
        // causal attention. Zero codes are found four at a time: codes are 0x00..0x7E,
        // so byte + 0x7F never carries and leaves bit 7 clear exactly for a zero code.
        const int hi = p.causal ? i_row : p.N - 1;
        int n_hi = hi - jb - 4 * half + 1, n_lo = p.n_sink - jb - 4 * half;
        // In the option-carrying variant this branch sits in the loop over the parts of a
        // block; its masks do not depend on the part, and without this opaque (empty)
        // redefinition the compiler computes them ahead of the branch on every block.
        if constexpr (EXT) asm volatile("" : "+v"(n_hi), "+v"(n_lo));
        z = 0;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int k = 32 * t + 8 * a;   // word (t, a) holds keys jb + 4 half + k .. + 3
            const unsigned zero = ~((unsigned)pw[4 * t + a] + 0x7F7F7F7Fu) & 0x80808080u;
            const unsigned live = bytes_below(n_hi - k) & ~bytes_below(n_lo - k);
            z += __builtin_popcount(zero & live);
          }
        // by value: a conditional update of one of the two counters lets the compiler
        // merge the updates into a store through a selected address, in scratch
        cnt_zero_sink += z & (0u - (unsigned)sink_block);
      } else {
        // every key counts: for a code byte b in [0, 126], |b - 1| + |b - 127| is 126,
        // plus 2 when b = 0, so two accumulating v_sad_u8 per dword sum to
        // 8 * 4 * 126 + 2 * (zero codes) over the block's 32 codes of this lane
        unsigned sad = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          sad = __builtin_amdgcn_sad_u8((unsigned)pw[q], 0x01010101u, sad);
          sad = __builtin_amdgcn_sad_u8((unsigned)pw[q], 0x7F7F7F7Fu, sad);
        }
        z = (sad - 8u * 4u * 126u) >> 1;
      }
      cnt_zero += z;
    }
    if (OUT) {
      // Rescale only when some row's max moved: alpha == 1 exactly otherwise, and a
      // multiply by 1 changes nothing, so skipping it is exact.
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int u = 0; u < DU; ++u) acc[u] *= alpha;
      }

      // the cast codes are the P.V operand as they stand (the V tile's row order matches)
#pragma unroll
      for (int q = 0; q < 8; ++q) pop[q] = pw[q];
    }
  };
  auto softmax = [&](f32x16 (&s)[2], int blk, i32x8& pop, int part) __attribute__((always_inline)) {
    const float mx = block_max(s, blk, part);
    softmax_from(s, blk, pop, part, __builtin_elementwise_maximum(m_run, mx * c));
  };

  // ---- O^T += V^T . P^T with the V tile in Vs (operands u < NVPRE already read)
  auto pv = [&](const uint8_t* Vs, const i32x8& pop, const i32x8 (&vpre)[NVARR]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const i32x8 vop = u < NVPRE ? vpre[u < NVPRE ? u : 0] : read_v(Vs, u);
      acc[u] = mfma_e4m3(vop, pop, acc[u]);
    }
    // issue order: each remaining MFMA right after its four operand reads
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      if (u >= NVPRE) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
    }
  };

  i32x8 pop = {0, 0, 0, 0, 0, 0, 0, 0};   // P of the block, in the B-operand layout of the P.V product
  if constexpr (NG > 1) {
    // Step n: group g visits position NG n + g. After its Q.K^T each wave puts its rows'
    // scaled block maxima r into xr; group g then takes as running maximum
    // max(M, r_0, .., r_g), M the running maximum through the previous step, which is the
    // maximum of the sequential walk at its position. The exchange costs one barrier.
    __shared__ float xr[NG][kBlockM];
    float M = -1e30f;   // running maximum through the last completed step (every group)
    if (grp < wg_nb) {
      dma_k(block_of(grp), kbuf(0));
      if (OUT) dma_v(block_of(grp), vbuf(0));
    }
    dma_wait_sync();
    const int nsteps = (wg_nb + NG - 1) / NG;
    auto step = [&](int n, int cur) __attribute__((always_inline)) {
      const int pos = NG * n + grp;
      if (pos + NG < wg_nb) {
        const int next = __builtin_amdgcn_readfirstlane(block_of(pos + NG));
        dma_k(next, kbuf(cur ^ 1));
        if (OUT) dma_v(next, vbuf(cur ^ 1));
      }
      const bool act = active(pos);
      const int blk = block_of(pos);
      f32x16 s[2];
      i32x8 vpre[NVARR];
      float r = -INFINITY;
      if (act) {
        qk(kbuf(cur), s);
        if (OUT) {
#pragma unroll
          for (int u = 0; u < NVPRE; ++u) vpre[u] = read_v(vbuf(cur), u);
        }
        r = block_max(s, blk, 0) * c;
      }
      if (half == 0) xr[grp][wave * kRowsPerWave + col] = r;
      __syncthreads();
      float m_pos = M;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        M = __builtin_elementwise_maximum(M, xr[g][wave * kRowsPerWave + col]);
        if (g == grp) m_pos = M;
      }
      if (act) {
        softmax_from(s, blk, pop, 0, m_pos);
        if (OUT) pv(vbuf(cur), pop, vpre);
      }
      dma_wait_sync();
    };
    for (int n = 0; n < nsteps; n += 2) {
      step(n, 0);
      if (n + 1 < nsteps) step(n + 1, 1);
    }
  } else {
    dma_k(block_of(0), kb0);
    if (OUT) dma_v(block_of(0), vb0);
    dma_wait_sync();
    // step n on buffers `cur` (a constant 0 or 1 at each call site); block n + 1 lands in
    // the other pair
    auto step = [&](int n, int cur) __attribute__((always_inline)) {
      if (n + 1 < wg_nb) {
        // wave-uniform by construction; said explicitly, since the buffer offset must sit
        // in a scalar register (the option-carrying variant otherwise wraps each load in a
        // loop over lanes)
        const int next = __builtin_amdgcn_readfirstlane(block_of(n + 1));
        dma_k(next, kbuf(cur ^ 1));
        if (OUT) dma_v(next, vbuf(cur ^ 1));
      }
      if (active(n)) {
        const int blk = block_of(n);
        // one visit, or two for block 0 under the sink split (its non-sink keys first)
        const bool split = EXT && p.sink_last && blk == 0;
        const int last_part = split ? 2 : 0;
        for (int part = split ? 1 : 0; part <= last_part; ++part) {
          f32x16 s[2];
          qk(kbuf(cur), s);
          i32x8 vpre[NVARR];
          if (OUT) {
#pragma unroll
            for (int u = 0; u < NVPRE; ++u) vpre[u] = read_v(vbuf(cur), u);
          }
          softmax(s, blk, pop, part);
          if (OUT) pv(vbuf(cur), pop, vpre);
        }
      }
      dma_wait_sync();
    };
    for (int n = 0; n < wg_nb; n += 2) {
      step(n, 0);
      if (n + 1 < wg_nb) step(n + 1, 1);
    }
  }

  if (CNT) {
    // Waves past the end of the sequence (they ran on rows that do not exist) count nothing.
    if (!wave_valid) cnt_zero = cnt_zero_sink = 0;
    // Workgroup total of the zero counts, then
    // at most one atomic per counter and workgroup. The pair counters were set in closed
    // form before the launch.
    __shared__ unsigned red[2][kWaves * NG];
    unsigned v0 = cnt_zero, v1 = cnt_zero_sink;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      v0 += __shfl_xor(v0, off);
      v1 += __shfl_xor(v1, off);
    }
    if (lane == 0) {
      red[0][wave_g] = v0;
      red[1][wave_g] = v1;
    }
    __syncthreads();
    if (tid == 0) {
      unsigned long long z = 0, zs = 0;
#pragma unroll
      for (int w = 0; w < kWaves * NG; ++w) {
        z += red[0][w];
        zs += red[1][w];
      }
      if (z) atomicAdd(p.counts + 0, z);
      if (zs) atomicAdd(p.counts + 1, zs);
    }
  }
  if constexpr (NG > 1 && OUT) {
    // Merge the walk groups' states: group 1 hands (acc, l, m) to group 0 through LDS (the
    // K/V buffers are free after the loop's last barrier); output tile u of a lane goes to
    // buffer array u, 16 bytes per lane, lane-contiguous.
    static_assert(NG == 2 && DU == 4, "one hand-over, four output tiles");
    static_assert(kWaves * 64 * 16 * 4 <= NG * TILE && kWaves * 64 * 16 * 4 <= NG * TILE_K, "a tile per array");
    __shared__ float xlm[kWaves][2][64];
    float* const xa[4] = {(float*)kb0, (float*)kb1, (float*)vb0, (float*)vb1};
    if (grp == 1) {
#pragma unroll
      for (int u = 0; u < DU; ++u)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *(f32x4*)(xa[u] + ((wave * 4 + a) * 64 + lane) * 4) =
              f32x4{acc[u][4 * a], acc[u][4 * a + 1], acc[u][4 * a + 2], acc[u][4 * a + 3]};
      xlm[wave][0][lane] = m_run;
      xlm[wave][1][lane] = l_run;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xlm[wave][0][lane], l1 = xlm[wave][1][lane];
    const float m = __builtin_elementwise_maximum(m_run, m1);
    const float e0 = fast_exp2(m_run - m), e1 = fast_exp2(m1 - m);
    l_run = fmaf(l1, e1, l_run * e0);
#pragma unroll
    for (int u = 0; u < DU; ++u)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 o1 = *(const f32x4*)(xa[u] + ((wave * 4 + a) * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[u][4 * a + e] = fmaf(o1[e], e1, acc[u][4 * a + e] * e0);
      }
  }
  if (!wave_valid) return;
  if (OUT) {
    // O = acc vd / (sum of P~ S) = acc vd / (S l); both halves hold partial row sums.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float scale = p.v_descale[b * p.Hkv + hk] / l_tot;
    float* orow = p.o + q_head + (size_t)i_row * D + 4 * half;
#pragma unroll
    for (int u = 0; u < DU; ++u)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 val = {acc[u][4 * a + 0] * scale, acc[u][4 * a + 1] * scale,
                           acc[u][4 * a + 2] * scale, acc[u][4 * a + 3] * scale};
        *(f32x4*)(orow + 32 * u + 8 * a) = val;
      }
  }
}

template <int D, bool POW2, bool OUT, bool CNT, bool EXT, bool QX>
__global__ FP8ATTN_BOUNDS(64 * waves_for(D), QX ? (D <= 128 ? 3 : 2) : min_waves_per_simd(D)) void fwd_kernel(const Params p) {
  fwd_body<D, POW2, OUT, CNT, EXT, QX, 1>(p);
}

// d = 128, the plain options: 64-row tiles walked by two groups of two waves
template <bool POW2, bool OUT, bool CNT>
__global__ FP8ATTN_BOUNDS(2 * 64 * kPairWaves, 2) void fwd_pair_kernel(const Params p) {
  fwd_body<128, POW2, OUT, CNT, false, false, 2>(p);
}

// K (E4M3) -> the same values as bf16, in the slice layout the exact Q.K^T kernel reads.
// Thread t converts 16 codes: row R = 16 t / d of all heads' keys, d = e0 .. e0 + 15 with
// e0 = 16 t % d, into 32 bytes at slice e0 / 16, row R % 64 of key block R / 64 (blocks
// of 64 rows, 128 d bytes each; N is a multiple of 64, so no block spans two heads).
__global__ void keys_to_bf16_kernel(const uint8_t* __restrict__ k, uint8_t* __restrict__ kx, int64_t n16, int d) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n16) return;
  const int64_t R = 16 * t / d;
  const int e0 = (int)(16 * t - R * d);
  const int64_t out = (R / kKvBlock) * (int64_t)(kKvBlock * 2 * d) + 2048 * (e0 / 16) + 32 * (R % kKvBlock);
  const i32x4 w = ((const i32x4*)k)[t];
  const i32x2 a = e4m3x4_to_bf16x4(w.x), b = e4m3x4_to_bf16x4(w.y);
  const i32x2 c = e4m3x4_to_bf16x4(w.z), e = e4m3x4_to_bf16x4(w.w);
  *(i32x8*)(kx + out) = i32x8{a.x, a.y, b.x, b.y, c.x, c.y, e.x, e.y};
}

// Zero counts start at 0; the pair counts are known in closed form before the launch.
__global__ void init_counts_kernel(unsigned long long* counts, unsigned long long pairs,
                                   unsigned long long pairs_sink) {
  if (threadIdx.x == 0) {
    counts[0] = 0ull;
    counts[1] = 0ull;
    counts[2] = pairs;
    counts[3] = pairs_sink;
  }
}

template <int D, bool OUT, bool CNT, bool EXT, bool QX>
void launch_one(const Params& p, bool pow2, hipStream_t stream) {
  const dim3 grid((unsigned)num_workgroups(p, D)), block(64 * waves_for(D));
  if (pow2) hipLaunchKernelGGL((fwd_kernel<D, true, OUT, CNT, EXT, QX>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((fwd_kernel<D, false, OUT, CNT, EXT, QX>), grid, block, 0, stream, p);
}

template <bool OUT, bool CNT>
void launch_pairs(const Params& p, bool pow2, hipStream_t stream) {
  const int64_t tiles = (p.N + kRowsPerWave * kPairWaves - 1) / (kRowsPerWave * kPairWaves);
  const dim3 grid((unsigned)((int64_t)p.B * p.H * tiles)), block(2 * 64 * kPairWaves);
  if (pow2) hipLaunchKernelGGL((fwd_pair_kernel<true, OUT, CNT>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((fwd_pair_kernel<false, OUT, CNT>), grid, block, 0, stream, p);
}

template <int D, bool OUT, bool CNT>
void launch_d(const Params& p, bool pow2, hipStream_t stream) {
  const bool ext = p.sink_last || p.qden;
  if constexpr (D <= 128) {
    if (p.exact_qk) {
      if (ext) launch_one<D, OUT, CNT, true, true>(p, pow2, stream);
      else launch_one<D, OUT, CNT, false, true>(p, pow2, stream);
      return;
    }
  }
  if constexpr (D == 128) {
    if (fwd_walk_groups(p, D) == 2) {
      launch_pairs<OUT, CNT>(p, pow2, stream);
      return;
    }
  }
  if (ext) launch_one<D, OUT, CNT, true, false>(p, pow2, stream);
  else launch_one<D, OUT, CNT, false, false>(p, pow2, stream);
}

template <bool OUT, bool CNT>
hipError_t launch(const Params& p, int d, bool pow2, hipStream_t stream) {
  if (CNT) {
    hipLaunchKernelGGL(init_counts_kernel, dim3(1), dim3(64), 0, stream, p.counts, p.pairs, p.pairs_sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.exact_qk && d > 128) return hipErrorInvalidValue;
  if (fwd_tile_rows(p, d) == 16) return launch_fwd16(p, pow2, OUT, CNT, stream);
  switch (d) {
    case 64: launch_d<64, OUT, CNT>(p, pow2, stream); break;
    case 128: launch_d<128, OUT, CNT>(p, pow2, stream); break;
    case 256: launch_d<256, OUT, CNT>(p, pow2, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Compute units of the current device, looked up once per device (0 if unknown).
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

// Build-time override of the kernel choice, for measurements: 1 = 32-row waves alone,
// 2 = 32-row waves in walk groups of two, 3 = 16-row waves, 0 = the measured rule below.
#ifndef FP8ATTN_FORCE_VARIANT
#define FP8ATTN_FORCE_VARIANT 0
#endif

int fwd_walk_groups(const Params& p, int d) {
  if (d != 128 || p.sink_last || p.qden || p.exact_qk) return 1;
  if (FP8ATTN_FORCE_VARIANT != 0) return FP8ATTN_FORCE_VARIANT == 2 ? 2 : 1;
  // measured on MI355X (256 compute units), T = 128-row tiles: the two walk groups win
  // where the grid leaves SIMDs with one wave, with causal masking up to T = 1.5 per
  // compute unit (10-30% faster than the 32-row and 5-12% faster than the 16-row kernel),
  // without it up to T = 0.5 per compute unit (17-27% and 8-10%); at one tile per compute
  // unit without masking they tie with the 32-row kernel, and beyond they lose 5-20%
  const int cus = device_cu_count();
  const int64_t tiles = num_workgroups(p, d);
  return cus > 0 && (p.causal ? 2 * tiles <= 3ll * cus : 2 * tiles <= cus) ? 2 : 1;
}

int fwd_tile_rows(const Params& p, int d) {
  if (d != 128 || p.sink_last || p.qden || p.exact_qk) return 32;
  if (FP8ATTN_FORCE_VARIANT != 0) return FP8ATTN_FORCE_VARIANT == 3 ? 16 : 32;
  if (fwd_walk_groups(p, d) == 2) return 32;
  // measured on MI355X (256 compute units): with causal masking, between 1.5 and 2 tiles of
  // 128 rows per compute unit, 64-row workgroups of 16-row waves balance the unequal tiles
  // better (8% faster than the 32-row kernel, 9-11% faster than the walk groups)
  const int cus = device_cu_count();
  const int64_t tiles = num_workgroups(p, d);
  return cus > 0 && p.causal && tiles <= 2ll * cus ? 16 : 32;
}

hipError_t launch_fwd(const Params& p, int d, bool pow2_scale, hipStream_t stream) {
  return launch<true, false>(p, d, pow2_scale, stream);
}

hipError_t launch_keys_to_bf16(const uint8_t* k, uint8_t* kx, int64_t n_elements, int d, hipStream_t stream) {
  const int64_t n16 = n_elements / 16;
  if (n16 <= 0) return hipSuccess;
  const int64_t blocks = (n16 + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(keys_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k, kx, n16, d);
  return hipGetLastError();
}

hipError_t launch_count(const Params& p, int d, bool pow2_scale, hipStream_t stream) {
  return launch<false, true>(p, d, pow2_scale, stream);
}

hipError_t launch_fwd_count(const Params& p, int d, bool pow2_scale, hipStream_t stream) {
  return launch<true, true>(p, d, pow2_scale, stream);
}

}  // namespace fp8attn
