// Split-KV decode of the FP8 (OCP E4M3) P-cast attention: one query row per (batch,
// head) attending to all N keys, the key range cut into n_split contiguous block ranges.
//
// Computation: the online softmax with the P-cast of "P-Cast Precision in FP8 Attention"
// (gist.science technical summary, section 1: running max per KV block, P~ times the
// static scale S cast to E4M3 before P.V, the KV blocks walked forward or reverse) run
// separately over each split's keys; the split states (m, l, acc) are merged exactly
// through their maxima, as split-KV FlashAttention does. The P cast therefore depends on
// the partition; the split count is an argument.
//
// Layout of the work
// ------------------
// * One wave = one workgroup = one (batch, KV head, group of up to 32 query heads, split).
//   The query heads of a KV head (grouped-query attention) share its K/V stream: they are
//   the 32 "rows" of the MFMA tiles (unused rows hold zero queries and are not written).
// * Per 64-key block: S^T = K.Q^T (v_mfma_f32_32x32x64_f8f6f4, A = 32 keys of K from LDS,
//   B = the query rows), lane-local running max with one lane-half exchange, exp2, the
//   E4M3 cast, and O^T += V^T.P^T with V^T read by ds_read_b64_tr_b8, exactly as in the
//   prefill kernel (fwd.hip). Every lane's row is its own query head, so the logit scale
//   qd kd log2(e)/sqrt(d) is per lane.
// * V blocks go HBM -> LDS by buffer_load ... lds into two buffers; K blocks (d <= 128) go
//   straight to registers, one block ahead, with ordinary loads (at d = 256 K is staged
//   through LDS like V). The wave waits only for its own loads, so no barrier is needed.
// * The partial state of each (row, split) goes to the caller's workspace as a record of
//   d + 4 floats, [acc[0..d), m (log2 units), l, 2 unused] (16-byte aligned records);
//   decode_merge_kernel combines the splits.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "kernel_common.h"
#include "launch.h"

namespace fp8attn {
namespace {

template <int D, bool POW2>
__global__ FP8ATTN_BOUNDS(64, 2) void decode_kernel(const DecodeParams p) {
  constexpr int DM = D / 64;             // QK^T MFMAs per 32-key tile
  constexpr int DU = D / 32;             // 32-column output tiles
  constexpr int CH = D / 16;             // 16-byte chunks per row
  constexpr int SWZ = (CH >= 8 ? 8 : CH) - 1;
  constexpr int TILE = kKvBlock * D;     // bytes of one K or V block
  constexpr int RPW = TILE / 1024;       // DMA instructions per tile (one wave)
  // d <= 128: K goes HBM -> registers, one block ahead (its MFMA operand is 32 contiguous
  // bytes of a key row per lane), so that only V occupies LDS and more waves fit on a
  // compute unit; d = 256 stages K through LDS as well (its operands would not fit)
  constexpr bool KREG = D <= 128;
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[KREG ? 16 : TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[KREG ? 16 : TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[TILE];
  auto swz = [](int j) { return swz_row<SWZ>(j); };

  const int lane = threadIdx.x;
  const int col = lane & 31;
  const int half = lane >> 5;

  // workgroup -> (split, query group, kv head, batch), split fastest; kept in scalar
  // registers (the buffer resources built from them must be wave-uniform)
  int L = blockIdx.x;
  const int split = __builtin_amdgcn_readfirstlane(L % p.n_split);
  L /= p.n_split;
  const int qg = __builtin_amdgcn_readfirstlane(L % p.n_qgroups);
  L /= p.n_qgroups;
  const int hk = __builtin_amdgcn_readfirstlane(L % p.Hkv);
  const int b = __builtin_amdgcn_readfirstlane(L / p.Hkv);

  const int G = p.H / p.Hkv;
  const int r = qg * 32 + col;                 // this lane's query head within the group
  const bool row_valid = r < G;
  const int h = hk * G + (row_valid ? r : 0);

  const int nkb = p.N / kKvBlock;
  const int blk0 = (int)((int64_t)split * nkb / p.n_split);
  const int blk1 = (int)((int64_t)(split + 1) * nkb / p.n_split);
  const int nb = blk1 - blk0;

  const size_t kv_head = ((size_t)b * p.Hkv + hk) * (size_t)p.N * D;
  const uint8_t* __restrict__ Kg = p.k + kv_head;
  const uint8_t* __restrict__ Vg = p.v + kv_head;

  // per-row logit scale in log2 units
  const float c = p.q_descale[b * p.H + h] * p.k_descale[b * p.Hkv + hk] * p.log2e_rsqrt_d;

  // Q operand: lane (col, half) holds q[row col][64m + 32 half .. +32]; rows past the group
  // are zero (their scores are 0, their state is never written)
  i32x8 qop[DM];
  {
    const uint8_t* qrow = p.q + ((size_t)b * p.H + h) * D + 32 * half;
#pragma unroll
    for (int m = 0; m < DM; ++m) {
      if (row_valid) {
        const i32x4 lo = *(const i32x4*)(qrow + 64 * m);
        const i32x4 hi = *(const i32x4*)(qrow + 64 * m + 16);
        qop[m] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      } else {
        qop[m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }

  // LDS operand offsets (the same swizzled image as the prefill kernel)
  constexpr int KT = (SWZ & 4) ? 1 : 0;
  int koff[DM][2];
#pragma unroll
  for (int m = 0; m < DM; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) koff[m][e] = col * D + (((4 * m + 2 * half + e) ^ swz(col)) << 4);
  auto kaddr = [&](int t, int m, int e) { return koff[m ^ (KT * t)][e] + 32 * t * D; };
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
  int goff[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const int j = (1024 / D) * q + lane / CH, cs = lane % CH;
    goff[q] = j * D + ((cs ^ swz(j)) << 4);
  }
  // the DMA destinations stay in the LDS address space (no generic-pointer round trip)
  auto dma_block = [&](int blk, lds_u8* kdst, lds_u8* vdst) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      if (!KREG) lds_dma16(Kg, p.N * D, kdst + q * 1024, goff[q], blk * TILE);
      lds_dma16(Vg, p.N * D, vdst + q * 1024, goff[q], blk * TILE);
    }
  };
  // K operands of a block straight from HBM (KREG): operand (t, m) of lane (col, half) is
  // key 32t + col, bytes 64m + 32 half .. + 32
  typedef i32x8 kops_t[2][DM];
  const uint8_t* const krow = Kg + (size_t)col * D + 32 * half;
  auto load_k = [&](int blk, kops_t& ko) __attribute__((always_inline)) {
    const uint8_t* base = krow + (size_t)blk * TILE;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int m = 0; m < DM; ++m) {
        const i32x4 lo = *(const i32x4*)(base + 32 * t * D + 64 * m);
        const i32x4 hi = *(const i32x4*)(base + 32 * t * D + 64 * m + 16);
        ko[t][m] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
  };
  auto block_of = [&](int n) { return p.reverse ? (blk1 - 1 - n) : (blk0 + n); };

  float m_run = -1e30f;       // running max (log2 units), finite: see the prefill kernel
  float l_run = 0.f;          // this lane half's share of the row sum of P~ S
  f32x16 acc[DU];
#pragma unroll
  for (int u = 0; u < DU; ++u) acc[u] = f32x16{0};
  const float bias_s = POW2 ? p.log2_S : 0.f;

  auto step = [&](const uint8_t* Ks, const uint8_t* Vs, const kops_t& kr) __attribute__((always_inline)) {
    // S^T = K . Q^T
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x16{0};
#pragma unroll
      for (int m = 0; m < DM; ++m) {
        if constexpr (KREG) {
          s[t] = mfma_e4m3(kr[t][m], qop[m], s[t]);
        } else {
          const i32x4 lo = *(const i32x4*)(Ks + kaddr(t, m, 0));
          const i32x4 hi = *(const i32x4*)(Ks + kaddr(t, m, 1));
          s[t] = mfma_e4m3(i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}, qop[m], s[t]);
        }
      }
    }
    // running max of the row over the block (raw), then in log2 units
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 16; ++q) mx = fmaxf(mx, s[t][q]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(mx, __uint_as_float(half ? sw[0] : sw[1]));
    }
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    const float bias = bias_s - m_new;
    // P~ S, row sum, E4M3 cast
    int pw[8];
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
        lsum += (x0 + x1) + (x2 + x3);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __builtin_nondeterministic_value(0), false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
        pw[4 * t + a] = w;
      }
    l_run = alpha * l_run + lsum;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int u = 0; u < DU; ++u) acc[u] *= alpha;
    }
    // P pairs of 8 consecutive keys (B operand of O^T = V^T . P^T)
    i32x8 pop;
#pragma unroll
    for (int tw = 0; tw < 4; ++tw) {
      const auto rr = __builtin_amdgcn_permlane32_swap(pw[2 * tw], pw[2 * tw + 1], false, false);
      pop[2 * tw] = (int)rr[0];
      pop[2 * tw + 1] = (int)rr[1];
    }
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      i32x8 vop;
#pragma unroll
      for (int tw = 0; tw < 4; ++tw) {
        const i32x2 rr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(Vs + vaddr(u, tw)));
        vop[2 * tw] = rr.x;
        vop[2 * tw + 1] = rr.y;
      }
      acc[u] = mfma_e4m3(vop, pop, acc[u]);
    }
  };

  // Block n is in buffer n & 1. Before step n the wave waits for its DMA (issued during
  // step n - 1), then issues block n + 1 into the other buffer, whose previous contents
  // (block n - 1) were consumed in step n - 1.
  lds_u8* const k0 = (lds_u8*)kb0;
  lds_u8* const k1 = (lds_u8*)kb1;
  lds_u8* const v0 = (lds_u8*)vb0;
  lds_u8* const v1 = (lds_u8*)vb1;
  // (KREG: K of block n in kr0 for even n, kr1 for odd n, loaded with V's DMA)
  kops_t kr0, kr1;
  dma_block(block_of(0), k0, v0);
  if constexpr (KREG) load_k(block_of(0), kr0);
  for (int n = 0; n < nb; n += 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): block n has landed
    if (n + 1 < nb) {
      dma_block(block_of(n + 1), k1, v1);
      if constexpr (KREG) load_k(block_of(n + 1), kr1);
    }
    step(kb0, vb0, kr0);
    if (n + 1 < nb) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      if (n + 2 < nb) {
        dma_block(block_of(n + 2), k0, v0);
        if constexpr (KREG) load_k(block_of(n + 2), kr0);
      }
      step(kb1, vb1, kr1);
    }
  }

  if (!row_valid) return;
  // partial state of (row, split): acc over d, m (log2 units), l (both lane halves)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  float* ws = p.ws + (((size_t)b * p.H + h) * p.n_split + split) * decode_record_floats(D);
#pragma unroll
  for (int u = 0; u < DU; ++u)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 val = {acc[u][4 * a + 0], acc[u][4 * a + 1], acc[u][4 * a + 2], acc[u][4 * a + 3]};
      *(f32x4*)(ws + 32 * u + 8 * a + 4 * half) = val;
    }
  if (half == 0) {
    ws[D] = m_run;
    ws[D + 1] = l_tot;
  }
}

// O[b][h][c] = vd * sum_s acc_s[c] 2^(m_s - m) / sum_s l_s 2^(m_s - m), m = max_s m_s.
// One workgroup of kMergeThreads per (b, h, 64 output columns): all threads find m, then
// thread t sums column c0 + t % 64 over the splits s = t / 64, t / 64 + P, ... (P = 4),
// unrolled so that many loads are in flight, and the P partial sums meet in LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeCols = 64;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const DecodeParams p) {
  constexpr int REC = decode_record_floats(D);
  constexpr int P = kMergeThreads / kMergeCols;
  __shared__ float red[kMergeThreads];
  __shared__ float part_num[P][kMergeCols];
  __shared__ float part_den[P];
  const int bh = blockIdx.x / (D / kMergeCols);
  const int c0 = (blockIdx.x % (D / kMergeCols)) * kMergeCols;
  const int b = bh / p.H, h = bh - b * p.H;
  const int hk = h / (p.H / p.Hkv);
  const int tid = threadIdx.x;
  const float* ws = p.ws + (size_t)bh * p.n_split * REC;

  float m = -INFINITY;
  for (int s = tid; s < p.n_split; s += kMergeThreads) m = fmaxf(m, ws[(size_t)s * REC + D]);
  red[tid] = m;
  __syncthreads();
  for (int w = kMergeThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  m = red[0];

  const int cl = tid % kMergeCols, part = tid / kMergeCols;
  const int c = c0 + cl;
  float num = 0.f, den = 0.f;
  int s = part;
  for (; s + 3 * P < p.n_split; s += 4 * P) {
    float mm[4], aa[4], ll[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* st = ws + (size_t)(s + i * P) * REC;
      mm[i] = st[D];
      ll[i] = st[D + 1];
      aa[i] = st[c];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float w = fast_exp2(mm[i] - m);
      num = fmaf(aa[i], w, num);
      den = fmaf(ll[i], w, den);
    }
  }
  for (; s < p.n_split; s += P) {
    const float* st = ws + (size_t)s * REC;
    const float w = fast_exp2(st[D] - m);
    num = fmaf(st[c], w, num);
    den = fmaf(st[D + 1], w, den);
  }
  part_num[part][cl] = num;
  if (cl == 0) part_den[part] = den;
  __syncthreads();
  if (part == 0) {
    float nt = 0.f, dt = 0.f;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      nt += part_num[q][cl];
      dt += part_den[q];
    }
    p.o[(size_t)bh * D + c] = p.v_descale[b * p.Hkv + hk] * nt / dt;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int d, bool pow2, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.B * p.Hkv * p.n_qgroups * p.n_split)), block(64);
  const dim3 mgrid((unsigned)(p.B * p.H * (d / kMergeCols)));
#define FP8ATTN_DECODE(D)                                                                        \
  {                                                                                              \
    if (pow2) hipLaunchKernelGGL((decode_kernel<D, true>), grid, block, 0, stream, p);           \
    else hipLaunchKernelGGL((decode_kernel<D, false>), grid, block, 0, stream, p);               \
    const hipError_t e = hipGetLastError();                                                      \
    if (e != hipSuccess) return e;                                                               \
    hipLaunchKernelGGL((decode_merge_kernel<D>), mgrid, dim3(kMergeThreads), 0, stream, p);      \
  }
  switch (d) {
    case 64: FP8ATTN_DECODE(64) break;
    case 128: FP8ATTN_DECODE(128) break;
    case 256: FP8ATTN_DECODE(256) break;
    default: return hipErrorInvalidValue;
  }
#undef FP8ATTN_DECODE
  return hipGetLastError();
}

}  // namespace fp8attn
