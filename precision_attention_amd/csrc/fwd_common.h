// Pieces shared by the two forward kernels (fwd.hip: 32 query rows per wave; fwd16.hip:
// 16 rows per wave, for small grids): the
// grid-to-tile mapping, a byte-mask helper, and the host side of the choice between them.
// Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace fp8attn {
namespace {

// Map the linear workgroup id to (b, h, query tile). Workgroups are dispatched to the
// 8 XCDs round-robin (id % 8); when the kv heads divide evenly, every XCD gets whole kv
// heads (all their query heads), so K/V of one head stay in one XCD's L2, and within an
// XCD the tiles run longest-first for causal masking. The order within an XCD is
//  * rank-major (by default): tile rank r of every head of the XCD, then rank r + 1, so
//    that the query heads sharing a kv head read the same K/V blocks at about the same time;
//  * head-major (p.head_major: one query head per kv head and a head's K/V small enough
//    for the XCD's 4 MB L2): all tiles of one head, then the next head, so that one head's
//    K/V stays in L2 while its tiles run instead of many heads' K/V passing through it.
__device__ __forceinline__ void map_tile(const Params& p, int ntiles, int& b, int& h, int& hk, int& qt) {
  const int G = p.H / p.Hkv;
  const int U = p.B * p.Hkv;
  const int total = U * G * ntiles;
  const int L = blockIdx.x;
  int rank, unit, member;
  if ((total & 7) == 0 && (U & 7) == 0) {
    const int xcd = L & 7, slot = L >> 3;
    const int upx = U >> 3;
    if (p.head_major) {
      const int uix = slot / ntiles;
      rank = slot - uix * ntiles;
      unit = xcd * upx + uix;
      member = 0;
    } else {
      const int per_rank = upx * G;
      rank = slot / per_rank;
      const int rem = slot - rank * per_rank;
      unit = xcd * upx + rem / G;
      member = rem % G;
    }
  } else {
    const int BH = p.B * p.H;
    rank = L / BH;
    const int bh = L - rank * BH;
    unit = bh / G;
    member = bh % G;
  }
  b = unit / p.Hkv;
  hk = unit - b * p.Hkv;
  h = hk * G + member;
  qt = p.causal ? (ntiles - 1 - rank) : rank;
}

// Bit 7 of each of the first n bytes of a word (n clamped to 0 .. 4).
__device__ __forceinline__ unsigned bytes_below(int n) {
  return n >= 4 ? 0x80808080u : (n <= 0 ? 0u : (0x80808080u & ((1u << (8 * n)) - 1u)));
}

}  // namespace

// Query rows per wave of the forward launch for these parameters: 16 (fwd16.hip) for
// d = 128 without the fwd_ex options or the exact Q.K^T when the 128-row query tiles number
// at most two per compute unit of the current device (causal) or at most one per two
// compute units (not causal), else 32.
int fwd_tile_rows(const Params& p, int d);
// Walk groups of the 32-row forward launch: 2 when 64-row tiles are walked by two groups
// of two waves (d = 128 without the fwd_ex options or the exact Q.K^T), else 1.
int fwd_walk_groups(const Params& p, int d);
// The 16-row forward (d = 128); the caller has set the counts if `count`.
hipError_t launch_fwd16(const Params& p, bool pow2, bool out, bool count, hipStream_t stream);

}  // namespace fp8attn
