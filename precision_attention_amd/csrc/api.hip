// C ABI of the FP8 P-cast attention forward (declared in include/fp8attn.h).
// Every argument is checked here before any HIP call; kernels live in fwd.hip.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fp8attn.h"
#include "launch.h"
#include "fwd_common.h"

namespace {

constexpr float kE4M3Max = 448.0f;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Shared checks of the shapes, flags and scale. Returns FP8ATTN_OK or a negative status.
int check_common(int B, int H, int Hkv, int N, int d, int causal, int kv_order, float S) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return FP8ATTN_EINVAL;
  if (H % Hkv != 0) return FP8ATTN_EINVAL;
  if (causal != 0 && causal != 1) return FP8ATTN_EINVAL;
  if (kv_order != FP8ATTN_KV_FORWARD && kv_order != FP8ATTN_KV_REVERSE &&
      kv_order != FP8ATTN_KV_REVERSE_SINK_LAST)
    return FP8ATTN_EINVAL;
  if (!(S > 0.0f && S <= kE4M3Max)) return FP8ATTN_EINVAL;   // also rejects NaN
  if (d != 64 && d != 128 && d != 256) return FP8ATTN_EUNSUPPORTED;
  if (N % fp8attn::kKvBlock != 0) return FP8ATTN_EUNSUPPORTED;
  if ((int64_t)N * d > INT32_MAX) return FP8ATTN_EUNSUPPORTED;   // one head's K/V in a buffer range
  const int bm = fp8attn::block_m_for(d);
  const int64_t tiles = (N + bm - 1) / bm;
  if ((int64_t)B * H * tiles > INT32_MAX) return FP8ATTN_EUNSUPPORTED;
  return FP8ATTN_OK;
}

// Unmasked non-sink (query, key) pairs over all B H heads, and those among them that lie in
// KV blocks holding a sink token (keys n_sink .. E - 1, E = n_sink rounded up to a block).
// Row i sees keys j <= i when causal, all N keys otherwise; keys j < n_sink are sinks.
void pair_totals(int B, int H, int N, int causal, int n_sink, unsigned long long* all,
                 unsigned long long* sink) {
  const uint64_t n = (uint64_t)N, m = n - n_sink;
  const uint64_t e = ((uint64_t)n_sink + fp8attn::kKvBlock - 1) / fp8attn::kKvBlock * fp8attn::kKvBlock;
  const uint64_t k = e - n_sink;
  uint64_t per_head_all, per_head_sink;
  if (causal) {
    per_head_all = m * (m + 1) / 2;                 // rows n_sink + x see x + 1 such keys
    per_head_sink = k * (k + 1) / 2 + k * (n - e);  // rows below e, then k keys per row
  } else {
    per_head_all = n * m;
    per_head_sink = n * k;
  }
  *all = (uint64_t)B * H * per_head_all;
  *sink = (uint64_t)B * H * per_head_sink;
}

// n_sink for the counts and the sink split: within [0, N], and at most one block when
// block 0 is split.
bool n_sink_ok(int n_sink, int N, int kv_order) {
  if (n_sink < 0 || n_sink > N) return false;
  return kv_order != FP8ATTN_KV_REVERSE_SINK_LAST || n_sink <= fp8attn::kKvBlock;
}

fp8attn::Params make_params(const void* q, const void* k, const void* v, float* o,
                            int B, int H, int Hkv, int N, int d, int causal, int kv_order,
                            float S, const float* qd, const float* kd, const float* vd,
                            int n_sink, unsigned long long* counts, int denominator = FP8ATTN_DENOM_FP32) {
  fp8attn::Params p{};
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.o = o;
  p.q_descale = qd;
  p.k_descale = kd;
  p.v_descale = vd;
  p.counts = counts;
  p.B = B; p.H = H; p.Hkv = Hkv; p.N = N;
  p.causal = causal;
  p.reverse = kv_order != FP8ATTN_KV_FORWARD;
  p.n_sink = n_sink;
  p.sink_last = kv_order == FP8ATTN_KV_REVERSE_SINK_LAST && n_sink > 0;
  p.qden = denominator == FP8ATTN_DENOM_QUANTIZED;
  p.S = S;
  int e2 = 0;
  frexpf(S, &e2);                       // S = 2^k gives a mantissa of 1/2 and e2 = k + 1
  p.log2_S = (float)(e2 - 1);
  p.log2e_rsqrt_d = (float)(1.4426950408889634 / sqrt((double)d));
  if (counts) pair_totals(B, H, N, causal, n_sink, &p.pairs, &p.pairs_sink);
  // one query head per kv head whose K and V (E4M3: 2 N d bytes) fit half an XCD's 4 MB L2
#ifndef FP8ATTN_HEAD_MAJOR_BYTES
#define FP8ATTN_HEAD_MAJOR_BYTES (2ll << 20)
#endif
  p.head_major = H == Hkv && 2ll * N * d <= FP8ATTN_HEAD_MAJOR_BYTES;
  return p;
}

bool is_pow2(float S) {
  int e2 = 0;
  return frexpf(S, &e2) == 0.5f;
}

}  // namespace

extern "C" {

int fp8_attn_fwd(const void* q, const void* k, const void* v, float* o,
                 int B, int H, int Hkv, int N, int d,
                 int causal, int kv_order, float S,
                 const float* q_descale, const float* k_descale, const float* v_descale,
                 void* stream) {
  if (!q || !k || !v || !o || !q_descale || !k_descale || !v_descale) return FP8ATTN_EINVAL;
  if (kv_order == FP8ATTN_KV_REVERSE_SINK_LAST) return FP8ATTN_EINVAL;   // needs n_sink
  const int st = check_common(B, H, Hkv, N, d, causal, kv_order, S);
  if (st != FP8ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FP8ATTN_EUNSUPPORTED;
  const fp8attn::Params p = make_params(q, k, v, o, B, H, Hkv, N, d, causal, kv_order, S,
                                        q_descale, k_descale, v_descale, 0, nullptr);
  const hipError_t e = fp8attn::launch_fwd(p, d, is_pow2(S), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8ATTN_OK : FP8ATTN_ELAUNCH;
}

int fp8_attn_p_collapse_count(const void* q, const void* k,
                              int B, int H, int Hkv, int N, int d,
                              int causal, int kv_order, float S,
                              const float* q_descale, const float* k_descale,
                              int n_sink, unsigned long long* counts, void* stream) {
  if (!q || !k || !q_descale || !k_descale || !counts) return FP8ATTN_EINVAL;
  const int st = check_common(B, H, Hkv, N, d, causal, kv_order, S);
  if (st != FP8ATTN_OK) return st;
  if (!n_sink_ok(n_sink, N, kv_order)) return FP8ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k)) return FP8ATTN_EUNSUPPORTED;
  const fp8attn::Params p = make_params(q, k, nullptr, nullptr, B, H, Hkv, N, d, causal, kv_order, S,
                                        q_descale, k_descale, nullptr, n_sink, counts);
  const hipError_t e = fp8attn::launch_count(p, d, is_pow2(S), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8ATTN_OK : FP8ATTN_ELAUNCH;
}

int fp8_attn_fwd_counted(const void* q, const void* k, const void* v, float* o,
                         int B, int H, int Hkv, int N, int d,
                         int causal, int kv_order, float S,
                         const float* q_descale, const float* k_descale, const float* v_descale,
                         int n_sink, unsigned long long* counts, void* stream) {
  if (!q || !k || !v || !o || !q_descale || !k_descale || !v_descale || !counts) return FP8ATTN_EINVAL;
  const int st = check_common(B, H, Hkv, N, d, causal, kv_order, S);
  if (st != FP8ATTN_OK) return st;
  if (!n_sink_ok(n_sink, N, kv_order)) return FP8ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FP8ATTN_EUNSUPPORTED;
  const fp8attn::Params p = make_params(q, k, v, o, B, H, Hkv, N, d, causal, kv_order, S,
                                        q_descale, k_descale, v_descale, n_sink, counts);
  const hipError_t e = fp8attn::launch_fwd_count(p, d, is_pow2(S), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8ATTN_OK : FP8ATTN_ELAUNCH;
}

int fp8_attn_fwd_ex(const void* q, const void* k, const void* v, float* o,
                    int B, int H, int Hkv, int N, int d,
                    int causal, int kv_order, float S,
                    const float* q_descale, const float* k_descale, const float* v_descale,
                    int n_sink, int denominator, unsigned long long* counts, void* stream) {
  if (!q || !k || !v || !o || !q_descale || !k_descale || !v_descale) return FP8ATTN_EINVAL;
  const int st = check_common(B, H, Hkv, N, d, causal, kv_order, S);
  if (st != FP8ATTN_OK) return st;
  if (!n_sink_ok(n_sink, N, kv_order)) return FP8ATTN_EINVAL;
  if (denominator != FP8ATTN_DENOM_FP32 && denominator != FP8ATTN_DENOM_QUANTIZED) return FP8ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FP8ATTN_EUNSUPPORTED;
  const fp8attn::Params p = make_params(q, k, v, o, B, H, Hkv, N, d, causal, kv_order, S,
                                        q_descale, k_descale, v_descale, n_sink, counts, denominator);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool pow2 = is_pow2(S);
  const hipError_t e = counts ? fp8attn::launch_fwd_count(p, d, pow2, s) : fp8attn::launch_fwd(p, d, pow2, s);
  return e == hipSuccess ? FP8ATTN_OK : FP8ATTN_ELAUNCH;
}

unsigned long long fp8_attn_fwd_exact_qk_workspace_bytes(int B, int Hkv, int N, int d) {
  if (B <= 0 || Hkv <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
  return (unsigned long long)B * Hkv * N * d * 2ull;
}

int fp8_attn_fwd_exact_qk(const void* q, const void* k, const void* v, float* o,
                          int B, int H, int Hkv, int N, int d,
                          int causal, int kv_order, float S,
                          const float* q_descale, const float* k_descale, const float* v_descale,
                          int n_sink, int denominator, unsigned long long* counts,
                          void* workspace, unsigned long long workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !q_descale || !k_descale || !v_descale || !workspace) return FP8ATTN_EINVAL;
  const int st = check_common(B, H, Hkv, N, d, causal, kv_order, S);
  if (st != FP8ATTN_OK) return st;
  if (d != 64 && d != 128) return FP8ATTN_EUNSUPPORTED;
  if (2ll * N * d > INT32_MAX) return FP8ATTN_EUNSUPPORTED;   // one head's bf16 keys in a buffer range
  if (!n_sink_ok(n_sink, N, kv_order)) return FP8ATTN_EINVAL;
  if (denominator != FP8ATTN_DENOM_FP32 && denominator != FP8ATTN_DENOM_QUANTIZED) return FP8ATTN_EINVAL;
  if (workspace_bytes < fp8_attn_fwd_exact_qk_workspace_bytes(B, Hkv, N, d)) return FP8ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace))
    return FP8ATTN_EUNSUPPORTED;
  fp8attn::Params p = make_params(q, k, v, o, B, H, Hkv, N, d, causal, kv_order, S,
                                  q_descale, k_descale, v_descale, n_sink, counts, denominator);
  p.kx = static_cast<const uint8_t*>(workspace);
  p.exact_qk = 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = fp8attn::launch_keys_to_bf16(p.k, static_cast<uint8_t*>(workspace), (int64_t)B * Hkv * N * d, d, s);
  if (e != hipSuccess) return FP8ATTN_ELAUNCH;
  const bool pow2 = is_pow2(S);
  e = counts ? fp8attn::launch_fwd_count(p, d, pow2, s) : fp8attn::launch_fwd(p, d, pow2, s);
  return e == hipSuccess ? FP8ATTN_OK : FP8ATTN_ELAUNCH;
}

unsigned long long fp8_attn_decode_workspace_bytes(int B, int H, int d, int n_split) {
  if (B <= 0 || H <= 0 || n_split <= 0 || (d != 64 && d != 128 && d != 256)) return 0;
  return (unsigned long long)B * H * n_split * fp8attn::decode_record_floats(d) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks and launch of the split-KV decode with its split records in `workspace` (NULL:
// the library's static scratch of the current device, whose size is checked here).
int decode_impl(const void* q, const void* k, const void* v, float* o,
                int B, int H, int Hkv, int N, int d, int kv_order, float S,
                const float* q_descale, const float* k_descale, const float* v_descale,
                int n_split, void* workspace, unsigned long long workspace_bytes, bool static_scratch,
                void* stream);

}  // namespace

extern "C" {

int fp8_attn_decode(const void* q, const void* k, const void* v, float* o,
                    int B, int H, int Hkv, int N, int d, int kv_order, float S,
                    const float* q_descale, const float* k_descale, const float* v_descale,
                    int n_split, void* workspace, unsigned long long workspace_bytes, void* stream) {
  if (!workspace) return FP8ATTN_EINVAL;
  return decode_impl(q, k, v, o, B, H, Hkv, N, d, kv_order, S, q_descale, k_descale, v_descale, n_split,
                     workspace, workspace_bytes, false, stream);
}

int fp8_attn_decode_static(const void* q, const void* k, const void* v, float* o,
                           int B, int H, int Hkv, int N, int d, int kv_order, float S,
                           const float* q_descale, const float* k_descale, const float* v_descale,
                           int n_split, void* stream) {
  return decode_impl(q, k, v, o, B, H, Hkv, N, d, kv_order, S, q_descale, k_descale, v_descale, n_split,
                     nullptr, 0, true, stream);
}

}  // extern "C"

namespace {

// The static scratch of fp8_attn_decode_static: one array per GPU the library runs on,
// held until the process ends. In host code its name is a host-side stand-in, never a
// device address: the device address is looked up once per device (with that device
// current) and only that address is handed to the kernels.
static __device__ __align__(256) unsigned char scratch[FP8ATTN_STATIC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, or NULL if it cannot be found.
void* current_device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

int decode_impl(const void* q, const void* k, const void* v, float* o,
                int B, int H, int Hkv, int N, int d, int kv_order, float S,
                const float* q_descale, const float* k_descale, const float* v_descale,
                int n_split, void* workspace, unsigned long long workspace_bytes, bool static_scratch,
                void* stream) {
  if (!q || !k || !v || !o || !q_descale || !k_descale || !v_descale) return FP8ATTN_EINVAL;
  if (kv_order == FP8ATTN_KV_REVERSE_SINK_LAST) return FP8ATTN_EINVAL;
  const int st = check_common(B, H, Hkv, N, d, 0, kv_order, S);
  if (st != FP8ATTN_OK) return st;
  if (n_split < 1 || n_split > N / fp8attn::kKvBlock) return FP8ATTN_EINVAL;
  const unsigned long long need = fp8_attn_decode_workspace_bytes(B, H, d, n_split);
  if (static_scratch) {
    if (need > FP8ATTN_STATIC_SCRATCH_BYTES) return FP8ATTN_ESCRATCH;
  } else if (workspace_bytes < need) {
    return FP8ATTN_EINVAL;
  }
  const int G = H / Hkv;
  const int n_qgroups = (G + 31) / 32;
  if ((int64_t)B * Hkv * n_qgroups * n_split > INT32_MAX) return FP8ATTN_EUNSUPPORTED;
  if ((int64_t)B * H > INT32_MAX) return FP8ATTN_EUNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (!static_scratch && !aligned16(workspace)))
    return FP8ATTN_EUNSUPPORTED;
  if (static_scratch) {
    workspace = current_device_scratch();
    if (!workspace) return FP8ATTN_ELAUNCH;
  }
  fp8attn::DecodeParams p{};
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.o = o;
  p.ws = static_cast<float*>(workspace);
  p.q_descale = q_descale;
  p.k_descale = k_descale;
  p.v_descale = v_descale;
  p.B = B; p.H = H; p.Hkv = Hkv; p.N = N;
  p.n_split = n_split;
  p.n_qgroups = n_qgroups;
  p.reverse = kv_order == FP8ATTN_KV_REVERSE;
  p.S = S;
  int e2 = 0;
  frexpf(S, &e2);
  p.log2_S = (float)(e2 - 1);
  p.log2e_rsqrt_d = (float)(1.4426950408889634 / sqrt((double)d));
  const hipError_t e = fp8attn::launch_decode(p, d, is_pow2(S), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8ATTN_OK : FP8ATTN_ELAUNCH;
}

}  // namespace

extern "C" {

int fp8_attn_fwd_tile_rows(int B, int H, int Hkv, int N, int d, int causal, int kv_order, float S,
                           int n_sink, int denominator, int exact_qk) {
  const int st = check_common(B, H, Hkv, N, d, causal, kv_order, S);
  if (st != FP8ATTN_OK) return st;
  if (!n_sink_ok(n_sink, N, kv_order)) return FP8ATTN_EINVAL;
  if (denominator != FP8ATTN_DENOM_FP32 && denominator != FP8ATTN_DENOM_QUANTIZED) return FP8ATTN_EINVAL;
  if (exact_qk != 0 && exact_qk != 1) return FP8ATTN_EINVAL;
  if (exact_qk && (d > 128 || 2ll * N * d > INT32_MAX)) return FP8ATTN_EUNSUPPORTED;
  fp8attn::Params p = make_params(nullptr, nullptr, nullptr, nullptr, B, H, Hkv, N, d, causal, kv_order, S,
                                  nullptr, nullptr, nullptr, n_sink, nullptr, denominator);
  p.exact_qk = exact_qk;
  return fp8attn::fwd_tile_rows(p, d);
}

int fp8_attn_fwd_walk_groups(int B, int H, int Hkv, int N, int d, int causal, int kv_order, float S,
                             int n_sink, int denominator, int exact_qk) {
  const int rows = fp8_attn_fwd_tile_rows(B, H, Hkv, N, d, causal, kv_order, S, n_sink, denominator, exact_qk);
  if (rows < 0) return rows;
  fp8attn::Params p = make_params(nullptr, nullptr, nullptr, nullptr, B, H, Hkv, N, d, causal, kv_order, S,
                                  nullptr, nullptr, nullptr, n_sink, nullptr, denominator);
  p.exact_qk = exact_qk;
  return fp8attn::fwd_walk_groups(p, d);
}

int fp8_attn_kv_block(void) { return fp8attn::kKvBlock; }

const char* fp8_attn_version(void) { return "fp8attn-gfx950 0.2.0"; }

const char* fp8_attn_status_string(int status) {
  switch (status) {
    case FP8ATTN_OK: return "ok";
    case FP8ATTN_EINVAL: return "invalid argument";
    case FP8ATTN_EUNSUPPORTED: return "unsupported shape or alignment";
    case FP8ATTN_ELAUNCH: return "kernel launch failed";
    case FP8ATTN_ESCRATCH: return "request exceeds the static scratch of fp8_attn_decode_static";
    default: return "unknown status";
  }
}

}  // extern "C"
