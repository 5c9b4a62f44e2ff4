/*
 * fp8attn.h -- C ABI of the MI355X (gfx950) FP8 P-cast attention forward.
 *
 * The operation. Attention O = softmax(Q K^T / sqrt(d)) V computed block-wise with an
 * online softmax, where Q, K, V are OCP E4M3 ("e4m3fn") codes with fp32 descales, and
 * the probability tile P~ = exp(s - m) is multiplied by a static scale S and cast to
 * E4M3 before the P.V product; S is divided back out in the epilogue. The KV blocks
 * (64 keys each, aligned at key 0) are visited in forward (0 -> N) or reverse (N -> 0)
 * order; the running max m is updated once per block. This is the computation analysed
 * in "P-Cast Precision in FP8 Attention: Sink-Induced Collapse and the Optimality of
 * S=2^8" (gist.science technical summary, section 1 "Problem statement": P cast to E4M3
 * before P.V, the running max m, the KV block order and the static scale S; section 2
 * "Optimization 2", condition 1: S = 2^k makes the scale and its inverse exact).
 *
 * Per query row i (natural-log logits s_ij = (q_i . k_j) qd kd / sqrt(d)):
 *   for each visited block b:  m' = max(m, max_j s_ij);  a = exp(m - m');
 *                              P~_ij = exp(s_ij - m');    P8_ij = E4M3_RNE(P~_ij * S);
 *                              l = a l + sum_j P~_ij;     acc = a acc + sum_j P8_ij v_j;
 *   O_i = acc / (S l)
 * The row sum uses the unquantized P~. The kernel evaluates exponentials as exp2 of
 * log2(e)-scaled logits in fp32, accumulates both GEMMs in fp32 on the FP8 matrix
 * cores, and for S = 2^k applies the scale as an exponent offset (exact).
 *
 * Conventions shared by every entry point.
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or retains them. Tensors are dense, row-major, 16-byte aligned:
 *      q  [B][H][N][d]   uint8 E4M3 codes      o [B][H][N][d] float32 (written)
 *      k  [B][Hkv][N][d] uint8 E4M3 codes      v [B][Hkv][N][d] uint8 E4M3 codes
 *      q_descale [B*H], k_descale [B*Hkv], v_descale [B*Hkv] float32, each > 0 and
 *      finite (decoded value = code value * descale; per-tensor = the same value repeated).
 *  - Grouped-query attention: query head h reads kv head h / (H / Hkv).
 *  - causal != 0 masks key j > query i (equal query and key lengths).
 *  - kv_order: FP8ATTN_KV_FORWARD (0), FP8ATTN_KV_REVERSE (1), or, where an entry point
 *    takes n_sink, FP8ATTN_KV_REVERSE_SINK_LAST (2): the reverse walk with block 0 visited
 *    in two steps, its non-sink keys [n_sink, 64) first and the sink keys [0, n_sink)
 *    last (needs n_sink <= 64; n_sink = 0 is plain reverse). This carries the reason the
 *    technical summary gives for the reverse order (section 2, "Optimization 1": the sink
 *    should raise m only after every other P has been cast) to the tokens that share
 *    block 0 with the sinks.
 *  - 0 < S <= 448 (the E4M3 maximum; P~ <= 1 so P~ S never overflows). S = 2^k is exact;
 *    other values are accepted and round like any fp32 multiply.
 *  - stream: a hipStream_t passed as void* (NULL = the default stream). Calls are
 *    asynchronous: they enqueue kernels and return; no host synchronisation.
 *  - Errors: every argument is validated BEFORE any HIP call; on a negative status
 *    nothing has been launched and no memory was touched. FP8ATTN_ELAUNCH reports the
 *    HIP error recorded right after the launch. Device-side faults (bad pointers) are
 *    reported by HIP on later calls, as for any kernel.
 *  - NaN codes (0x7F / 0xFF) or non-finite descales propagate NaN into O; not detected.
 *  - Thread-safe; no exceptions cross the ABI. The only global state is the static device
 *    array of fp8_attn_decode_static (below) and a per-device cache of the compute-unit
 *    count that fp8_attn_fwd_tile_rows and fp8_attn_fwd_walk_groups read.
 */
#ifndef FP8ATTN_H
#define FP8ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8ATTN_OK = 0,
  FP8ATTN_EINVAL = -1,       /* null pointer, size <= 0, H % Hkv != 0, S not in (0,448],
                                causal not 0/1, kv_order not one the entry point takes,
                                n_sink out of [0, N] (out of [0, 64] for SINK_LAST),
                                denominator not 0/1 */
  FP8ATTN_EUNSUPPORTED = -2, /* d not in {64,128,256}, N % 64 != 0, N*d > 2^31-1,
                                pointer not 16-byte aligned, grid larger than 2^31-1
                                workgroups */
  FP8ATTN_ELAUNCH = -3,      /* HIP reported an error for the launch */
  FP8ATTN_ESCRATCH = -4      /* fp8_attn_decode_static: the split records need more than
                                FP8ATTN_STATIC_SCRATCH_BYTES */
} fp8attn_status;

enum { FP8ATTN_KV_FORWARD = 0, FP8ATTN_KV_REVERSE = 1, FP8ATTN_KV_REVERSE_SINK_LAST = 2 };

/* What the row sum l accumulates (fp8_attn_fwd_ex):
 *   FP8ATTN_DENOM_FP32       the unquantized P~ (times S), as in every other entry point;
 *   FP8ATTN_DENOM_QUANTIZED  the decoded cast operand dec(P8) = dec(E4M3(P~ S)), so that
 *                            the same quantized P forms numerator and denominator; then
 *                            O_i = acc / l. The EFQ-Softmax abstract ("EFQ-Softmax:
 *                            Exp-Free Quantization for Softmax") presents this consistency
 *                            for its own low-bit P; here it is applied to the E4M3 cast. */
enum { FP8ATTN_DENOM_FP32 = 0, FP8ATTN_DENOM_QUANTIZED = 1 };

/* The forward pass: writes o (every element of [B][H][N][d]). kv_order 0 or 1. */
int fp8_attn_fwd(const void* q, const void* k, const void* v, float* o,
                 int B, int H, int Hkv, int N, int d,
                 int causal, int kv_order, float S,
                 const float* q_descale, const float* k_descale, const float* v_descale,
                 void* stream);

/* P-collapse diagnostic: runs the same Q.K^T, running-max, exp and P~ S -> E4M3 path as
 * fp8_attn_fwd (same block order and S; no P.V, no output; kv_order 0, 1 or 2, where the
 * sink split of SINK_LAST does not change which blocks count as holding a sink) and
 * counts, over unmasked pairs (i, j) with key j >= n_sink ("non-sink"), the cast operands
 * that are the E4M3 zero. A collapse is a non-sink probability that underflows to zero under the running
 * max (technical summary, section 1; the fraction is the F(Delta, S) of section 2).
 *   counts[0]  collapsed non-sink P, all blocks
 *   counts[1]  of which in blocks that contain a sink key (64*b < n_sink)
 *   counts[2]  unmasked non-sink pairs, all blocks
 *   counts[3]  of which in blocks that contain a sink key
 * counts: DEVICE pointer to 4 uint64, overwritten (zeroed on `stream` by a kernel, then
 * accumulated with atomics). Read it after synchronising the stream. */
int fp8_attn_p_collapse_count(const void* q, const void* k,
                              int B, int H, int Hkv, int N, int d,
                              int causal, int kv_order, float S,
                              const float* q_descale, const float* k_descale,
                              int n_sink, unsigned long long* counts, void* stream);

/* The forward pass and the collapse diagnostic in one pass over the data: writes o exactly
 * as fp8_attn_fwd does and counts[0..3] exactly as fp8_attn_p_collapse_count does (same
 * arguments, same meaning, same ownership and error rules). */
int fp8_attn_fwd_counted(const void* q, const void* k, const void* v, float* o,
                         int B, int H, int Hkv, int N, int d,
                         int causal, int kv_order, float S,
                         const float* q_descale, const float* k_descale, const float* v_descale,
                         int n_sink, unsigned long long* counts, void* stream);

/* The forward pass with every option: kv_order 0, 1 or 2 (n_sink sets the sink tokens
 * of SINK_LAST and of the counts), the row-sum denominator (FP8ATTN_DENOM_*), and counts
 * either NULL (no diagnostic: o exactly as fp8_attn_fwd_counted would write it) or a
 * DEVICE pointer to 4 uint64 filled exactly as by fp8_attn_p_collapse_count. With
 * kv_order 0/1 and FP8ATTN_DENOM_FP32 the results equal those of fp8_attn_fwd and
 * fp8_attn_fwd_counted. Ownership, alignment and error rules as above. */
int fp8_attn_fwd_ex(const void* q, const void* k, const void* v, float* o,
                    int B, int H, int Hkv, int N, int d,
                    int causal, int kv_order, float S,
                    const float* q_descale, const float* k_descale, const float* v_descale,
                    int n_sink, int denominator, unsigned long long* counts, void* stream);

/* The forward pass of fp8_attn_fwd_ex (same arguments, options, outputs and counts) with
 * Q.K^T formed from exact E4M3 x E4M3 products accumulated in fp32, as the technical
 * summary's computation assumes (section 1: only P is cast; the logits are those of the
 * E4M3 operands). The FP8 matrix-core instruction of the other entry points truncates
 * small products inside its adder tree (up to ~2^-13 of the largest product of a group of
 * 8 k-slots); here S^T is formed on the bf16 matrix cores, which hold every E4M3 value
 * exactly, at half the FP8 rate. P.V stays on the FP8 matrix cores.
 *   d: 64 or 128, with 2*N*d <= 2^31-1 (one head's bf16 keys; EUNSUPPORTED otherwise).
 *   workspace: DEVICE buffer of at least fp8_attn_fwd_exact_qk_workspace_bytes(B, Hkv, N, d)
 *   bytes (the keys as bf16), 16-byte aligned, owned by the caller; its contents on entry do
 *   not matter and on return are unspecified. Calls sharing one workspace must not overlap.
 * Two kernels are enqueued on `stream`: the key conversion and the forward pass. Errors as
 * for fp8_attn_fwd_ex, plus EINVAL for a NULL or too small workspace. */
unsigned long long fp8_attn_fwd_exact_qk_workspace_bytes(int B, int Hkv, int N, int d);
int fp8_attn_fwd_exact_qk(const void* q, const void* k, const void* v, float* o,
                          int B, int H, int Hkv, int N, int d,
                          int causal, int kv_order, float S,
                          const float* q_descale, const float* k_descale, const float* v_descale,
                          int n_sink, int denominator, unsigned long long* counts,
                          void* workspace, unsigned long long workspace_bytes, void* stream);

/* Decode with the key range split (one query row per head, every query sees all N keys).
 * The N / 64 KV blocks are shared into n_split contiguous ranges (split s holds blocks
 * [floor(s nb / n_split), floor((s+1) nb / n_split)), 1 <= n_split <= N / 64). Each split
 * runs the online softmax with the P-cast above over its own keys -- its own running max,
 * its blocks in kv_order (0 or 1), S as above -- and the split states (m, l, acc) are
 * merged exactly through their maxima: with m = max_s m_s,
 *   O = sum_s acc_s e^(m_s - m) / (S sum_s l_s e^(m_s - m)),
 * the split-KV form of the FlashAttention recurrence the technical summary's section 1
 * describes. The cast depends on the partition (a split that does not hold the sink
 * tokens never sees their max).
 *   q  [B][H][d] uint8 E4M3, k, v [B][Hkv][N][d], o [B][H][d] float32 (written);
 *   q_descale [B*H], k_descale and v_descale [B*Hkv];
 *   workspace: DEVICE buffer of at least fp8_attn_decode_workspace_bytes(B, H, d, n_split)
 *   bytes, 16-byte aligned, owned by the caller; its contents on entry do not matter and
 *   on return are unspecified. Calls sharing one workspace must not overlap in time.
 * Errors as above (EINVAL also for a workspace that is NULL or too small, or n_split out
 * of range; EUNSUPPORTED for d not in {64,128,256}, N % 64 != 0 or a misaligned pointer).
 * Two kernels are enqueued on `stream`: the split pass and the merge. */
unsigned long long fp8_attn_decode_workspace_bytes(int B, int H, int d, int n_split);
int fp8_attn_decode(const void* q, const void* k, const void* v, float* o,
                    int B, int H, int Hkv, int N, int d, int kv_order, float S,
                    const float* q_descale, const float* k_descale, const float* v_descale,
                    int n_split, void* workspace, unsigned long long workspace_bytes, void* stream);

/* fp8_attn_decode for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same computation, arguments and
 * errors, with the split records held in a static device array of the library instead of
 * a caller workspace. Nothing is allocated (no hipMalloc, hipFree or allocating library
 * routine); the array, FP8ATTN_STATIC_SCRATCH_BYTES per GPU, is part of the library's code
 * object and held by every GPU it runs on until the process ends.
 *   Uses the array of the current device (the stream must belong to it); its device address
 *   is looked up once per device, on the first call there.
 *   FP8ATTN_ESCRATCH if fp8_attn_decode_workspace_bytes(B, H, d, n_split) exceeds
 *   FP8ATTN_STATIC_SCRATCH_BYTES (nothing launched).
 *   Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 *   (other streams, other threads) race and give undefined results; calls in one stream are
 *   ordered. No record needs clearing: each call writes every record it reads. */
#define FP8ATTN_STATIC_SCRATCH_BYTES (8u << 20)
int fp8_attn_decode_static(const void* q, const void* k, const void* v, float* o,
                           int B, int H, int Hkv, int N, int d, int kv_order, float S,
                           const float* q_descale, const float* k_descale, const float* v_descale,
                           int n_split, void* stream);

/* Query rows per wave of the forward kernels (fp8_attn_fwd, _counted, _ex,
 * _p_collapse_count, _exact_qk) for these arguments on the current device. Let C be the
 * device's compute units and T = B * H * ceil(N / 128) the tiles of 128 query rows. The
 * result is 16 when all of these hold, else 32:
 *  - d = 128;
 *  - no fwd_ex option is in effect: kv_order is not FP8ATTN_KV_REVERSE_SINK_LAST with
 *    n_sink > 0, and denominator is FP8ATTN_DENOM_FP32;
 *  - exact_qk is 0;
 *  - the forward has causal masking and 1.5 C < T <= 2 C. Below that the walk groups of
 *    fp8_attn_fwd_walk_groups take the grid.
 * Both shapes compute the same method within the same parity tolerance. The 16-row kernel
 * forms Q.K^T on the 16x16x128 FP8 matrix-core instruction, which accumulates by the same
 * rule as the 32x32x64 one. It forms P.V on the 16x16x32 one, whose own accumulation moves
 * O by a few 1e-4. Its workgroups of 64 rows fill and balance such a grid better.
 * Returns 16 or 32, or the negative status (EINVAL / EUNSUPPORTED) that the forward entry
 * points would return for these arguments. No GPU work; reads the device's compute-unit
 * count. */
int fp8_attn_fwd_tile_rows(int B, int H, int Hkv, int N, int d, int causal, int kv_order, float S,
                           int n_sink, int denominator, int exact_qk);

/* Walk groups of the 32-row forward kernel for these arguments on the current device (same
 * arguments and statuses as fp8_attn_fwd_tile_rows; C and T as there). The result is 2 when
 * d = 128, no fwd_ex option is in effect, exact_qk is 0, and the grid is small: 2 T <= 3 C
 * with causal masking, 2 T <= C without. Else it is 1.
 * With 2, a workgroup of 4 waves takes 64 query rows, and two groups of 2 waves split the
 * walk over the KV blocks: group g visits the walk positions g, g + 2, g + 4, ... After each
 * block's Q.K^T the groups trade their block row maxima through LDS. Each block's running
 * maximum, and so every P~ and its E4M3 code, is then the one of the sequential walk
 * ("P-Cast Precision in FP8 Attention", technical summary section 1: the running max
 * updated per KV block in the visiting order). The two partial states are merged once at
 * the end, which changes only the fp32 summation order of O. Counts are the same as with 1.
 * No GPU work; reads the device's compute-unit count. */
int fp8_attn_fwd_walk_groups(int B, int H, int Hkv, int N, int d, int causal, int kv_order, float S,
                             int n_sink, int denominator, int exact_qk);

/* Width in keys of the KV blocks between running-max updates (64). */
int fp8_attn_kv_block(void);

/* Library version string (static storage). */
const char* fp8_attn_version(void);

/* Human-readable name of a status code (static storage). */
const char* fp8_attn_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* FP8ATTN_H */
