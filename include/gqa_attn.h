/*
 * gqa_attn.h - exact grouped-query attention forward pass on AMD MI355X (gfx950).
 *
 * Operation (PyTorch profiling guide part 3, "the computational challenge of
 * attention" formula; Llama-2 GQA article, section 1.2):
 *
 *     O[b,i,h,:] = sum_j softmax_j(scale * Q[b,i,h,:] . K[b,j,g,:]) * V[b,j,g,:]
 *     LSE[b,h,i] = ln sum_j exp(scale * Q[b,i,h,:] . K[b,j,g,:])
 *
 * over the keys j visible to query i, where the query head h reads key/value
 * head g = h / (Hq/Hk): with Hq=6, Hk=2, query heads 0-2 read KV head 0 and
 * heads 3-5 read KV head 1, and Hq must be a multiple of Hk (batch-sensitivity
 * article, "core design of grouped-query attention"; rise-and-fall tuning
 * article, "root cause"). With causal != 0, key j is visible to query i iff
 * j <= i + Sk - Sq (bottom-right alignment; the usual j <= i when Sq == Sk).
 * A query that sees no key gets O = 0 and LSE = -inf. The result is exact up
 * to floating-point rounding: tiles, the online softmax, PackGQA and split-KV
 * only reorder the arithmetic.
 *
 * pack_gqa and num_splits are the two knobs of the pages' flash_attn_func
 * (Stable-Diffusion GQA guide, "dynamic batch scheduling"; batch-sensitivity
 * article, strategy 2 "PackGQA and num_splits"; rise-and-fall tuning article,
 * "fix" table): pack_gqa puts the query heads of one KV group into one tile
 * so each K/V tile is read once per group, and num_splits cuts the key axis
 * into parts whose partial results are merged with log-sum-exp weights
 * ("split + combine").
 *
 * Layouts (all row-major, last dimension contiguous, no padding):
 *   q, out : [B, Sq, Hq, d] bf16 (stored as 16-bit words)
 *   k, v   : [B, Sk, Hk, d] bf16
 *   lse    : [B, Hq, Sq] fp32, natural logarithm, or NULL to skip it
 * All tensor pointers are device pointers on the current HIP device and must
 * be 16-byte aligned. d must be 64 or 128.
 *
 * Ownership: the caller owns every tensor. The library allocates only
 * transient workspaces (the split-KV fp32 partial outputs and log-sums, the
 * work list of variable-length prefill, the backward's D and base-2
 * log-sum-exp), stream-ordered on the caller's stream
 * (hipMallocFromPoolAsync/hipFreeAsync) from a memory pool the library
 * creates per device, so calls on different streams never share them.
 * Workspaces of up to 64 MiB are kept per (device, stream handle), for the
 * first 16 such pairs, and reused by later calls on the same stream without
 * a new allocation (calls on one stream run in order); a call that needs
 * more grows the kept buffer stream-ordered. Kept buffers are held until the
 * process ends. Because they are tied to the stream handle, a stream that
 * ran such calls must have finished its work before it is destroyed (for
 * example hipStreamSynchronize first), so that a stream created later with
 * the same handle cannot overlap it. Calls during graph capture, calls on
 * further streams and larger workspaces are allocated and released per
 * call. The pool keeps up to 256 MiB of freed workspace reserved for later
 * calls and returns anything above that to the device at the next
 * synchronisation; the device's default pool is not modified. Other state:
 * a per-device cache of the compute-unit count (and, for
 * gqa_attn_fwd_noalloc, its fixed scratch array).
 *
 * Calls are asynchronous with respect to the host and never synchronize the
 * stream. They are thread-safe. No C++ exception crosses this boundary. A
 * forward call whose split count resolves to 1 enqueues exactly one kernel
 * and nothing else (no allocation, memset or copy), so it can be captured in
 * a HIP graph and replayed; split calls also enqueue the combine kernel
 * (and, where the workspace is not a kept one, its allocation and release), and
 * variable-length prefill calls of very different lengths a scheduling kernel
 * and its workspace.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. Every error is reported before anything is launched, and
 * leaves out and lse untouched, except GQA_ERR_HIP, which reports a failed
 * HIP call (allocation of the workspace aside) or launch. */
typedef enum {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = -1, /* null tensor pointer, negative size, Hq % Hk != 0,
                                 Sk == 0 while B*Sq > 0, pack_gqa not in {-1,0,1},
                                 num_splits < 0, non-finite scale, size overflow;
                                 paged: page_size, max_pages or num_pages <= 0;
                                 fp8: non-finite k_scale or v_scale */
    GQA_ERR_UNSUPPORTED = -2, /* d not in {64,128}, pointer not 16-byte aligned;
                                 fp8 K/V (contiguous or paged): more than 32
                                 query rows per head unit; paged: page_size %
                                 16 != 0, table pointers not 4-byte aligned */
    GQA_ERR_NOMEM = -3,       /* the split-KV workspace could not be allocated */
    GQA_ERR_HIP = -4,         /* a HIP call or kernel launch failed */
    GQA_ERR_SCRATCH = -5      /* gqa_attn_fwd_noalloc: the split-KV workspace of
                                 the call exceeds GQA_NOALLOC_SCRATCH_BYTES */
} gqa_status_t;

/* Forward pass.
 *   q, k, v, out, lse : see Layouts above. lse may be NULL.
 *   B, Sq, Sk         : batch size, query length, key length (B*Sq == 0: no-op).
 *   Hq, Hk, d         : query heads, key/value heads, head dimension.
 *   causal            : 0 or non-zero (bottom-right aligned mask, see above).
 *   scale             : softmax scale applied to Q.K (callers usually pass
 *                       1/sqrt(d)); any finite value, including 0 and negatives.
 *   pack_gqa          : 1 pack the G = Hq/Hk heads of a group into one tile,
 *                       0 one head per tile, -1 let gqa_attn_choose decide.
 *   num_splits        : >= 1 split the keys of every tile into that many parts
 *                       (clamped to the number of key tiles), 0 automatic.
 *   stream            : HIP stream the kernels are enqueued on (0 = null stream).
 * Returns a gqa_status_t. */
int gqa_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int Sq, int Sk, int Hq, int Hk, int d,
                 int causal, float scale, int pack_gqa, int num_splits,
                 hipStream_t stream);

/* Size of the fixed split-KV workspace of gqa_attn_fwd_noalloc, per GPU. */
#define GQA_NOALLOC_SCRATCH_BYTES (64LL << 20)

/* gqa_attn_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, semantics, checks and kernels as gqa_attn_fwd; the only
 * difference is where a split call (num_splits resolving to > 1) keeps its
 * fp32 partials: in a fixed device array of GQA_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends, instead
 * of a stream-ordered allocation. The call never allocates or frees memory
 * (no hipMalloc, hipMallocAsync, hipFree or allocating library routine).
 * The workspace a call needs is gqa_attn_plan's workspace_bytes
 * (num_splits * B*Sq*Hq * (4*d + 8)); a call that needs more returns
 * GQA_ERR_SCRATCH before anything is launched. The array's device address is
 * looked up on a device's first call (GQA_ERR_HIP if that fails). Every
 * call on one GPU shares that GPU's array: split calls that may overlap in
 * time on one GPU (different streams, or threads) race and must be ordered
 * by the caller. A call writes every partial it reads, so no state carries
 * over from the previous call. */
int gqa_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int Sq, int Sk, int Hq, int Hk, int d,
                         int causal, float scale, int pack_gqa, int num_splits,
                         hipStream_t stream);

/* Backward pass: gradients of the forward pass for an upstream gradient dout.
 *
 * The pages time the forward and backward passes of flash attention
 * together (batch-sensitivity article, "performance analysis"); the
 * gradients follow from the forward definition by the chain rule. With
 * P = softmax(scale * Q K^T) over the visible keys (recomputed from q, k and
 * the forward's lse), O = out and dO = dout, for query head h of KV head g:
 *   dV_g = sum_{h in g} P^T dO,  dK_g = scale * sum_{h in g} dS^T Q_h,
 *   dQ_h = scale * dS K_g,  dS = P * (dO V^T - D),  D_i = sum_c dO[i,c] O[i,c].
 * The query heads of a group share K and V, so their contributions add up.
 *   q, out, dout, dq : [B, Sq, Hq, d] bf16;  k, v, dk, dv : [B, Sk, Hk, d] bf16
 *   lse              : [B, Hq, Sq] fp32, the forward's log-sum-exp (required)
 *   causal, scale    : as passed to the forward call
 * out and lse must come from gqa_attn_fwd on the same inputs. The library
 * allocates a stream-ordered fp32 workspace of 2*B*Hq*Sq values (D and the
 * log-sum-exp in base 2). dq, dk
 * and dv are overwritten (keys no query sees get 0). With B*Sq == 0 only
 * dK = dV = 0 is written and q, out, lse, dout and dq may be null. Same validation,
 * alignment and stream rules as gqa_attn_fwd; additionally Sq*Hq*d*2 must
 * be below 2^31. */
int gqa_attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv,
                 int B, int Sq, int Sk, int Hq, int Hk, int d, int causal, float scale,
                 hipStream_t stream);

/* Forward pass over a batch of sequences of different lengths, packed along
 * the token axis.
 *
 * The pages list variable-length sequences among the uses of grouped-query
 * attention (batch-sensitivity article, "applicable scenarios") and the
 * continuous batching of generation requests (Llama-2 GQA article, section
 * 4.1), without a layout; this is the plainest reading:
 *   q, out        : [total_q, Hq, d] bf16, the B sequences' tokens one after another
 *   k, v          : [total_k, Hk, d] bf16
 *   lse           : [Hq, total_q] fp32, or NULL
 *   cu_seqlens_q  : [B+1] int32 device memory: sequence b owns query tokens
 *                   cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (non-decreasing, from 0)
 *   cu_seqlens_k  : [B+1] int32 device memory, the same for keys
 *   max_seqlen_q  : upper bound of every sequence's query count (sizes the grid)
 *   max_seqlen_k  : upper bound of every key count (used by the heuristic)
 * Every sequence is computed exactly as gqa_attn_fwd would compute it alone,
 * with its own lengths and bottom-right causal alignment; a sequence without
 * keys gives O = 0 and LSE = -inf. The offsets live on the device and are not
 * validated on the host: the kernels clamp them into [0, total] and a query
 * count to max_seqlen_q, so bad offsets give wrong results (tokens past
 * max_seqlen_q of a sequence are not written), never an out-of-bounds
 * access. Pointers as for gqa_attn_fwd (the offset arrays 4-byte aligned).
 * Calls with more than 32 query rows per head unit whose sequences hold
 * fewer than 3/4 of B * max_seqlen_q query tokens, and every call that runs
 * on the 8-wavefront kernel (unsplit, d = 128, enough rows), first run a small
 * scheduling kernel that lists, from the offsets, the (sequence, row tile)
 * work items that exist, heaviest first (causal calls on the 8-wavefront
 * kernel: pairs of a sequence's row tiles R-1-i and i, run by one workgroup),
 * into a stream-ordered workspace of 4 * (1 + 2 * (ceil(total_q * G / M) + B))
 * bytes (G = Hq/Hk with PackGQA, else 1; M = 128 rows per tile, 256 on the
 * 8-wavefront kernel, 512 for its causal pairs) taken from the library's pool
 * with the split workspace, if any.
 * Returns a gqa_status_t (B*max_seqlen_q == 0 or total_q == 0: no-op). */
int gqa_attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k,
                        int B, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                        int Hq, int Hk, int d, int causal, float scale, int pack_gqa, int num_splits,
                        hipStream_t stream);

/* Forward pass over a paged KV cache: decode, and prefill of a chunk of new
 * tokens against cached keys.
 *
 * The pages serve dynamic-length sequences (and caches of sequences longer
 * than 8192 tokens) with FlashAttention's paged KV cache (Stable-Diffusion
 * GQA guide, application scenario one and the troubleshooting checklist);
 * they fix no layout, so this one is the plainest reading:
 *   k_cache, v_cache : [num_pages, page_size, Hk, d] bf16, a pool of pages
 *   block_table      : [B, max_pages] int32, device memory. Entry (b, p) is
 *                      the pool page holding keys p*page_size ..
 *                      (p+1)*page_size - 1 of sequence b, so key j of
 *                      sequence b is row j % page_size of page
 *                      block_table[b][j / page_size].
 *   seqlens_k        : [B] int32, device memory: the number of keys of
 *                      sequence b (0 allowed: its rows get O = 0, LSE = -inf).
 *   q, out, lse      : as for gqa_attn_fwd ([B, Sq, Hq, d], [B, Hq, Sq]).
 * The result for sequence b is gqa_attn_fwd's over its seqlens_k[b] keys,
 * with the causal alignment of that length (key j visible to query i iff
 * j <= i + seqlens_k[b] - Sq). Table entries past a sequence's last page
 * and page rows past its last key are never read.
 *
 * Head units of at most 32 query rows (G * Sq with PackGQA, Sq without:
 * decode and a few speculative tokens) run on the decode kernel, larger ones
 * on the 4-wavefront tiled kernel, whose tile copies look up each group of
 * key rows' page in the table. Limits: page_size a positive multiple of 16.
 * num_splits and pack_gqa are resolved as for a contiguous call with
 * Sk = max_pages * page_size.
 * seqlens_k and block_table live on the device and are not validated on the
 * host: the kernel clamps a length to [0, max_pages * page_size] and a page
 * number to [0, num_pages - 1], so bad values give wrong results, never an
 * out-of-bounds read. Pointers to the caches, q and out 16-byte aligned,
 * block_table and seqlens_k 4-byte aligned. Ownership, errors, streams and
 * the split workspace are as for gqa_attn_fwd. */
int gqa_attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                       const int* block_table, const int* seqlens_k, void* out, float* lse,
                       int B, int Sq, int Hq, int Hk, int d,
                       int num_pages, int page_size, int max_pages,
                       int causal, float scale, int pack_gqa, int num_splits,
                       hipStream_t stream);

/* Forward pass with K and V stored as fp8, for decode-shaped calls.
 *
 * The pages name FP8 e4m3 as the way to halve the bandwidth pressure of
 * inference (rise-and-fall tuning article, "verification and further
 * directions"; Stable-Diffusion GQA guide, FP8 intermediate precision). Here
 * k and v hold OCP float8 e4m3 bytes (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, subnormals, no infinity, S.1111.111 = NaN), layout
 * [B, Sk, Hk, d] (one byte per element); q, out and lse are as for
 * gqa_attn_fwd. With per-tensor factors k_scale and v_scale the operation is
 * gqa_attn_fwd's over K = k_scale * k8 and V = v_scale * v8, computed as
 * scores (scale * k_scale) * q.k8 and output v_scale * sum_j P_j v8_j:
 * exact up to rounding like the bf16 path (every e4m3 value is exact in bf16).
 * k_scale and v_scale: any finite fp32 values (INVALID_ARG otherwise).
 * Decode-shaped calls only (at most 32 query rows per head unit, else
 * GQA_ERR_UNSUPPORTED); other rules as for gqa_attn_fwd. */
int gqa_attn_fwd_kv8(const void* q, const void* k, const void* v, float k_scale, float v_scale,
                     void* out, float* lse, int B, int Sq, int Sk, int Hq, int Hk, int d,
                     int causal, float scale, int pack_gqa, int num_splits, hipStream_t stream);

/* gqa_attn_fwd_paged over fp8 page pools ([num_pages, page_size, Hk, d]
 * e4m3 bytes), with gqa_attn_fwd_kv8's factors and rules. */
int gqa_attn_fwd_paged_kv8(const void* q, const void* k_cache, const void* v_cache,
                           float k_scale, float v_scale, const int* block_table, const int* seqlens_k,
                           void* out, float* lse, int B, int Sq, int Hq, int Hk, int d,
                           int num_pages, int page_size, int max_pages,
                           int causal, float scale, int pack_gqa, int num_splits,
                           hipStream_t stream);

/* Forward pass with Q and K stored as fp8: the scores on the fp8 matrix cores.
 *
 * The same FP8 e4m3 format as gqa_attn_fwd_kv8 (rise-and-fall tuning article,
 * "verification and further directions"; Stable-Diffusion GQA guide, FP8
 * intermediate precision), applied where it pays in compute-bound prefill:
 * q holds e4m3 bytes [B, Sq, Hq, d] and k e4m3 bytes [B, Sk, Hk, d]; v, out
 * and lse are bf16 / fp32 as for gqa_attn_fwd. With per-tensor factors
 * q_scale and k_scale the operation is gqa_attn_fwd's over Q = q_scale * q8,
 * K = k_scale * k8 and V, computed as scores (scale * q_scale * k_scale) *
 * q8.k8 on the 32x32x64 fp8 products, whose e4m3 x e4m3 products are exact
 * in the fp32 accumulation, and P V on the bf16 products exactly as
 * gqa_attn_fwd: the same tolerances as the bf16 path apply. Quantising Q and
 * K to e4m3 is the caller's step. q_scale, k_scale: any finite fp32 values
 * (INVALID_ARG otherwise). Decode-shaped calls run on the tiled kernel (no
 * decode specialisation); other rules as for gqa_attn_fwd. */
int gqa_attn_fwd_qk8(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                     void* out, float* lse, int B, int Sq, int Sk, int Hq, int Hk, int d,
                     int causal, float scale, int pack_gqa, int num_splits, hipStream_t stream);

/* The host heuristic behind pack_gqa = -1 / num_splits = 0. It follows the
 * pages' rationale (rise-and-fall tuning article, "root cause" and "fix"
 * table; batch-sensitivity article, "performance analysis"): pack when the
 * query rows of one head fill a tile poorly (short or ragged Sq, decode),
 * split the keys when there are too few tiles to fill the compute units.
 * The thresholds are chosen for MI355X, not copied from the pages' H100
 * tables. num_cus <= 0 means "ask the current device" (a host-only call
 * otherwise: no HIP call is made). Writes *pack_gqa in {0,1} and
 * *num_splits >= 1. Returns GQA_OK, or GQA_ERR_INVALID_ARG for invalid sizes
 * or null outputs. */
int gqa_attn_choose(int B, int Sq, int Sk, int Hq, int Hk, int d, int causal, int num_cus,
                    int* pack_gqa, int* num_splits);

/* Launch plan of one call, for tests and benchmarks. Host only: no HIP call
 * is made when num_cus > 0.
 * Environment: GQA_ATTN_FORCE_TILED=1 (read at every call's plan) keeps every
 * prefill call on the 4-wavefront tiled kernel instead of the 8-wavefront
 * one; the two compute the same results bit for bit, so the switch changes
 * only the speed (for comparisons and diagnosis). */
typedef struct {
    int pack_gqa;          /* resolved pack flag */
    int num_splits;        /* resolved and clamped split count */
    int block_m;           /* query rows per tile */
    int block_n;           /* keys per tile */
    int row_tiles;         /* row tiles per (batch, head unit) */
    int key_tiles;         /* key tiles of the longest row tile */
    long long grid;        /* workgroups of the attention kernel */
    long long combine_grid;/* workgroups of the combine kernel (0 if none) */
    long long workspace_bytes; /* split-KV workspace (0 if num_splits == 1) */
    int threads;           /* threads per attention workgroup: 64 (decode-shaped calls),
                              256 (tiled, 128-row tiles) or 512 (large unsplit bf16
                              calls: 256-row tiles, one workgroup per compute unit) */
} gqa_attn_plan_t;

/* Resolve pack_gqa / num_splits exactly as gqa_attn_fwd would and describe
 * the launches. Returns GQA_OK or the status gqa_attn_fwd would return for
 * these sizes (pointer checks aside). */
int gqa_attn_plan(int B, int Sq, int Sk, int Hq, int Hk, int d, int causal,
                  int pack_gqa, int num_splits, int num_cus, gqa_attn_plan_t* plan);

/* Static, human-readable text of a status code. */
const char* gqa_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
