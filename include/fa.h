/*
 * fa.h — C ABI of the MI355X (gfx950) exact tiled-attention library libfa.so.
 *
 * The operation is standard scaled-dot-product attention computed tile by
 * tile: Q/K/V blocks are staged on chip, QK^T feeds an online softmax that
 * keeps a running row max and row sum, the result is multiplied into V, and
 * the n x n score matrix is never written to memory.  The backward pass
 * recomputes scores from the saved log-sum-exp.  (Page "FlashAttention
 * 实战指南：如何把训练内存省 20 倍、速度提 4 倍", sections "长序列注意力为什么会爆内存"
 * and "FlashAttention 的做法是三个手段配合"; the result equals standard
 * attention exactly, same section.)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every tensor pointer is a DEVICE pointer unless stated otherwise,
 *   contiguous, innermost dimension stride 1, 16-byte aligned.  The caller
 *   allocates and frees every buffer, including workspaces; the library
 *   keeps no per-call state and allocates no device memory.
 * Layouts: q/out (B, Sq, Hq, D); k/v (B, Sk, Hkv, D) — the (batch, seqlen,
 *   nheads, headdim) layout of section "上手 FlashAttention 的三步走";
 *   lse float32 (B, Hq, Sq).  Packed varlen tensors are (total, H, D) with
 *   lse (Hq, total_q).
 * dtype: FA_DTYPE_FP16 or FA_DTYPE_BF16 for q/k/v/out/dout/dq/dk/dv; all
 *   accumulation is float32.
 * Score transform, in this order (section "进阶参数如何配置causal、window_size 与
 *   MQA/GQA"): s = scale * q.k; softcap c > 0 gives z = c * tanh(s / c);
 *   alibi gives z -= slope[h] * |i + Sk - Sq - j|; keys outside the window
 *   [i' - window_left, i' + window_right] (i' = i + Sk - Sq, -1 = unbounded,
 *   causal forces window_right = 0) are masked.  A row with no visible key
 *   returns O = 0 and LSE = +inf.  LSE is the natural-log log-sum-exp of z.
 * GQA/MQA: Hq must be a multiple of Hkv; query head h reads K/V head
 *   h / (Hq / Hkv).
 * Streams: `stream` is a hipStream_t passed as void* (NULL = default
 *   stream).  Calls only enqueue work; they never synchronise the device.
 * Errors: every call validates its arguments on the host before launching
 *   anything; on error it returns a non-zero fa_status and writes nothing.
 *   FA_ERR_LAUNCH reports a launch failure seen by hipGetLastError.
 * Device preconditions that are NOT checked (the data lives on the device):
 *   cu_seqlens non-decreasing with cu[0] = 0 and cu[nseq] = total;
 *   every block_table entry that covers a live position is a valid page;
 *   cache capacity covers cache_seqlens[b] + Sq_new.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* a size, pointer, option or alignment is invalid */
  FA_ERR_UNSUPPORTED = 2, /* valid request the library has no kernel for (e.g. D = 80) */
  FA_ERR_WORKSPACE = 3,   /* workspace pointer NULL or smaller than the size query */
  FA_ERR_LAUNCH = 4,      /* hipGetLastError reported an error after a launch */
  FA_ERR_SCRATCH_LIMIT = 5 /* fa_fwd_kvcache_noalloc: partials exceed its static scratch */
} fa_status;

typedef enum { FA_DTYPE_FP16 = 0, FA_DTYPE_BF16 = 1 } fa_dtype;

/* Human-readable text for a status code (static storage, never NULL). */
const char* fa_status_string(int status);

/*
 * Forward pass (section "FlashAttention 的做法是三个手段配合": tiles, online
 * softmax; section "进阶参数如何配置…": causal, window, softcap, alibi, GQA).
 *   q (B,Sq,Hq,D), k/v (B,Sk,Hkv,D) in: 16-bit, read only.
 *   out (B,Sq,Hq,D) out: 16-bit, rounded once from float32.
 *   lse (B,Hq,Sq) out: float32; may be NULL when the caller does not need it.
 *   D in {32, 64, 96, 128, 256} (96 runs on the 128-wide kernels with the
 *   head padded on chip); scale > 0 finite; softcap >= 0 (0 = off);
 *   alibi_slopes: NULL or float32 (Hq,) device array, one slope per query head.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
           int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
           float scale, int causal, int window_left, int window_right, float softcap,
           const float* alibi_slopes, void* stream);

/*
 * Backward pass: recomputes the attention weights from q, k and the saved
 * lse instead of storing them (section "FlashAttention 的做法是三个手段配合",
 * recomputation).  Inputs as for fa_fwd plus out, dout (B,Sq,Hq,D) and the
 * forward's lse.  Outputs dq (B,Sq,Hq,D), dk/dv (B,Sk,Hkv,D), 16-bit,
 * overwritten (not accumulated into).  GQA gradients are summed over the
 * query heads of each group in a fixed order.
 * deterministic (section "进阶参数如何配置…", deterministic=True): this
 *   implementation never uses atomics, so every call is bitwise reproducible
 *   whatever the flag; the flag is accepted for API compatibility.
 * workspace: device buffer of at least fa_bwd_workspace_size(...) bytes.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
           float scale, int causal, int window_left, int window_right, float softcap,
           const float* alibi_slopes, int deterministic,
           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fa_bwd needs (host-only, pure): two float32 row arrays
 * (B, Hq, Sq) -- the negated row term -sum_d dO*O and the LSE in log2
 * units -- each padded to 256 bytes. */
size_t fa_bwd_workspace_size(int B, int Sq, int Sk, int Hq, int Hkv, int D, int deterministic);

/*
 * Packed variable-length forward / backward (section "上手 FlashAttention 的三步走":
 * batches of sequences with different lengths use the varlen interface).
 *   q/out/dout/dq (total_q, Hq, D); k/v/dk/dv (total_k, Hkv, D); lse (Hq, total_q).
 *   cu_seqlens_q/k: int32 device arrays (nseq + 1), prefix sums of lengths.
 *   max_seqlen_q/k: upper bounds of the per-sequence lengths.
 * Sequence s is attention over rows [cu_q[s], cu_q[s+1]) x [cu_k[s], cu_k[s+1]),
 * independent of every other sequence.  dk/dv rows that belong to no
 * sequence are left untouched.
 * Scheduling: a small kernel first writes, into the workspace, the list of
 * the real (sequence, tile) pairs from cu_seqlens (on the device, no host
 * synchronisation); the attention kernels then run one work-group per
 * (list entry, head) and no work-group for tiles past a sequence's end.
 * With up to 4096 sequences the list takes the sequences longest first, in
 * groups of max(1, 32 / heads), each group level by level with its heaviest
 * causal tiles first (so about four (sequence, head) pairs share each of the
 * chip's eight L2 caches at a time); with more, it goes level by level over
 * all sequences.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                  int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                  int Hq, int Hkv, int D, int dtype,
                  float scale, int causal, int window_left, int window_right, float softcap,
                  const float* alibi_slopes, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for fa_fwd_varlen: the tile list, 8 bytes per entry for at
 * most (total_q + 127 nseq) / 128 entries, padded to 256 bytes (0 when
 * total_q == 0, and the pointer may then be NULL). */
size_t fa_fwd_varlen_workspace_size(int nseq, int total_q, int Hq, int D);

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                  int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                  int Hq, int Hkv, int D, int dtype,
                  float scale, int causal, int window_left, int window_right, float softcap,
                  const float* alibi_slopes, int deterministic,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for fa_bwd_varlen: two float32 (Hq, total_q) row arrays, then
 * the list of 128-row query tiles (for dQ) and the list of key tiles (256
 * keys; 128 at D = 256, for dK/dV), each padded to 256 bytes. */
size_t fa_bwd_varlen_workspace_size(int nseq, int total_q, int total_k, int Hq, int D, int deterministic);

/*
 * Packed layouts (section "上手 FlashAttention 的三步走": when Q, K and V are
 * already packed into one tensor, the qkvpacked call is the faster route).
 *   fa_*_qkvpacked: qkv (B, S, 3, H, D) in -- q, k, v interleaved per token,
 *     so Sq = Sk = S and Hq = Hkv = H; dqkv (B, S, 3, H, D) out.
 *   fa_*_kvpacked: q (B, Sq, Hq, D), kv (B, Sk, 2, Hkv, D); dkv likewise.
 *   out, dout (B, Sq, Hq, D) and lse are laid out as for fa_fwd / fa_bwd.
 * Same kernels as fa_fwd / fa_bwd, reading and writing with the packed row
 * strides; same options, results and workspace (fa_bwd_workspace_size).
 */
int fa_fwd_qkvpacked(const void* qkv, void* out, float* lse, int B, int S, int H, int D, int dtype,
                     float scale, int causal, int window_left, int window_right, float softcap,
                     const float* alibi_slopes, void* stream);

int fa_bwd_qkvpacked(const void* qkv, const void* out, const void* dout, const float* lse,
                     void* dqkv, int B, int S, int H, int D, int dtype,
                     float scale, int causal, int window_left, int window_right, float softcap,
                     const float* alibi_slopes, int deterministic,
                     void* workspace, size_t workspace_bytes, void* stream);

int fa_fwd_kvpacked(const void* q, const void* kv, void* out, float* lse,
                    int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                    float scale, int causal, int window_left, int window_right, float softcap,
                    const float* alibi_slopes, void* stream);

int fa_bwd_kvpacked(const void* q, const void* kv, const void* out, const void* dout,
                    const float* lse, void* dq, void* dkv,
                    int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                    float scale, int causal, int window_left, int window_right, float softcap,
                    const float* alibi_slopes, int deterministic,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 forward (page "FlashAttention实战指南：如何在AMD GPU上突破大模型训练瓶颈",
 * section "性能优化技巧", item "FP8混合精度支持": FP8 support on AMD GPUs for
 * lower memory bandwidth at kept accuracy; page "FlashAttention 实战指南…",
 * section "版本怎么选": an FP8 forward pass).  q (B,Sq,Hq,D), k/v (B,Sk,Hkv,D): OCP
 * e4m3 bytes (torch.float8_e4m3fn); descale_q / descale_k / descale_v:
 * NULL or float32 (B, Hkv) device arrays, the factor that turns the stored
 * fp8 value of batch entry b, K/V head h (for q: its query heads) back into
 * the real value.  out (B,Sq,Hq,D) bfloat16; lse as fa_fwd.  The result is
 * attention on the dequantised inputs: S = q.k is formed exactly from the
 * fp8 products on the fp8 matrix instruction and scaled by
 * descale_q * descale_k; P V runs in bfloat16 after an exact fp8 -> bfloat16
 * copy of v into the workspace, and O is scaled by descale_v.  D in {64, 128};
 * options as fa_fwd.  workspace: fa_fwd_fp8_workspace_size(...) bytes.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
               int B, int Sq, int Sk, int Hq, int Hkv, int D,
               float scale, int causal, int window_left, int window_right, float softcap,
               const float* alibi_slopes, const float* descale_q, const float* descale_k,
               const float* descale_v, void* workspace, size_t workspace_bytes, void* stream);

size_t fa_fwd_fp8_workspace_size(int B, int Sk, int Hkv, int D);

/*
 * Dropout on the attention weights (the dropout_p argument of the attention
 * call in section "上手 FlashAttention 的三步走" and in the interface listing
 * of page "终极指南：如何通过FlashAttention实现Transformer模型的4倍加速与20倍内存优化").
 * Same arguments and outputs as fa_fwd / fa_bwd / fa_fwd_varlen /
 * fa_bwd_varlen, plus:
 *   dropout_p in [0, 255.5/256): the drop probability, rounded to
 *     t / 256 with t = round(256 p) (ties to even); t = 0 runs the plain
 *     kernels.  Kept weights are scaled by 256 / (256 - t).
 *   seed: 64-bit key of the counter-based generator Philox4x32-10
 *     (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *     1, 2, 3", SC 2011); offset: its low 32 bits are counter word 3, so
 *     successive steps pass distinct offsets.
 * Pair (query row i, key j) of batch entry b (varlen: sequence b; i, j
 * counted within the sequence) and query head h is kept when byte j % 4 of
 * word i % 4 of Philox4x32-10(counter = (j / 4, i / 4, b * Hq + h, offset),
 * key = seed) is >= t.  out = (P * keep * 256 / (256 - t)) V; lse is that of
 * the undropped weights.  The backward must get the same p, seed and offset
 * as the forward; it regenerates the mask and stores nothing.
 * Returns FA_ERR_INVALID_ARG for p outside the range or NaN.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                   int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                   float scale, int causal, int window_left, int window_right, float softcap,
                   const float* alibi_slopes, float dropout_p, unsigned long long seed,
                   unsigned long long offset, void* stream);

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* out, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv,
                   int B, int Sq, int Sk, int Hq, int Hkv, int D, int dtype,
                   float scale, int causal, int window_left, int window_right, float softcap,
                   const float* alibi_slopes, float dropout_p, unsigned long long seed,
                   unsigned long long offset, int deterministic,
                   void* workspace, size_t workspace_bytes, void* stream);

int fa_fwd_varlen_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                          const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                          int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                          int Hq, int Hkv, int D, int dtype,
                          float scale, int causal, int window_left, int window_right, float softcap,
                          const float* alibi_slopes, float dropout_p, unsigned long long seed,
                          unsigned long long offset, void* workspace, size_t workspace_bytes, void* stream);

int fa_bwd_varlen_dropout(const void* q, const void* k, const void* v, const void* out,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          const int* cu_seqlens_q, const int* cu_seqlens_k, int nseq,
                          int max_seqlen_q, int max_seqlen_k, int total_q, int total_k,
                          int Hq, int Hkv, int D, int dtype,
                          float scale, int causal, int window_left, int window_right, float softcap,
                          const float* alibi_slopes, float dropout_p, unsigned long long seed,
                          unsigned long long offset, int deterministic,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Incremental decode against a (paged) KV cache (section "增量解码场景
 * flash_attn_with_kvcache"): the new k/v are appended to the cache in place
 * and the new queries attend over the cache plus the appended tokens.
 *   q (B, Sq_new, Hq, D) in; (Hq / Hkv) * Sq_new <= 32 (the new queries of
 *     one K/V head are the 32 columns of one matrix tile), D in
 *     {32, 64, 96, 128} (96 padded to 128 on chip).
 *   k_new/v_new (B, Sq_new, Hkv, D) in, or both NULL (attend without append).
 *   k_cache/v_cache in/out: paged (n_pages, page_size, Hkv, D) when
 *     block_table != NULL, else contiguous (B, max_blocks_per_seq*page_size, Hkv, D).
 *   cache_seqlens: int32 (B,) valid length of each cache BEFORE the append;
 *     never modified (the caller advances it).
 *   block_table: int32 (B, max_blocks_per_seq); entry p of row b is the
 *     physical page of logical positions [p*page_size, (p+1)*page_size).
 *   page_size: a positive multiple of 32.
 *   rotary_cos/rotary_sin: NULL or float32 (max_pos, rotary_dim/2) tables;
 *     the half-split rotation of pairs (x_i, x_{i+rotary_dim/2}) at position
 *     cache_seqlens[b] + t is applied to q and k_new (not to v, not to the
 *     cached keys).  rotary_dim: multiple of 16, <= D (0 = no rotary).
 *   out (B, Sq_new, Hq, D) out; lse (B, Hq, Sq_new) float32 out or NULL.
 *   num_splits >= 1: the keys of each sequence are cut into num_splits
 *     contiguous page ranges processed in parallel and merged exactly; the
 *     result does not depend on it beyond float32 rounding.  num_splits == 0:
 *     the library chooses (about 1024 work-groups over B * Hkv, at most 32
 *     splits and at most max_blocks_per_seq).
 *   Positions: with k_new the keys are the cache plus the Sq_new appended
 *     rows; new query t sits at key position n_keys - Sq_new + t
 *     (bottom-right alignment) and is rotated at cache_seqlens[b] + t.
 *   causal: new query t sees the keys up to its own position (with
 *     Sq_new == 1 that is every key); otherwise it sees every key.
 *   window_left / window_right (-1 = unbounded): keys outside
 *     [position - window_left, position + window_right] are masked (causal
 *     sets window_right to 0).
 *   softcap (0 = off) and alibi_slopes (NULL or float32 (Hq,)): as in
 *     fa_fwd, with the ALiBi distance measured from each new query's position.
 *   With Sq_new > 1 the append runs as its own kernel before the attention;
 *   with Sq_new == 1 the attention kernel appends in its prologue.
 *   workspace: fa_kvcache_workspace_size(...) bytes (0 when num_splits == 1),
 *     computed with the same num_splits argument (0 included).
 * Appended slot (b, cache_seqlens[b] + t) receives the rotated k_new rounded
 * once to the cache dtype and v_new unchanged; no other cache byte changes.
 */
int fa_fwd_kvcache(const void* q, const void* k_new, const void* v_new,
                   void* k_cache, void* v_cache, const int* cache_seqlens,
                   const int* block_table, int max_blocks_per_seq, int page_size,
                   const float* rotary_cos, const float* rotary_sin, int rotary_dim,
                   void* out, float* lse,
                   int B, int Sq_new, int Hq, int Hkv, int D, int dtype,
                   float scale, int causal, int window_left, int window_right, float softcap,
                   const float* alibi_slopes, int num_splits,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for fa_fwd_kvcache: float32 split partials O_s (B,Hq,Sq_new,num_splits,D)
 * and LSE_s (B,Hq,Sq_new,num_splits), or 0 when num_splits == 1; num_splits == 0
 * returns the size for 32 splits, enough for any automatic choice. */
size_t fa_kvcache_workspace_size(int B, int Sq_new, int Hq, int D, int num_splits);

/*
 * fa_fwd_kvcache without a workspace argument, for callers that cannot
 * allocate device memory around the call (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * semantics and results as fa_fwd_kvcache (the same kernels run); the split
 * partials go to a static device array of fa_kvcache_noalloc_max_bytes()
 * bytes (8 MiB) that the library holds on each GPU it runs on until the
 * process ends.  The call allocates nothing and calls no allocating routine;
 * on the first call on a device it looks up that device's copy of the array
 * (hipGetSymbolAddress) and keeps the address.
 *   The current device must be the device of `stream` and of the tensors.
 *   Returns FA_ERR_SCRATCH_LIMIT when fa_kvcache_workspace_size(B, Sq_new,
 *   Hq, D, splits) exceeds the array, with splits = num_splits or, for
 *   num_splits == 0, the library's automatic choice (e.g. D = 128:
 *   B * Sq_new * Hq * splits <= 16256).
 *   Every call on a GPU shares that GPU's array: calls that may overlap on
 *   one GPU (different streams, or several host threads) race and must be
 *   ordered by the caller.  The array needs no clearing: each call writes
 *   every partial it reads.
 */
int fa_fwd_kvcache_noalloc(const void* q, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, const int* cache_seqlens,
                           const int* block_table, int max_blocks_per_seq, int page_size,
                           const float* rotary_cos, const float* rotary_sin, int rotary_dim,
                           void* out, float* lse,
                           int B, int Sq_new, int Hq, int Hkv, int D, int dtype,
                           float scale, int causal, int window_left, int window_right, float softcap,
                           const float* alibi_slopes, int num_splits, void* stream);

/* Bytes of the static scratch array behind fa_fwd_kvcache_noalloc. */
size_t fa_kvcache_noalloc_max_bytes(void);

/*
 * Kernel timing (for benchmarks and profiles).  When enabled, every kernel
 * the library launches is bracketed by a pair of HIP events recorded on the
 * launch stream (created without the system-scope fence, which would add the
 * write-back of the kernel's output to the interval).  fa_profiler_read synchronises on the recorded events and
 * returns, per kernel kind, the summed duration in milliseconds and the
 * number of launches since the last reset.  Event pairs come from a pool
 * created by fa_profiler_enable(1, capacity); launches past the capacity are
 * not timed.  Host-side state, not thread safe; intended for one thread.
 */
typedef enum {
  FA_KERNEL_FWD = 0,
  FA_KERNEL_BWD_PREPROCESS = 1, /* kept for numbering; no longer launched (the dQ kernel forms the row terms) */
  FA_KERNEL_BWD_DKDV = 2,
  FA_KERNEL_BWD_DQ = 3,
  FA_KERNEL_DECODE_SPLIT = 4,
  FA_KERNEL_DECODE_COMBINE = 5,
  FA_KERNEL_KIND_COUNT = 6
} fa_kernel_kind;

int fa_profiler_enable(int enable, int capacity);
int fa_profiler_reset(void);
int fa_profiler_read(int kind, double* total_ms, long* launches);
const char* fa_kernel_name(int kind);

#ifdef __cplusplus
}
#endif
#endif /* FA_H_ */
