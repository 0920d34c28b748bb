/*
 * dsa_sparse_mla.h -- C ABI of the DSA sparse MLA forward (and its backward)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation: for each query token t and query head h, attention over only
 * the KV rows that the token's index row names. One latent KV row per key is
 * shared by every head (kv_group = 1). Rows are 576 bf16 wide (512 latent +
 * 64 rope); scores use all 576 columns, values are the leading 512. The call
 * returns the bf16 output O[t, h, 0:512] and the fp32 log-sum-exp LSE[t, h].
 *
 * Sources (pages on the web about this method):
 *   - "[Feature] Add optional FlashMLA backend for DSA Sparse MLA"
 *     (InternLM/xtuner PR 2083), sections Motivation and Runtime constraints:
 *     the forward returns output and LSE; kv_group = 1; value width 512.
 *   - "feat: add XTuner TileLang sparse MLA backend" (InternLM/lmdeploy PR
 *     4904), section Performance > Isolated sparse MLA forward (bf16 Q/KV,
 *     dqk 576, dv 512, topk 2048, 8 TP-local heads) and Validation (-1-padded
 *     index rows); section Summary (packed prefill and zero-copy bf16
 *     paged-cache decode run the same kernel) and the per-file overview
 *     (logical-to-physical index mapping through the page table).
 *
 * Conventions shared by every entry point:
 *   - Tensors are plain device pointers. Strides are in elements; the last
 *     dimension of q, kv, out is contiguous. bf16 pointers must be 16-byte
 *     aligned and bf16 strides multiples of 8 elements; lse must be 4-byte
 *     aligned.
 *   - Ownership: every buffer belongs to the caller, scratch included (each
 *     entry point that needs scratch has a workspace query and takes a
 *     caller-provided workspace). The library allocates no device memory,
 *     keeps no pointer after it returns, and holds no state except a
 *     per-device property cache filled once. Calls may come from several host
 *     threads.
 *   - Asynchrony: a call only enqueues kernels on `stream` (a hipStream_t;
 *     NULL is the default stream). It never synchronises. Faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - Index entries are never checked on the host (that would need a sync).
 *     The kernel skips an entry that names no row (-1 padding or any value
 *     out of range), so no index value can make it read out of bounds.
 *     Duplicate entries count once per occurrence.
 *   - A token with no valid entry gets O = 0 and LSE = -inf.
 *   - LSE is the natural log of sum_j exp(sm_scale * q . k_j).
 *   - num_tokens == 0 is a no-op that returns DSA_OK.
 *   - Each workgroup gathers at most 2048 index entries; a longer topk is split
 *     over several workgroups whose partial results are merged by a second
 *     kernel through the caller's workspace. Shorter rows may also be split
 *     for parallelism (num_splits = 0 lets the library choose).
 *   - Every entry point returns a dsa_status and never throws.
 *   - Outputs may not overlap inputs or other outputs. The host compares byte
 *     extents (first to last element of each strided tensor), so two views
 *     that interleave inside one allocation are rejected even where they
 *     share no element.
 */
#ifndef DSA_SPARSE_MLA_H
#define DSA_SPARSE_MLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_DQK 576       /* query/key width: 512 latent + 64 rope */
#define DSA_DV 512        /* value width: the latent part */
#define DSA_MAX_HEADS 128
#define DSA_MAX_TOPK 65536
#define DSA_SEGMENT 2048  /* index entries one workgroup gathers */

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, stride or alignment */
  DSA_ERR_UNSUPPORTED = 2,      /* device is not gfx950, or a size past the limits above */
  DSA_ERR_HIP = 3,              /* a HIP runtime call or kernel launch failed */
  DSA_ERR_WORKSPACE = 4         /* the chosen split needs more workspace than given */
} dsa_status;

/*
 * Workspace query for dsa_sparse_mla_fwd / dsa_sparse_mla_fwd_paged.
 *
 * num_tokens, num_heads, topk: as in the forward call.
 * num_splits: 0 = let the library choose; otherwise the split count the caller
 *   will request. Must be >= ceil(topk / 2048) and <= topk.
 * *splits_out (may be NULL): the split count a forward call with these
 *   arguments uses, on the current device.
 * *bytes_out: workspace bytes that call needs (0 when it does not split).
 * Returns DSA_OK or DSA_ERR_INVALID_ARGUMENT / DSA_ERR_UNSUPPORTED.
 */
int dsa_sparse_mla_workspace_size(int64_t num_tokens, int32_t num_heads, int32_t topk,
                                  int32_t num_splits, int32_t* splits_out,
                                  int64_t* bytes_out);

/*
 * Sparse MLA forward over a flat KV array (packed or varlen prefill).
 * Pages: xtuner PR 2083 (Motivation, Runtime constraints); lmdeploy PR 4904
 * (Summary; Performance > Isolated sparse MLA forward; Validation).
 *
 * q        bf16 [num_tokens, num_heads, 576]; element (t,h,d) at
 *          q + t*q_stride_tok + h*q_stride_head + d
 * kv       bf16 [num_kv, 576]; row i at kv + i*kv_stride_row. Packed batches
 *          use one array for all documents and global row ids in `indices`.
 * indices  int32 [num_tokens, topk]; entry (t,j) at indices + t*idx_stride_tok + j.
 *          A key iff 0 <= value < num_kv; anything else is skipped.
 * sm_scale softmax scale applied to q . k; finite and >= 0 (the kernels
 *          fold it into the exponent after taking the raw-score max).
 * out      bf16 [num_tokens, num_heads, 512] (written), strides as for q.
 * lse      fp32 [num_tokens, num_heads] (written); (t,h) at lse + t*lse_stride_tok + h.
 * num_splits 0 = library's choice, else the split count (see the workspace query).
 * workspace/workspace_bytes  device scratch of at least the queried size when
 *          the call splits; may be NULL/0 otherwise. Its contents on entry do
 *          not matter; calls that share one workspace must be stream-ordered.
 * stream   hipStream_t to enqueue on.
 *
 * Limits: 1 <= num_heads <= 128, 1 <= topk <= 65536, num_kv * kv_stride_row * 2
 * bytes < 64 GiB. out, lse and the workspace must not overlap the inputs or
 * each other (checked on the host: DSA_ERR_INVALID_ARGUMENT).
 */
int dsa_sparse_mla_fwd(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                       const void* kv, int64_t kv_stride_row, int64_t num_kv,
                       const int32_t* indices, int64_t idx_stride_tok,
                       int64_t num_tokens, int32_t num_heads, int32_t topk, float sm_scale,
                       void* out, int64_t out_stride_tok, int64_t out_stride_head,
                       float* lse, int64_t lse_stride_tok,
                       int32_t num_splits, void* workspace, int64_t workspace_bytes,
                       void* stream);

/*
 * Sparse MLA forward over a paged bf16 KV cache (decode), with no gather copy.
 * Pages: lmdeploy PR 4904, Summary (zero-copy BF16 paged-cache decode with
 * the same kernel) and the per-file overview (logical-to-physical index
 * mapping); page size 64 in the decode workload.
 *
 * Query token t belongs to sequence b = t / q_per_seq; num_tokens = num_seqs * q_per_seq.
 * kv_pages   bf16 [num_pages, page_size, 576]; row r of page p at
 *            kv_pages + p*kv_stride_page + r*kv_stride_row.
 * page_size  a power of two, 1..4096.
 * page_table int32 [num_seqs, max_pages_per_seq]; (b,s) at page_table + b*page_table_stride + s.
 * seq_lens   int32 [num_seqs]: tokens held in the cache for each sequence.
 * indices    int32 [num_tokens, topk] logical positions p within the token's
 *            sequence. p maps to row p % page_size of page
 *            page_table[b, p / page_size]. The entry is skipped when p < 0,
 *            p >= seq_lens[b], p / page_size >= max_pages_per_seq, or the
 *            page id is outside [0, num_pages).
 * Other arguments as in dsa_sparse_mla_fwd. Limits as there, with
 * num_pages * kv_stride_page * 2 bytes < 64 GiB.
 */
int dsa_sparse_mla_fwd_paged(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                             const void* kv_pages, int64_t kv_stride_page, int64_t kv_stride_row,
                             int64_t num_pages, int32_t page_size,
                             const int32_t* page_table, int64_t page_table_stride,
                             int32_t max_pages_per_seq, const int32_t* seq_lens,
                             const int32_t* indices, int64_t idx_stride_tok,
                             int32_t num_seqs, int32_t q_per_seq, int32_t num_heads,
                             int32_t topk, float sm_scale,
                             void* out, int64_t out_stride_tok, int64_t out_stride_head,
                             float* lse, int64_t lse_stride_tok,
                             int32_t num_splits, void* workspace, int64_t workspace_bytes,
                             void* stream);

/*
 * Sparse MLA forward over a paged FP8 MLA KV cache (decode), with no gather
 * copy: the rows are dequantised on the way into the kernel's LDS tiles.
 * Pages: "feat: add XTuner TileLang sparse MLA backend" (lmdeploy PR 4904),
 * Summary (that backend rejects the FP8 MLA KV-cache path) and per-file
 * overview (BF16 and FP8 sparse decode behaviour; the DeepSeek-V3.2
 * configuration defaults the DSA MLA cache to BF16 with an FP8 policy
 * possible elsewhere). The pages do not lay out an FP8 row; the layout taken
 * here is the published DeepSeek-V3.2 sparse-attention FP8 cache row:
 *
 *   bytes   0 .. 511  512 latent values, float8 e4m3 (OCP: bias 7, no
 *                     infinities, S.1111.111 is NaN), in 4 groups of 128;
 *   bytes 512 .. 527  4 float32 scales, one per group;
 *   bytes 528 .. 655  64 rope values, bfloat16.
 *
 * A key's row is latent[g*128 + i] = e4m3 * scale[g], rope as stored; the
 * result is the BF16 paged forward on those rows, except that each latent
 * value is rounded to bf16 (round to nearest even) after the scaling, as the
 * kernel's MFMA operands are bf16.
 *
 * kv_pages   uint8 [num_pages, page_size, >= 656]: row r of page p at byte
 *            p*kv_stride_page_bytes + r*kv_stride_row_bytes (16-byte aligned,
 *            strides multiples of 16).
 * Other arguments, limits and results as in dsa_sparse_mla_fwd_paged, with
 * num_heads <= 32 (DSA_ERR_UNSUPPORTED above).
 */
#define DSA_FP8_ROW_BYTES 656
int dsa_sparse_mla_fwd_paged_fp8(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                 const void* kv_pages, int64_t kv_stride_page_bytes,
                                 int64_t kv_stride_row_bytes, int64_t num_pages, int32_t page_size,
                                 const int32_t* page_table, int64_t page_table_stride,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens,
                                 const int32_t* indices, int64_t idx_stride_tok,
                                 int32_t num_seqs, int32_t q_per_seq, int32_t num_heads,
                                 int32_t topk, float sm_scale,
                                 void* out, int64_t out_stride_tok, int64_t out_stride_head,
                                 float* lse, int64_t lse_stride_tok,
                                 int32_t num_splits, void* workspace, int64_t workspace_bytes,
                                 void* stream);

/*
 * dsa_sparse_mla_fwd_paged without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, and harnesses that forbid allocation. The split partials go to a
 * scratch array of DSA_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on (from the module's load until the process ends); the call
 * itself allocates nothing.
 *
 * Arguments, limits and results are those of dsa_sparse_mla_fwd_paged,
 * without workspace/workspace_bytes. A call whose split partials
 * (num_seqs * q_per_seq * splits * num_heads * 2056 bytes, splits as the
 * workspace query reports) exceed DSA_NOALLOC_SCRATCH_BYTES returns
 * DSA_ERR_WORKSPACE and launches nothing; num_splits = 1 needs no scratch.
 * Every slot of the array that a call reads is written earlier in the same
 * call, so nothing needs clearing between calls. All calls on one GPU share
 * that GPU's array: calls that may overlap in time on one GPU (different
 * streams without ordering, or several host threads) race on it and must be
 * serialised by the caller.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (32 << 20)
int dsa_sparse_mla_fwd_paged_noalloc(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                     const void* kv_pages, int64_t kv_stride_page, int64_t kv_stride_row,
                                     int64_t num_pages, int32_t page_size,
                                     const int32_t* page_table, int64_t page_table_stride,
                                     int32_t max_pages_per_seq, const int32_t* seq_lens,
                                     const int32_t* indices, int64_t idx_stride_tok,
                                     int32_t num_seqs, int32_t q_per_seq, int32_t num_heads,
                                     int32_t topk, float sm_scale,
                                     void* out, int64_t out_stride_tok, int64_t out_stride_head,
                                     float* lse, int64_t lse_stride_tok,
                                     int32_t num_splits, void* stream);

/*
 * Sparse MLA backward over a flat KV array: the gradients of the forward's
 * output O with respect to q and kv, for an upstream gradient dout.
 * Pages: xtuner PR 2083, Motivation (the forward's output and LSE feed the
 * backward that the page keeps); the prime-rl pull request 4078 that adds a
 * `cudnn_flashmla` DSA backend (a separate DSA backward kernel, timed per
 * call). LSE is taken as an auxiliary output with no upstream gradient.
 *
 * With J the valid entries of token t's row, P the forward's softmax weights
 * (recomputed from q, kv and lse), dP = dout . V^T, D = dout . out and
 * dS = P (dP - D), per head:
 *   dq[t]          = sm_scale * dS . K
 *   dkv[J]        += sm_scale * dS^T . q[t]     (all 576 columns)
 *   dkv[J, 0:512] += P^T . dout[t]               (the value columns)
 * Rows that no valid entry names get 0. Duplicates count once per occurrence.
 *
 * q, kv, indices, num_tokens, num_heads, topk, sm_scale: as in dsa_sparse_mla_fwd
 *          (any topk up to 65536; the call does not split rows).
 * out      bf16 [num_tokens, num_heads, 512]: the forward output for these inputs.
 * lse      fp32 [num_tokens, num_heads]: the forward LSE for these inputs.
 * dout     bf16 [num_tokens, num_heads, 512], strides as for out.
 * dq       fp32 [num_tokens, num_heads, 576] (written); element (t,h,d) at
 *          dq + t*dq_stride_tok + h*dq_stride_head + d.
 * dkv      fp32 [num_kv, 576] (written: zeroed, then accumulated with atomic
 *          adds of partial sums, so the order of additions into a row is not
 *          fixed and two calls may differ in the last bits); row i at
 *          dkv + i*dkv_stride_row.
 *          16-byte aligned, dkv_stride_row a multiple of 4 and >= 576.
 * stream   hipStream_t to enqueue on.
 *
 * Three schedules, chosen from the sizes alone (dsa_sparse_mla_bwd_workspace_size
 * reports which one a call takes). Token-major: one workgroup per token and
 * head block adds each named row's gradient into dkv; it needs no workspace.
 * The other two serve rows that name a large share of kv (as in causal
 * prefill), when 0 < num_kv <= 262144:
 *   kv-major (num_heads <= 16 and 3 * num_kv * num_heads <= 256 * topk,
 *     workspace at most 1 GiB): one workgroup per (64 kv rows, 64-token
 *     chunk) keeps the rows' dkv in registers and adds dq with atomics
 *     instead, so dq too may then differ in the last bits between calls;
 *   split (num_heads > 16 and num_kv <= 16 * topk, workspace at most
 *     64 GiB): a token-major pass computes and writes dq (no atomics on dq)
 *     and stores P and s*dS of every (token, named row) in the workspace
 *     (topk * num_heads * 4 bytes per token, the bulk of it); a kv-major pass
 *     per (256 kv rows, half of the columns, 64-token chunk) then forms dkv
 *     from them.
 * Tokens whose row names some kv row twice go to the token-major kernel
 * within the same call.
 * workspace/workspace_bytes  device scratch owned by the caller, at least the
 *          size dsa_sparse_mla_bwd_workspace_size reports for these sizes and
 *          256-byte aligned; may be NULL/0 when that size is 0. Its contents
 *          on entry do not matter; calls that share one workspace must be
 *          stream-ordered. A smaller or misaligned workspace returns
 *          DSA_ERR_WORKSPACE (the call never allocates and never changes
 *          schedule because of the workspace).
 * Limits: 1 <= num_heads <= 128, 1 <= topk <= 65536. dq, dkv and the
 * workspace must not overlap the inputs or each other (checked on the host:
 * DSA_ERR_INVALID_ARGUMENT).
 */
int dsa_sparse_mla_bwd(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                       const void* kv, int64_t kv_stride_row, int64_t num_kv,
                       const int32_t* indices, int64_t idx_stride_tok,
                       int64_t num_tokens, int32_t num_heads, int32_t topk, float sm_scale,
                       const void* out, int64_t out_stride_tok, int64_t out_stride_head,
                       const float* lse, int64_t lse_stride_tok,
                       const void* dout, int64_t dout_stride_tok, int64_t dout_stride_head,
                       float* dq, int64_t dq_stride_tok, int64_t dq_stride_head,
                       float* dkv, int64_t dkv_stride_row,
                       void* workspace, int64_t workspace_bytes,
                       void* stream);

/* Backward schedules reported by dsa_sparse_mla_bwd_workspace_size. */
#define DSA_BWD_TOKEN_MAJOR 0
#define DSA_BWD_KV_MAJOR 1
#define DSA_BWD_SPLIT 2

/*
 * Workspace query for dsa_sparse_mla_bwd. The pages that motivate it: the
 * prime-rl pull request 4078 that adds a `cudnn_flashmla` DSA backend
 * describes a backward that always failed because it did not provide the
 * workspace its kernel required; here the caller learns the size up front.
 *
 * num_tokens, num_heads, num_kv, topk: as in the backward call.
 * *schedule_out (may be NULL): DSA_BWD_TOKEN_MAJOR, DSA_BWD_KV_MAJOR or
 *   DSA_BWD_SPLIT, the schedule a backward call with these sizes takes (on
 *   any device).
 * *bytes_out: workspace bytes that call needs (0 for the token-major schedule).
 * Returns DSA_OK, DSA_ERR_INVALID_ARGUMENT (negative sizes, NULL bytes_out) or
 * DSA_ERR_UNSUPPORTED (num_heads or topk out of range).
 */
int dsa_sparse_mla_bwd_workspace_size(int64_t num_tokens, int32_t num_heads, int64_t num_kv,
                                      int32_t topk, int32_t* schedule_out, int64_t* bytes_out);

/*
 * Top-k index selection: turns each query token's row of indexer scores into
 * the -1-padded index row that the sparse forward consumes.
 * Pages: "feat: add XTuner TileLang sparse MLA backend" (lmdeploy PR 4904),
 * Summary (DSA index production kept for short prefill) and per-file overview
 * (prefill scores computed over chunks of query rows; the short-prefill
 * scoring skip); Validation (-1-padded index rows); "[Feature] Add optional
 * FlashMLA backend for DSA Sparse MLA" (xtuner PR 2083), Changes (an indexer
 * in front of the sparse kernel). The score function is the caller's.
 *
 * scores     fp32 [num_tokens, num_cols]; (t, j) at scores + t*score_stride_tok + j.
 *            May be NULL when no row has more than topk candidates (then no
 *            score is read; see below).
 * key_start, key_end  int32 [num_tokens]: token t's candidates are columns
 *            key_start[t] <= j < key_end[t], clipped to [0, num_cols); an
 *            empty range selects nothing. Packed causal prefill: the token's
 *            document start and its own row + 1 (column = global kv row);
 *            decode: 0 and the context length (column = logical position).
 * indices    int32 [num_tokens, topk] (written); row t at indices + t*idx_stride_tok.
 *
 * Row t holds the selected column ids in ascending order, then -1:
 *   - at most topk candidates: all of them, and the row's scores are never
 *     read (the short-prefill skip: such rows need no scoring at all);
 *   - otherwise the topk candidates first in this order: larger score; for
 *     equal scores (-0 equals +0) the smaller column; NaN after every number
 *     (NaNs among themselves by column).
 *   - with scores NULL a row of more than topk candidates selects nothing.
 * The result is exact and deterministic (integer work, no tolerance).
 *
 * Limits: 1 <= topk <= 65536, num_cols <= 2^31 - 1, num_tokens < 2^31.
 * indices must not overlap scores, key_start or key_end (DSA_ERR_INVALID_ARGUMENT).
 */
int dsa_topk_indices(const float* scores, int64_t score_stride_tok, int64_t num_cols,
                     const int32_t* key_start, const int32_t* key_end,
                     int64_t num_tokens, int32_t topk,
                     int32_t* indices, int64_t idx_stride_tok,
                     void* stream);

/* Human-readable name of a dsa_status value (a static string). The status
 * codes carry the explicit rejections of unsupported paths that
 * "feat: add XTuner TileLang sparse MLA backend" (lmdeploy PR 4904), Summary,
 * describes. */
const char* dsa_status_string(int status);

/* 1 if HIP device `device` is a gfx950 (MI355X class) GPU, 0 if not or on error.
 * The runtime availability check that "[Feature] Add optional FlashMLA backend
 * for DSA Sparse MLA" (xtuner PR 2083), Changes, performs before selecting its
 * backend; here every entry point also returns DSA_ERR_UNSUPPORTED on other
 * devices. */
int dsa_device_supported(int device);

/* Library version as major*10000 + minor*100 + patch. */
int dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_SPARSE_MLA_H */
