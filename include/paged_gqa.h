/*
 * paged_gqa.h -- C ABI of a gfx950 (MI355X) library for paged grouped-query
 * attention with head_dim 256 over a block-table-indexed KV cache.
 *
 * Three attention calls, one per problem on the source pages:
 *   paged_attn_verify          short multi-token speculative-verify queries
 *                              (SGLang PR #36330, "... MTP unified attention on
 *                              gfx950": Motivation, Modifications)
 *   paged_attn_prefill_prefix  new tokens against a cached prefix with
 *                              bottom-right causal masking (ROCm/ATOM PR #2534,
 *                              "asm FP8 FMHA for prefix-hit prefill ...": the
 *                              FMHA commit message and Summary)
 *   sparse_paged_attn          each query row attends only its own list of
 *                              selected tokens (vLLM PR #62590, "Tune sparse GQA
 *                              prefill profile on gfx942 and gfx950": Overview,
 *                              Earlier results)
 * and the step ahead of the FP8 prefill:
 *   prefill_quantize_fp8       per-tensor FP8 quantisation of Q and of the new
 *                              tokens' keys and values into the page pool
 *                              (ROCm/ATOM PR #2534: the casts to FP8 counted in
 *                              its prefill timings)
 *
 * What every attention call computes, for sequence b, query token t (0 <= t < Lq_b) and
 * query head h, with r = num_q_heads / num_kv_heads and g = h / r:
 *   s_j  = softmax_scale * q_descale * k_descale * <q[t,h,:], K_j[g,:]>
 *   out  = v_descale * sum_j softmax(s)_j * V_j[g,:]       (bf16, RNE)
 *   lse  = ln sum_j exp(s_j)                                (fp32, optional)
 * over the visible keys j: 0 <= j <= Lk_b - Lq_b + t (verify, prefill), or the
 * entries of the row's index list that lie in [0, Lk_b) (sparse).  Lk_b counts
 * the sequence's new tokens, so its last query token sees all Lk_b keys.  A row
 * with no visible key gets out = 0 and lse = -inf.
 *
 * Memory.  Every pointer except `kv` (a host struct) is device memory owned by
 * the caller; nothing is allocated, freed or retained by the library.  Q and
 * out are row-major [T, num_q_heads, 256] with T = cu_seqlens_q[num_seqs]; lse
 * is [T, num_q_heads].  Logical key j of sequence b lives in pool page
 * block_table[b * block_table_stride + j / page_size], slot j % page_size; the
 * element offset of (page, slot, kv head, d) is
 *   page * stride_page + slot * stride_token + head * stride_head + d
 * (strides in elements, d unit-stride), which covers [pages, slots, heads, d]
 * and [pages, heads, slots, d] pools alike (ROCm/ATOM PR #2830, summary
 * paragraph: the block-table stride is a runtime argument).
 *
 * Numbers.  BF16 or OCP FP8 E4M3FN codes; real value = code * descale.  The
 * descales are per-tensor fp32 scalars in device memory (NULL means 1.0).
 *
 * Errors.  Every host-checkable condition is checked before anything is
 * launched; on error the call returns a nonzero PGA_ERR_* code, launches
 * nothing and leaves `out`, `lse` and the workspace untouched.  Device data is
 * not validated (that would need a synchronisation): block-table entries
 * outside [0, num_pages) are never dereferenced, but the result for a sequence
 * that has one is undefined.  There is no silent fallback path.
 *
 * Threading.  Calls are asynchronous on `stream` (a hipStream_t; NULL is the
 * default stream), hold no global mutable state and may run concurrently on
 * different streams, provided their workspaces do not overlap.
 */
#ifndef PAGED_GQA_H_
#define PAGED_GQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PGA_ABI_VERSION 4
#define PGA_HEAD_DIM 256
/* Bytes of the fixed per-device scratch of paged_attn_verify_noalloc (128 MiB). */
#define PGA_VERIFY_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* Element encodings. */
enum pga_dtype {
  PGA_DTYPE_BF16 = 1,     /* bfloat16 */
  PGA_DTYPE_FP8_E4M3 = 2  /* OCP FP8 E4M3FN (no infinities, max 448) */
};

/* Status codes. */
enum pga_status {
  PGA_OK = 0,
  PGA_ERR_NULL = 1,        /* a required pointer is NULL */
  PGA_ERR_SHAPE = 2,       /* head_dim != 256, Hq % Hkv != 0, negative sizes, q-length envelope */
  PGA_ERR_DTYPE = 3,       /* unsupported dtype or q/kv dtype pair */
  PGA_ERR_UNSUPPORTED = 4, /* outside the kernel envelope: page size, alignment, rows per group */
  PGA_ERR_WORKSPACE = 5,   /* workspace smaller than the matching *_workspace_bytes() */
  PGA_ERR_LAUNCH = 6,      /* the HIP runtime refused a launch (or a copy / synchronisation failed) */
  PGA_ERR_INVALID_DATA = 7, /* pga_validate_inputs found device data that breaks a precondition */
  PGA_ERR_SCRATCH = 8       /* paged_attn_verify_noalloc: the call needs more than its fixed scratch */
};

/* The paged KV cache.  K and V share dtype, head count and page size; their
 * strides may differ.  All strides are in elements and must be multiples of
 * 16 bytes' worth of elements; k_cache and v_cache must be 16-byte aligned. */
typedef struct pga_paged_kv {
  const void* k_cache;
  const void* v_cache;
  int32_t dtype;              /* enum pga_dtype */
  int32_t num_kv_heads;       /* >= 1 */
  int32_t head_dim;           /* must be 256 */
  int32_t page_size;          /* tokens per page: a power of two, 16..1024 */
  int32_t num_pages;          /* pages in the pool; entries outside [0, num_pages) are never read */
  int32_t reserved;           /* set to 0 */
  int64_t k_stride_page, k_stride_token, k_stride_head;  /* elements; multiples of 16 bytes; */
  int64_t v_stride_page, v_stride_token, v_stride_head;  /* page_size * stride_token < 2 GiB */
  const int32_t* block_table; /* [num_seqs, block_table_stride] physical page ids */
  int64_t block_table_stride; /* >= ceil(max KV length / page_size) */
  const float* k_descale;     /* device scalar or NULL (1.0) */
  const float* v_descale;     /* device scalar or NULL (1.0) */
} pga_paged_kv;

/*
 * Speculative-verify attention: 1..4 query tokens per sequence against that
 * sequence's whole KV history (SGLang PR #36330, Motivation: short multi-token
 * queries, 16 query heads per KV head, head size 256, page size 16, FP8 KV).
 * All r * Lq_b query rows of one KV group are packed into one tile, so each KV
 * page is loaded once for every speculative token of the group
 * (Modifications: BLOCK_M = 16 x BLOCK_Q).  Long histories are split KV-wise
 * and the fp32 partial results are merged by a separate log-sum-exp kernel
 * (Modifications: 8-64 segments).  The split here is balanced rather than
 * fixed: a fixed set of persistent workgroups takes equal shares of the list
 * of (sequence, kv head, 64-key tile) work, so a history is cut where those
 * shares end, and additionally into segments of at most kv_split_tokens keys
 * when that is set.  Small calls (num_seqs * num_kv_heads * ceil(max_kv_len /
 * 64) <= 256 tiles, at most 64 per history) skip that plan: one workgroup per
 * 64-key tile, its partial rows merged the same way (kv_split_tokens then
 * changes nothing, every piece being one tile).
 *
 *   q             [T, num_q_heads, 256] bf16 (q_dtype must be PGA_DTYPE_BF16)
 *   q_descale     device scalar or NULL; used as a factor on the scores
 *   cu_seqlens_q  [num_seqs + 1] int32, non-decreasing, cu_seqlens_q[0] = 0
 *   seq_lens_k    [num_seqs] int32, Lk_b >= Lq_b, including the new tokens
 *   max_q_len     host upper bound of Lq_b, 1..4; (Hq / Hkv) * max_q_len <= 64
 *   max_kv_len    host upper bound of Lk_b
 *   kv_split_tokens  0 = no segment cap (cuts only where the balanced
 *                 shares end); otherwise the longest piece of one history
 *                 that one workgroup attends, a positive multiple of 64
 *   workspace     device buffer of at least paged_attn_verify_workspace_bytes()
 *                 bytes, 256-byte aligned; holds the partial rows (fp16 for
 *                 FP8 V, fp32 for BF16 V) and their lse values between the
 *                 two stages; caller-owned, its contents on entry do not
 *                 matter
 *   out           [T, num_q_heads, 256] bf16;  lse  [T, num_q_heads] fp32 or NULL
 * Returns PGA_OK or a PGA_ERR_* code.
 */
int paged_attn_verify(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                      int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                      int32_t max_q_len, int32_t max_kv_len, const pga_paged_kv* kv, float softmax_scale,
                      int32_t kv_split_tokens, void* workspace, size_t workspace_bytes, void* out, float* lse,
                      void* stream);

/* The two stages of paged_attn_verify, callable on their own with the same
 * arguments: the attention kernel over every (segment, kv head, sequence),
 * which writes the final output of single-segment sequences and fp32 partial
 * outputs plus lse values to the workspace for the others; then the
 * log-sum-exp merge of those partials.  paged_attn_verify is exactly stage 1
 * followed by stage 2 on the same stream.  A caller that shards a sequence's
 * segments across devices can gather the workspace partials and run stage 2. */
int paged_attn_verify_partials(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                               int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                               int32_t max_q_len, int32_t max_kv_len, const pga_paged_kv* kv, float softmax_scale,
                               int32_t kv_split_tokens, void* workspace, size_t workspace_bytes, void* out,
                               float* lse, void* stream);
int paged_attn_verify_merge(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                            int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                            int32_t max_q_len, int32_t max_kv_len, const pga_paged_kv* kv, float softmax_scale,
                            int32_t kv_split_tokens, void* workspace, size_t workspace_bytes, void* out,
                            float* lse, void* stream);

/*
 * paged_attn_verify without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It runs the same two kernels as
 * paged_attn_verify (same arguments and result) with the partial rows, their
 * lse values and the merge plan in a fixed scratch array of
 * PGA_VERIFY_NOALLOC_SCRATCH_BYTES that each device the library runs on holds
 * from the first such call until the process ends.  The call allocates and
 * frees nothing.  The scratch holds, for units = num_seqs * num_kv_heads,
 * segs = ceil(ceil(max_kv_len / 64) / (kv_split_tokens / 64)) (1 when
 * kv_split_tokens is 0), slots = units * segs + the grid (at most 2
 * workgroups per compute unit; units * ceil(max_kv_len / 64) for the small
 * calls above) and rows = (num_q_heads / num_kv_heads) *
 * max_q_len: slots * rows * 256 partial values (2 bytes each for FP8 V, 4 for
 * BF16 V) plus slots * rows lse values; a call whose bounds need more returns
 * PGA_ERR_SCRATCH and launches nothing.  Nothing in the scratch needs to
 * start at zero: every value the merge reads is written earlier in the same
 * call.  All calls on one device share that device's scratch, so two calls
 * that may overlap in time on one device (different streams, different host
 * threads) race: serialise them.  Returns PGA_OK or a PGA_ERR_* code
 * (PGA_ERR_LAUNCH also when the scratch's device address cannot be looked up).
 */
int paged_attn_verify_noalloc(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                              int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                              int32_t max_q_len, int32_t max_kv_len, const pga_paged_kv* kv, float softmax_scale,
                              int32_t kv_split_tokens, void* out, float* lse, void* stream);

/*
 * Measurement helper: the page gather of paged_attn_verify alone, the
 * practical bandwidth roof of that call on a given batch (SGLang PR #36330,
 * Motivation: the speculative-verify cost is the KV pages each query group
 * loads).  It runs the verify call's own work split and grid (the same
 * num_seqs, lengths, host bounds, kv and kv_split_tokens give the same pieces
 * and workgroups) and the same 16-byte non-temporal page copies into the same
 * LDS tiles on the same pipeline, in one launch, and only adds up what it
 * copies:
 *   out[b * num_kv_heads + g] += sum over keys j < min(Lk_b, max_kv_len) of
 *     every 32-bit word of K_j and of V_j of kv head g, mod 2^32
 *   (nothing for sequences with no query token), an exact, order-independent
 *   checksum when out starts at zero.
 * The query heads do not change the split, so none are passed.
 *   out  [num_seqs * num_kv_heads] uint32, 4-byte aligned, added into
 * Returns PGA_OK or a PGA_ERR_* code (the argument checks of
 * paged_attn_verify that apply).
 */
int paged_attn_verify_gather_sum(int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                 int32_t max_q_len, int32_t max_kv_len, const pga_paged_kv* kv,
                                 int32_t kv_split_tokens, uint32_t* out, void* stream);

/* Workspace bytes paged_attn_verify needs for these host bounds.  A balanced
 * split can cut any history, so this is > 0 whenever the bounds admit any
 * work; 0 for bounds with no work (no sequences, max_kv_len 0) or invalid
 * bounds. */
size_t paged_attn_verify_workspace_bytes(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                         int32_t max_q_len, int32_t max_kv_len, int32_t kv_split_tokens);

/* Longest piece of one history that one workgroup attends for these host
 * bounds: kv_split_tokens when set, otherwise max_kv_len rounded up to a
 * multiple of 64 (at least 64); 0 for invalid bounds. */
int32_t paged_attn_verify_split_tokens(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                                       int32_t max_q_len, int32_t max_kv_len, int32_t kv_split_tokens);

/*
 * Prefill of new tokens against a cached prefix (ROCm/ATOM PR #2534, FMHA
 * commit message: the cached+new keys are longer than the queries and the
 * causal mask is bottom-right aligned).  Keys are read from the pages in the
 * kernel; no gather to contiguous memory happens first (ROCm/ATOM PR #2830,
 * recipe commit).
 *
 *   q             [T, num_q_heads, 256], FP8 E4M3FN or bf16 (q_dtype)
 *   cu_seqlens_q  [num_seqs + 1] int32 prefix sums of Lq_b
 *   cu_seqlens_k  [num_seqs + 1] int32 prefix sums of Lk_b, Lk_b >= Lq_b
 *   max_seqlen_q, max_seqlen_k  host upper bounds of Lq_b and Lk_b
 *   out           [T, num_q_heads, 256] bf16;  lse  [T, num_q_heads] fp32 or NULL
 * FP8 Q requires FP8 KV.  Returns PGA_OK or a PGA_ERR_* code.
 */
int paged_attn_prefill_prefix(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                              int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t max_seqlen_q, int32_t max_seqlen_k, const pga_paged_kv* kv,
                              float softmax_scale, void* out, float* lse, void* stream);

/*
 * Selected-token attention (vLLM PR #62590, Overview and Earlier results: each
 * query row attends its own list of selected tokens, 2,051 per row at head
 * size 256, BF16 or FP8 K/V).  Row i of q (a token of the sequence given by
 * cu_seqlens_q) attends the logical positions indices[i * index_stride + e],
 * e < num_selected; entries outside [0, Lk_b) are padding and skipped.  One
 * list serves every head of the row; no causal rule is applied beyond it.
 *
 *   q             [num_q_tokens, num_q_heads, 256] bf16
 *   num_q_tokens  host copy of cu_seqlens_q[num_seqs]
 *   seq_lens_k    [num_seqs] int32; block_table_stride must cover each Lk_b
 *   indices       [num_q_tokens, index_stride] int32
 *   num_selected  entries read per row, 0 <= num_selected <= index_stride
 *   workspace     when few rows would leave the GPU idle (the launch profile
 *                 changes with the row count on the page: Overview, Measured
 *                 results), each row's list is cut into
 *                 sparse_paged_attn_splits() pieces, attended by separate
 *                 waves and merged by log-sum-exp; the pieces' rows and lse
 *                 values live in this caller-owned device buffer of at least
 *                 sparse_paged_attn_workspace_bytes() bytes, 256-byte aligned.
 *                 NULL with workspace_bytes 0 asks for the unsplit launch
 *                 (same result); a smaller non-empty buffer is an error.
 *   out           [num_q_tokens, num_q_heads, 256] bf16;  lse  [num_q_tokens, num_q_heads] fp32 or NULL
 * The pool must hold fewer than 2^31 tokens (num_pages * page_size).
 * Returns PGA_OK or a PGA_ERR_* code.
 */
int sparse_paged_attn(const void* q, int32_t q_dtype, const float* q_descale, int32_t num_q_heads,
                      int32_t num_q_tokens, int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                      const int32_t* indices, int64_t index_stride, int32_t num_selected, const pga_paged_kv* kv,
                      float softmax_scale, void* workspace, size_t workspace_bytes, void* out, float* lse,
                      void* stream);

/* Pieces each row's index list is cut into for these host arguments (1: no
 * split, no workspace needed), and the workspace that needs; 0 for invalid
 * arguments. */
int32_t sparse_paged_attn_splits(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_q_tokens,
                                 int32_t num_selected);
size_t sparse_paged_attn_workspace_bytes(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_q_tokens,
                                         int32_t num_selected);

/*
 * Measurement helper, not part of the attention path: the same-index gather
 * of sparse_paged_attn.  For every query row and kv head it copies exactly
 * the K and V rows that the row's valid list entries select (the same
 * index -> block-table page -> pool row translation and the same 16-byte
 * global-to-LDS copies as the attention kernel) and sums their 32-bit words:
 *   out[row][g][w] = sum over valid entries j of (word w of K_j[g] + word w
 *                    of V_j[g]) mod 2^32,  w < 256 * element bytes / 4
 * Its time prices the gather on its own: the practical bandwidth roof of
 * the selected-token call on the same selection (vLLM PR #62590, Measured
 * results: the row counts and selections whose kernel times it reports).
 * Arguments as in sparse_paged_attn; out is uint32 [num_q_tokens,
 * num_kv_heads, 64 (FP8) or 128 (BF16)], 16-byte aligned.  The pool must be
 * evenly spaced (stride_page = page_size * stride_token for K and V), hold at
 * most 2^24 token rows with token strides below 2^24 bytes, and have every
 * row's byte offset from its head's base below 2^32; otherwise
 * PGA_ERR_UNSUPPORTED.
 */
int sparse_gather_sum(int32_t num_q_tokens, int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                      const int32_t* indices, int64_t index_stride, int32_t num_selected, const pga_paged_kv* kv,
                      uint32_t* out, void* stream);

/*
 * Per-tensor FP8 (OCP E4M3FN) quantisation of a prefix-hit prefill's inputs,
 * the step ahead of paged_attn_prefill_prefix with FP8 Q (ROCm/ATOM PR #2534,
 * FMHA commit message and Results: its prefill timings include the casts of
 * Q, K and V to FP8).  The page fixes no scale rule; this call takes the
 * plainest one, in fp32:
 *   descale = fp32(amax / 448), amax = max |x| over the non-NaN elements
 *             (descale 1 when amax is 0)
 *   code    = the E4M3FN value nearest to fp32(x / descale), ties to the even
 *             code; finite values beyond +-448 saturate to +-448, NaN stays NaN
 * Q takes a dynamic descale (or a given one); the new tokens' keys and values
 * take the pool's own descales (kv->k_descale, kv->v_descale; NULL = 1), which
 * the cached prefix in the pool already uses, and are written into the pool
 * at logical position Lk_b - Lq_b + t of their sequence.
 *
 *   q             [num_q_tokens, num_q_heads, 256] bf16, 16-byte aligned
 *                 (q and q_fp8 may be NULL when num_q_tokens is 0)
 *   q_descale_in  device scalar with the descale to use, or NULL for the
 *                 dynamic one
 *   q_fp8         [num_q_tokens, num_q_heads, 256] codes out, 8-byte aligned
 *   q_descale_out device scalar out: the descale used (pass it as q_descale to
 *                 paged_attn_prefill_prefix); may be NULL when q_descale_in is set
 *   k_new, v_new  [num_q_tokens, kv->num_kv_heads, 256] bf16 in the token
 *                 order of cu_seqlens_q, 16-byte aligned; both NULL for Q only
 *   cu_seqlens_q, cu_seqlens_k  [num_seqs + 1] int32 prefix sums of Lq_b and
 *                 Lk_b (needed with k_new / v_new)
 *   kv            the FP8 pool (required with k_new / v_new).  The call WRITES
 *                 the new tokens' rows into kv->k_cache and kv->v_cache; other
 *                 slots are untouched.  A position before its sequence's start
 *                 or on a page id outside [0, num_pages) is not written.
 *   workspace     with the dynamic descale: a device buffer of at least
 *                 prefill_quantize_fp8_workspace_bytes() bytes, 256-byte
 *                 aligned, any contents (per-workgroup maxima, tagged with a
 *                 value unique to the call); otherwise unused.  Calls that may
 *                 run at the same time need workspaces of their own.
 * With the dynamic descale, a 16-byte aligned q_fp8 and Q of at most
 * 16 x 1024 x (CU count) 16-byte chunks (64 MiB on 256 CUs): one launch of one
 * workgroup per CU, each holding its share of Q in registers across a grid
 * barrier, so Q is read once.  The grid must be resident at once: on a stream
 * that may use fewer CUs the barrier's bounded wait expires (after more than
 * 0.2 s) and the codes of the workgroups that waited come out NaN.  Otherwise
 * two launches (a max-magnitude reduction over Q, then the coding pass, which
 * reads Q again).  With a given descale: one launch.  Returns PGA_OK or a
 * PGA_ERR_* code.
 */
int prefill_quantize_fp8(const void* q, int32_t num_q_heads, int32_t num_q_tokens, const float* q_descale_in,
                         void* q_fp8, float* q_descale_out, const void* k_new, const void* v_new, int32_t num_seqs,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const pga_paged_kv* kv,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes prefill_quantize_fp8 needs with the dynamic descale. */
size_t prefill_quantize_fp8_workspace_bytes(void);

/*
 * Checks the data-dependent preconditions that the calls above leave
 * unchecked because checking them would need a synchronisation (SGLang PR
 * #36330, review notes: a dispatch gate and a kernel assertion that disagree
 * are the failure the explicit checks here and there guard against).  For
 * tests and debugging, not for the hot path: it launches small kernels on `stream` and then
 * synchronises the stream.  Every device read stays inside the extents the
 * host arguments give, whatever the device data hold.
 *
 *   num_seqs, cu_seqlens_q  as in the attention calls
 *   num_q_tokens  host copy of cu_seqlens_q[num_seqs], or -1 when unknown
 *                 (required, >= 0, with indices)
 *   seq_lens_k, cu_seqlens_k  exactly one of them (verify and sparse take
 *                 seq_lens_k, prefill cu_seqlens_k)
 *   max_q_len, max_kv_len  the host bounds the caller passes to the call
 *                 (<= 0: not checked)
 *   kv            the pool: block_table, block_table_stride, page_size and
 *                 num_pages are read
 *   indices, index_stride, num_selected  sparse lists, or indices NULL
 *   counts_device device int32[4] scratch, overwritten
 *   counts_host   host int32[4] out, or NULL:
 *     [0] sequences with invalid lengths (cu_seqlens_q not starting at 0 or
 *         decreasing, Lk_b < Lq_b, cu_seqlens_q[num_seqs] != num_q_tokens)
 *     [1] sequences beyond the host bounds, or needing more block-table
 *         columns than block_table_stride
 *     [2] block-table entries, among those the keys 0 .. Lk_b - 1 map to,
 *         outside [0, num_pages)
 *     [3] index entries at or past their sequence's Lk_b (the sparse call
 *         skips them like padding; reported, not an error)
 * Returns PGA_OK when counts [0] .. [2] are zero, PGA_ERR_INVALID_DATA when
 * not, or another PGA_ERR_* code for invalid host arguments.
 */
int pga_validate_inputs(int32_t num_seqs, int32_t num_q_tokens, const int32_t* cu_seqlens_q,
                        const int32_t* seq_lens_k, const int32_t* cu_seqlens_k, int32_t max_q_len,
                        int32_t max_kv_len, const pga_paged_kv* kv, const int32_t* indices, int64_t index_stride,
                        int32_t num_selected, int32_t* counts_device, int32_t* counts_host, void* stream);

/* Human-readable text of a status code (static storage). */
const char* pga_status_string(int status);

/* PGA_ABI_VERSION of the loaded library. */
int pga_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_GQA_H_ */
