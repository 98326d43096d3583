/*
 * fa.h - C ABI of an exact tiled attention library for AMD MI355X (gfx950).
 *
 * Three operations, each exact up to floating-point reordering:
 *
 *   fa_forward         tiled attention forward with an online softmax and
 *                      causal tile skipping ("3.4 Attention Kernels",
 *                      section "FlashAttention: tiling"; "FlashAttention and
 *                      Optimized Kernels", section "The online softmax").
 *   fa_forward_paged   ragged query batches (prefill chunks and decode tokens of
 *                      many sequences) over a paged KV cache (section "Paged
 *                      and ragged layouts: FlashInfer").
 *   fa_cascade         the same for sequences sharing one prefix, whose
 *                      attention is computed once for all queries and merged
 *                      with each sequence's own suffix (cascade attention,
 *                      same section).
 *   fa_decode_paged    one query token per sequence against a paged, ragged
 *                      KV cache, the keys split into chunks whose partial
 *                      results are merged ("3.4 Attention Kernels", sections
 *                      "Decode attention and Flash-Decoding" and "Paged and
 *                      ragged layouts: FlashInfer").
 *   fa_decode_paged_ex the same with a sliding window and logit soft-capping
 *                      (section "Paged and ragged layouts: FlashInfer").
 *   fa_decode_graph_*  a decode step recorded once as a HIP graph and replayed
 *                      with one launch ("3.4 Attention Kernels", section
 *                      "Kernel launch overhead and CUDA graphs").
 *   fa_merge_partials  the merge of partial results computed on disjoint key
 *                      sets ("3.4 Attention Kernels", section "Online softmax",
 *                      last paragraph).
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library keeps no pointer after the call returns and allocates nothing.
 *   - Tensors are dense and contiguous in the layouts stated per call. The
 *     Q, K, V, O, q and K/V pool pointers must be 16-byte aligned device
 *     addresses below 2^48, the GPU's virtual address space (else
 *     FA_ERR_BAD_ARG); the kernels move them in 16-byte vectors and address
 *     K/V through buffer resources, whose base field holds 48 bits.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; outputs are valid once the
 *     stream has been synchronised. Apart from the one scratch buffer of
 *     fa_decode_paged_noalloc, the library holds no global mutable state, so
 *     calls on different streams may run concurrently provided their output
 *     buffers do not overlap.
 *   - Every argument is validated on the host BEFORE anything is launched.
 *     A call that returns an error status has enqueued no work and has not
 *     touched any buffer. Sizes whose launch would exceed HIP's limit of
 *     2^32 - 1 threads along a grid dimension return FA_ERR_BAD_SHAPE. FA_ERR_HIP reports a failed launch
 *     (hipGetLastError after the launch); no C++ exception crosses the ABI.
 *   - Softmax scale is explicit. LSE is the natural-log log-sum-exp of the
 *     scaled scores over the visible keys, m + ln(l) ("3.4 Attention
 *     Kernels", section "FlashAttention: tiling"). A query with no visible
 *     key gets O = 0 and LSE = -inf.
 *   - Grouped-query heads: query head h reads KV head h / (H / Hkv).
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_PTR = 1,    /* a required pointer is NULL                     */
  FA_ERR_BAD_SHAPE = 2,   /* a size is negative, inconsistent or too large  */
  FA_ERR_UNSUPPORTED = 3, /* valid but not implemented (head dim, dtype...) */
  FA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required        */
  FA_ERR_HIP = 5,         /* the HIP runtime reported a launch failure      */
  FA_ERR_BAD_ARG = 6,     /* a non-size argument is out of range            */
  FA_ERR_SCRATCH = 7      /* more partials than the fixed scratch buffer    */
} fa_status;

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

/* Largest number of key splits per sequence fa_decode_paged uses. */
#define FA_MAX_SPLITS 64
/* Token slots per KV page accepted by fa_decode_paged. */
#define FA_PAGE_SIZE 16
/* Largest number of key ranges fa_cascade splits the shared prefix into. */
#define FA_CASCADE_MAX_SPLITS 64

/*
 * fa_forward - exact attention forward for dense batched tensors.
 *
 * For every batch b, query head h and query row i:
 *   s_ij = scale * Q[b,i,h,:] . K[b,j,h/(H/Hkv),:]
 *   O[b,i,h,:] = sum_j softmax_j(s_ij) V[b,j,h/(H/Hkv),:],  LSE[b,h,i] = ln sum_j e^s_ij
 * over the visible keys j ("3.4 Attention Kernels", sections "Naive attention
 * and its memory traffic" and "FlashAttention: tiling"). With causal != 0 key
 * j is visible to query i iff j <= i + (Nk - Nq): the causal diagonal is
 * aligned to the bottom-right corner, as in the page's naive_attention code,
 * which equals the usual alignment when Nq == Nk. Key tiles that lie wholly
 * above the diagonal are never read (the causal tile skipping of section
 * "FlashAttention: tiling").
 *
 * Layouts (row-major, contiguous):
 *   Q   [B, Nq, H,   d]  in_dtype
 *   K,V [B, Nk, Hkv, d]  in_dtype
 *   O   [B, Nq, H,   d]  out_dtype (in_dtype, or FA_F32)
 *   LSE [B, H, Nq]       float
 * Arithmetic: bf16/fp16 inputs multiply on the matrix cores with fp32
 * accumulation; the probabilities are rounded to the input type for the P V
 * product. fp32 inputs use fp32 throughout. Outputs are rounded to nearest
 * even once, at the store.
 *
 * Supported: d in {64, 128}; in_dtype in {FA_F32, FA_F16, FA_BF16};
 * out_dtype == in_dtype or FA_F32; B, Nq, Nk >= 0; H, Hkv >= 1, H % Hkv == 0;
 * every tensor below 2^31 elements. B == 0 or Nq == 0 is a no-op. Nk == 0
 * writes O = 0 and LSE = -inf. Q, O, LSE (and K, V when Nk > 0) must be
 * non-NULL; scale must be finite and positive (else FA_ERR_BAD_ARG).
 */
fa_status fa_forward(const void* Q, const void* K, const void* V, void* O,
                     float* LSE, int B, int H, int Hkv, int Nq, int Nk, int d,
                     float scale, int causal, fa_dtype in_dtype,
                     fa_dtype out_dtype, void* stream);

/*
 * fa_forward_paged - exact attention for ragged query batches over a paged
 * KV cache: prefill chunks and decode tokens of many sequences in one call.
 *
 * "3.4 Attention Kernels", section "Paged and ragged layouts: FlashInfer":
 * the tokens of all sequences are concatenated without padding and an
 * offsets array (indptr) marks where each sequence starts; the K/V of each
 * sequence live in pages found through its block table. Sequence b owns
 * query rows qo_indptr[b] .. qo_indptr[b+1]-1 of Q and O (q_len_b rows) and
 * kv_lens[b] cached tokens, token t in page block_table[b*max_pages_per_seq +
 * t / page_size] at slot t % page_size. Its queries are its NEWEST q_len_b
 * positions: with causal != 0, its query i (0-based within the sequence)
 * sees key j iff j <= i + kv_lens[b] - q_len_b (bottom-right alignment, as
 * fa_forward); a decode step is simply q_len_b = 1. Otherwise as fa_forward:
 * the same arithmetic, scale, GQA mapping and outputs per (row, head).
 * Sequences with exactly one query row are computed as fa_decode_paged
 * computes a sequence with one chunk, by the decode kernel's page streaming
 * (one workgroup per sequence and KV head, in a launch of their own before
 * the other rows'); their results agree with the tiled kernel's to the
 * stated tolerance, not bit for bit. This applies when H / Hkv <= 16.
 *
 * Layouts (row-major, contiguous):
 *   Q            [total_q, H, d]                      dtype
 *   qo_indptr    [B + 1]                  int32       device memory
 *   K_pool,V_pool[num_pages, page_size, Hkv, d]       dtype
 *   block_table  [B, max_pages_per_seq]   int32       device memory
 *   kv_lens      [B]                      int32       device memory
 *   O            [total_q, H, d]                      out_dtype (dtype or FA_F32)
 *   LSE          [total_q, H]             float
 *
 * Supported: dtype in {FA_F16, FA_BF16}; d in {64, 128}; page_size ==
 * FA_PAGE_SIZE; H % Hkv == 0. max_q_len is an upper bound of every q_len_b
 * (it sizes the launch); B == 0, total_q == 0 or max_q_len == 0 is a no-op.
 * Rows of Q/O that belong to no sequence are not touched.
 * Device-side contract (not checkable on the host without a sync):
 * 0 <= qo_indptr[b] <= qo_indptr[b+1] <= total_q; q_len_b <= max_q_len;
 * 0 <= kv_lens[b] <= max_pages_per_seq * page_size; used table entries lie
 * in [0, num_pages). A sequence with broken indptr entries is skipped (its
 * rows are unknown); any other violation sets that sequence's O and LSE to
 * NaN (rows beyond max_q_len may be left unwritten). Nothing is read out of
 * bounds.
 */
fa_status fa_forward_paged(const void* Q, const int32_t* qo_indptr,
                           const void* K_pool, const void* V_pool,
                           const int32_t* block_table, const int32_t* kv_lens,
                           void* O, float* LSE, int B, int H, int Hkv, int d,
                           int total_q, int max_q_len, int page_size,
                           int max_pages_per_seq, int num_pages, float scale,
                           int causal, fa_dtype dtype, fa_dtype out_dtype,
                           void* stream);

/*
 * fa_cascade - fa_forward_paged for sequences that all start with one shared
 * prefix, with the prefix's attention computed once for every query.
 *
 * "3.4 Attention Kernels", section "Paged and ragged layouts: FlashInfer"
 * (cascade attention): the keys that many sequences have in common are
 * scored once against every query of those sequences, and that partial result
 * is then combined, per query, with the partial over the sequence's private
 * keys by the merge rule of section "Online
 * softmax". Sequence b's keys are the prefix_len prefix tokens (token t in
 * page prefix_pages[t / page_size], slot t % page_size, of the same pools)
 * followed by its own kv_lens[b] tokens (block_table, as fa_forward_paged).
 * Its q_len_b queries are its newest positions; with causal != 0 they see the
 * whole prefix and the suffix keys j <= i + kv_lens[b] - q_len_b. The result
 * equals attention over the concatenated keys, provided every query lies in
 * its own suffix (q_len_b <= kv_lens[b] when causal).
 *
 * The work: (1) all total_q query rows against the prefix, non-causal, the
 * prefix cut into S = fa_cascade_num_splits(prefix_len, total_q, H, Hkv,
 * prefix_splits) near-equal key ranges, each giving an fp32 partial (o, lse)
 * per (row, head); (2) every sequence's own suffix as fa_forward_paged, in
 * fp32; (3) the merge of the S + 1 parts of every (row, head) into O and LSE.
 * With prefix_len == 0 it is exactly fa_forward_paged.
 *
 * Layouts and support: as fa_forward_paged (Q, O [total_q, H, d]; LSE
 * [total_q, H]), plus prefix_pages [ceil(prefix_len / page_size)] int32 in
 * device memory and a device workspace of at least
 * fa_cascade_workspace_size(total_q, H, d, S) bytes when prefix_len > 0
 * (contents on entry ignored, on exit unspecified). 0 <= prefix_splits <=
 * FA_CASCADE_MAX_SPLITS (0 = automatic). Device-side contract: as
 * fa_forward_paged, plus qo_indptr[0] == 0 and qo_indptr[B] == total_q (rows
 * outside every sequence get unspecified output) and prefix page ids in
 * [0, num_pages); violations give NaN rows instead of out-of-bounds reads.
 */
int fa_cascade_num_splits(int prefix_len, int total_q, int H, int Hkv,
                          int prefix_splits);
size_t fa_cascade_workspace_size(int total_q, int H, int d, int num_splits);
fa_status fa_cascade(const void* Q, const int32_t* qo_indptr,
                     const void* K_pool, const void* V_pool,
                     const int32_t* prefix_pages, int prefix_len,
                     int prefix_splits, const int32_t* block_table,
                     const int32_t* kv_lens, void* O, float* LSE, int B, int H,
                     int Hkv, int d, int total_q, int max_q_len, int page_size,
                     int max_pages_per_seq, int num_pages, float scale,
                     int causal, fa_dtype dtype, fa_dtype out_dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * The split plan of fa_decode_paged ("3.4 Attention Kernels", sections
 * "Decode attention and Flash-Decoding", "Worked example" and "In practice":
 * the keys of a sequence are split so that enough workgroups stream the cache
 * to fill the GPU, the count chosen from the batch size, the head count and
 * the context length).
 *
 * With num_splits == 0 a sequence with v visible tokens (min(seq_lens[b],
 * window) with a window, else seq_lens[b]) is cut into min(ceil(v / C), K)
 * chunks, with P = B * Hkv (sequence, KV head) pairs,
 * C = clamp(4 * P, 1024, 4096) tokens and K = ceil(4096 / P): short chunks
 * when few pairs have to fill the GPU (one 32K-token sequence over 8 KV heads:
 * 32 chunks per head, 256 workgroups), long and few when the pairs already do
 * (64 sequences x 8 KV heads: chunks of 2048 tokens, at most 8). num_splits > 0
 * forces that count for every sequence. Chunks are near-equal and
 * page-aligned; the kernels evaluate the rule on the device from seq_lens.
 *
 * fa_decode_max_splits - partial slots per (sequence, head) in the
 * workspace: num_splits if > 0, else min(ceil(L / C), K) clamped to
 * [1, FA_MAX_SPLITS] with L = max_pages_per_seq * FA_PAGE_SIZE (or window if
 * window > 0 and smaller). Returns -1 for invalid input.
 *
 * fa_decode_plan - the same plan on the host for a host copy of the lengths:
 * writes each sequence's chunk count to splits_out[B]. For inspection and
 * tests; the decode call does not need it.
 */
int fa_decode_max_splits(int B, int Hkv, int max_pages_per_seq, int window,
                         int num_splits);
fa_status fa_decode_plan(const int32_t* seq_lens_host, int B, int Hkv,
                         int max_pages_per_seq, int window, int num_splits,
                         int32_t* splits_out);

/*
 * fa_decode_workspace_size - bytes of device workspace fa_decode_paged (and
 * fa_decode_paged_ex with the same window) needs for B sequences of H query
 * heads (Hkv KV heads) of dimension d: one fp32 partial (o[d], lse) per
 * (b, h, slot), fa_decode_max_splits(B, Hkv, max_pages_per_seq, window,
 * num_splits) slots each. Returns 0 for invalid sizes.
 */
size_t fa_decode_workspace_size(int B, int H, int Hkv, int d,
                                int max_pages_per_seq, int window,
                                int num_splits);

/*
 * fa_decode_paged - one query token per sequence against a paged KV cache.
 *
 * Sequence b has seq_lens[b] cached tokens; token t lives in page
 * block_table[b * max_pages_per_seq + t / page_size] at slot t % page_size
 * ("3.4 Attention Kernels", "Paged and ragged layouts": pages found through
 * a block table, the fill of the final page expressed here by the sequence
 * length). Table
 * entries past the last used page are never read. The tokens are cut into
 * the near-equal, page-aligned chunks of the split plan above (as many as
 * fa_decode_plan returns for the sequence, num_splits when it is > 0);
 * each chunk's partial (o = acc / l, lse = m + ln l) is computed
 * independently and the partials are merged by the merge rule
 * ("Decode attention and Flash-Decoding"). All query heads that share a KV
 * head are processed together so each loaded K/V row serves all of them
 * (the GQA paragraph of the same section). Arithmetic as fa_forward: the
 * scores and P V run on the matrix cores with fp32 accumulation, the
 * probabilities rounded to the input type for the P V product.
 *
 * Layouts (row-major, contiguous):
 *   q            [B, H, d]                          dtype
 *   K_pool,V_pool[num_pages, page_size, Hkv, d]     dtype
 *   block_table  [B, max_pages_per_seq]  int32      device memory
 *   seq_lens     [B]                     int32      device memory
 *   O            [B, H, d]                          out_dtype (dtype or FA_F32)
 *   LSE          [B, H]                  float
 *   workspace    >= fa_decode_workspace_size(B, H, Hkv, d, max_pages_per_seq,
 *                0, num_splits) bytes of device memory, 16-byte aligned (may
 *                be NULL when the slot count is 1); contents on entry are
 *                ignored, on exit unspecified.
 *
 * Supported: dtype in {FA_F16, FA_BF16}; d in {64, 128}; page_size ==
 * FA_PAGE_SIZE; 0 <= num_splits <= FA_MAX_SPLITS; H % Hkv == 0 and
 * 1 <= H / Hkv <= 16 (a larger group returns FA_ERR_UNSUPPORTED);
 * B, Hkv <= 65535. A sequence of length 0 gets O = 0, LSE = -inf.
 * Device-side contract (not checkable on the host without a sync):
 * 0 <= seq_lens[b] <= max_pages_per_seq * page_size and every used table
 * entry lies in [0, num_pages). A sequence that breaks it is not read out of
 * bounds: its O and LSE are set to NaN instead.
 */
fa_status fa_decode_paged(const void* q, const void* K_pool,
                          const void* V_pool, const int32_t* block_table,
                          const int32_t* seq_lens, void* O, float* LSE, int B,
                          int H, int Hkv, int d, int page_size,
                          int max_pages_per_seq, int num_pages, float scale,
                          int num_splits, fa_dtype dtype, fa_dtype out_dtype,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * fa_decode_paged_ex - fa_decode_paged with two score variants, the sliding
 * window and logit soft-capping that section "Paged and ragged layouts:
 * FlashInfer" of "3.4 Attention Kernels" lists among the attention variants.
 * The page does not define them; this library's readings are:
 *   window > 0   only the newest `window` cached tokens of each sequence are
 *                visible, i.e. tokens t with seq_lens[b] - window <= t <
 *                seq_lens[b] (the query's own token counts as one of them);
 *                window == 0 means all tokens. Pages before the window are
 *                neither split over nor read, and their block-table entries
 *                are ignored.
 *   softcap > 0  each scaled score x = scale * q.k is replaced by
 *                softcap * tanh(x / softcap) before the softmax; LSE is the
 *                log-sum-exp of the capped scores. softcap == 0 disables it.
 * The split plan counts visible tokens only (min(seq_lens[b], window) for
 * window > 0), and the workspace is fa_decode_workspace_size(B, H, Hkv, d,
 * max_pages_per_seq, window, num_splits) bytes.
 * Everything else (layouts, workspace, support, contract, NaN on contract
 * violation) is as for fa_decode_paged; window < 0 or a negative or
 * non-finite softcap returns FA_ERR_BAD_ARG. With window == 0 and
 * softcap == 0 the results equal fa_decode_paged's bit for bit.
 */
fa_status fa_decode_paged_ex(const void* q, const void* K_pool,
                             const void* V_pool, const int32_t* block_table,
                             const int32_t* seq_lens, void* O, float* LSE,
                             int B, int H, int Hkv, int d, int page_size,
                             int max_pages_per_seq, int num_pages, float scale,
                             int num_splits, int window, float softcap,
                             fa_dtype dtype, fa_dtype out_dtype,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * fa_decode_paged_noalloc - fa_decode_paged_ex for callers that cannot
 * allocate device memory or pass a workspace: code being recorded into a HIP
 * graph, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, validation, arithmetic and results as fa_decode_paged_ex
 * (bit for bit), without the workspace: the per-chunk partials go to a buffer
 * of FA_NOALLOC_SCRATCH_BYTES that the library holds on each device from its
 * first call there until the process ends (a file-scope device array; its
 * device address is looked up once per device). The call itself allocates
 * nothing. Every partial the merge reads is written by the same call first,
 * so nothing needs clearing between calls.
 *
 * Limit: fa_decode_workspace_size(B, H, Hkv, d, max_pages_per_seq, window,
 * num_splits) must not exceed FA_NOALLOC_SCRATCH_BYTES, else FA_ERR_SCRATCH
 * (nothing launched). The 64-sequence, 32/8-head, d = 128 batch of up to
 * 32768 tokens per sequence with automatic splits needs 8.5 MB.
 *
 * Runs on the current HIP device. All calls on one device share its buffer:
 * calls that overlap in time on one device (different streams, threads, or
 * graph replays running together) race and give wrong results; calls on one
 * stream are ordered and safe.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
fa_status fa_decode_paged_noalloc(const void* q, const void* K_pool,
                                  const void* V_pool, const int32_t* block_table,
                                  const int32_t* seq_lens, void* O, float* LSE,
                                  int B, int H, int Hkv, int d, int page_size,
                                  int max_pages_per_seq, int num_pages,
                                  float scale, int num_splits, int window,
                                  float softcap, fa_dtype dtype,
                                  fa_dtype out_dtype, void* stream);

/*
 * A decode step recorded once and replayed with one launch.
 *
 * "3.4 Attention Kernels", section "Kernel launch overhead and CUDA graphs":
 * a step made of short kernels is bound by the host's launch rate; recording
 * the launches once and replaying them as a graph removes that cost, provided
 * shapes and buffer addresses stay fixed, so a caller refreshes the contents
 * of the recorded buffers before every replay.
 *
 * fa_decode_graph_create validates exactly what fa_decode_paged_ex validates
 * (same arguments, same status codes, nothing recorded on error), then records
 * the decode kernel and, when chunks are merged, the merge kernel on a private
 * stream into an instantiated HIP graph, stored in *out. The graph binds the
 * pointers and sizes given here: every buffer must stay allocated, unmoved and
 * sized as given until fa_decode_graph_destroy. Contents may change between
 * launches (new q, new cache tokens, new seq_lens and block_table entries
 * within the recorded max_pages_per_seq and num_pages); each launch reads the
 * buffers as they are when it runs. Creating allocates host and driver
 * objects (graph, executable graph, a temporary stream); launching allocates
 * nothing. Failures of the HIP graph API return FA_ERR_HIP and leave *out
 * NULL.
 *
 * fa_decode_graph_launch enqueues one replay on `stream` (hipStream_t as
 * void*, NULL = default stream); results equal those of the eager call on
 * the same buffer contents, bit for bit. Replays of one graph must not
 * overlap in time on different streams (they share O, LSE and workspace).
 * A NULL graph returns FA_ERR_NULL_PTR.
 *
 * fa_decode_graph_destroy frees the graph; NULL is a no-op. The caller must
 * make sure no enqueued replay is still running.
 */
typedef struct fa_decode_graph fa_decode_graph;

fa_status fa_decode_graph_create(fa_decode_graph** out, const void* q,
                                 const void* K_pool, const void* V_pool,
                                 const int32_t* block_table,
                                 const int32_t* seq_lens, void* O, float* LSE,
                                 int B, int H, int Hkv, int d, int page_size,
                                 int max_pages_per_seq, int num_pages,
                                 float scale, int num_splits, int window,
                                 float softcap, fa_dtype dtype,
                                 fa_dtype out_dtype, void* workspace,
                                 size_t workspace_bytes);
fa_status fa_decode_graph_launch(const fa_decode_graph* graph, void* stream);
void fa_decode_graph_destroy(fa_decode_graph* graph);

/*
 * fa_merge_partials - merge partial results over disjoint key sets.
 *
 * For each row r the first n = num_parts[r] parts (all S when num_parts is
 * NULL) are combined with a common reference M = max_c lse[r,c]:
 *   w_c = e^(lse[r,c] - M),  O[r,:] = sum_c w_c o[r,c,:] / sum_c w_c,
 *   LSE[r] = M + ln sum_c w_c
 * ("3.4 Attention Kernels", section "Online softmax", the merge of (m, l, acc)
 * triples; a stored partial (o, lse) is the triple (lse, 1, o)). Parts with
 * lse = -inf are empty and contribute nothing; a row whose parts are all
 * empty gets O = 0, LSE = -inf. The sum runs in a fixed order (no atomics),
 * so repeated calls give bitwise identical results.
 *
 * Layouts: o_parts [R, S, d] float; lse_parts [R, S] float; num_parts [R]
 * int32 (device memory, each in [0, S]) or NULL; O [R, d] out_dtype; LSE [R]
 * float. Supported: R >= 0, 1 <= S <= 1024, 1 <= d <= 1024, any out_dtype.
 */
fa_status fa_merge_partials(const float* o_parts, const float* lse_parts,
                            const int32_t* num_parts, void* O, float* LSE,
                            int R, int S, int d, fa_dtype out_dtype,
                            void* stream);

/* Diagnostic, not part of the attention path: reads `bytes` of device memory
 * at `buf` once, front to back, with 16-byte non-temporal loads spread over
 * the whole chip, and writes nothing unless the data XOR to one fixed value
 * (then one word to *sink). Its duration gives the read bandwidth a purely
 * memory-bound kernel can reach on the device, the yardstick beside the
 * published peak for the decode and merge kernels. buf must be 16-byte
 * aligned and bytes a multiple of 16 (else FA_ERR_BAD_ARG); bytes == 0 does
 * nothing; sink is a device pointer to one writable unsigned word. */
fa_status fa_stream_read(const void* buf, size_t bytes, unsigned* sink,
                         void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* fa_status_string(fa_status status);

/* Library version as "major.minor.patch" (static storage). */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
