/*
 * bi_attn.h — batch-invariant causal GQA attention over a paged KV cache, for MI355X (gfx950).
 *
 * The method comes from public write-ups of "Defeating Nondeterminism in LLM Inference":
 * an attention kernel gives a token the same bits whatever the batch around it if (1) the KV
 * page table is brought up to date before the kernel launches, so the kernel always sees one
 * consistent KV layout, and (2) a split reduction over the sequence fixes the *size* of each
 * split rather than the number of splits, so the reduction order is the same however many
 * query tokens are processed (neican.ai insight page, section 技术原理与创新点解析,
 * batch-invariant attention item; xitu-tech.com report, section 构建确定性解决方案, attention
 * item). Prefill and decode must not reduce a token differently (liuwei.blog post, section
 * 破解之道：重塑GPU内核, FlashAttention-2 paragraph).
 *
 * Contract of every attention call: each query token's fp32 output is bit-identical whatever
 * the batch size, its position in the batch, the chunk size, and whether it is computed by
 * bi_attn_decode or bi_attn_prefill, within one build of this library on one device.
 *
 * Conventions shared by all calls
 *  - Pointers are device pointers unless stated, 16-byte aligned, and stay owned by the
 *    caller. The library never allocates, frees or synchronises; it is stateless apart from
 *    a lazily cached CU count per device, which only affects the split-by-batch policies.
 *  - Layouts (row-major, element type given by cfg->dtype unless stated):
 *      q            [T][Hq][D]                         (decode: T = batch)
 *      k_new, v_new [T][Hkv][D]
 *      k/v cache    [num_pages][Hkv][page_size][D]
 *      page_table   int32 [batch][max_pages]: physical page of positions
 *                   [i*page_size, (i+1)*page_size) of sequence b is page_table[b][i]
 *      seq_lens     int32 [batch]: tokens in the cache for sequence b AFTER this step
 *      q_starts     int32 [batch+1]: prefix sums of new tokens per sequence
 *      out          fp32 [T][Hq][D], fully overwritten
 *    A new token i of sequence b sits at absolute position seq_lens[b] - n_new[b] + i, and
 *    attends causally to positions 0..pos inclusive. Query head h reads KV head h / (Hq/Hkv).
 *  - Host scalars (batch, total_tokens, max_q_len, max_seq_len, max_pages, num_pages) size
 *    the grids and bound every index; per-sequence data stays in device arrays. Device data
 *    that breaks them (seq_lens[b] > max_seq_len, a page index outside [0, num_pages), more
 *    pages than max_pages) is never dereferenced: the affected rows come out NaN (attention)
 *    or are skipped (page update).
 *  - Errors: arguments are validated synchronously and a status other than BI_OK is returned
 *    with nothing launched. A failed launch returns BI_EHIP. Faults in device code surface at
 *    the caller's next synchronisation. No C++ exception crosses this interface.
 *  - All work is enqueued on `stream`; calls are asynchronous.
 */
#ifndef BI_ATTN_H_
#define BI_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { BI_F32 = 0, BI_BF16 = 1 } bi_dtype;

typedef enum {
  BI_OK = 0,
  BI_EINVAL = 1,        /* a null pointer, a negative size, Hq % Hkv != 0, ... */
  BI_EUNSUPPORTED = 2,  /* a valid but unimplemented shape: D not 64/128, page_size != 16, ... */
  BI_EWORKSPACE = 3,    /* workspace missing or smaller than bi_attn_workspace_bytes() */
  BI_EHIP = 4           /* the HIP runtime reported an error at launch */
} bi_status;

typedef enum {
  /* Fixed split size cfg->split_size, splits aligned to absolute position 0 (invariant). */
  BI_SPLIT_FIXED = 0,
  /* Comparison variant, measurement only: split size chosen per sequence from the batch size,
   * S' = roundup32(ceil(len / n)), n = clamp(ceil(2 * CUs / (batch * Hkv)), 1, ceil(len / 32)),
   * the way split-count heuristics pick their splits. Outputs change bits with the batch. */
  BI_SPLIT_BY_BATCH = 1,
  /* The same with n = clamp(ceil(8 * CUs / (batch * Hkv)), 1, ceil(len / 32)): enough splits
   * to fill the waves the attention kernels keep resident (8 per CU). Measurement only. */
  BI_SPLIT_BY_BATCH_FILL = 2
} bi_split_policy;

typedef struct {
  int32_t num_q_heads;   /* Hq; Hq % Hkv == 0; Hq / Hkv a power of two <= 64 */
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim;      /* D: 64 or 128 */
  int32_t page_size;     /* tokens per page: 16 */
  int32_t split_size;    /* S: fixed split length in keys, a positive multiple of 32 */
  int32_t dtype;         /* bi_dtype of q, k_new, v_new and the caches; out is always fp32 */
  float softmax_scale;   /* 0 => 1/sqrt(head_dim) */
  int32_t split_policy;  /* bi_split_policy */
} bi_attn_cfg;

/*
 * Page update: write the step's new tokens into the caches through the page table, before
 * any attention call of the step on the same stream (neican.ai insight page, section
 * 技术原理与创新点解析, batch-invariant attention item: the page table is updated before the
 * kernel launches so the KV layout is always consistent).
 * The caller has already chosen pages and written page_table[b][pos / page_size] for every
 * new position. Token i of sequence b (row q_starts[b] + i of k_new/v_new) goes to
 * cache[page_table[b][pos / page_size]][kv_head][pos % page_size][:], pos as above.
 * Only those slots are written; nothing else in the caches changes.
 */
int bi_kv_page_update(const bi_attn_cfg* cfg, const void* k_new, const void* v_new,
                      const int32_t* q_starts, const int32_t* seq_lens,
                      const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                      int32_t batch, int32_t total_tokens, void* k_cache, void* v_cache,
                      hipStream_t stream);

/*
 * Bytes of workspace bi_attn_decode needs for up to `rows_tokens` query tokens whose
 * sequences are at most `max_seq_len` long: per (token, q head, split) an fp32 partial
 * (max, sum of exponentials, D accumulators). bi_attn_prefill needs none. Returns 0 for an
 * invalid cfg. Host-only; queries the current device's CU count for the by-batch policies.
 */
size_t bi_attn_workspace_bytes(const bi_attn_cfg* cfg, int32_t rows_tokens, int32_t max_seq_len);

/*
 * Decode: one new query token per sequence (q [batch][Hq][D]), at position seq_lens[b] - 1,
 * whose K/V the page update has already written. Keys are reduced in fixed-size splits
 * [j*S, j*S + S) of absolute positions, each split to a partial (max, sum, acc) in the
 * workspace, and the partials are folded in ascending j (neican.ai insight page, section
 * 技术原理与创新点解析). The split arithmetic and the fold are the same code that
 * bi_attn_prefill runs, so a token gets identical bits from either call.
 * workspace: device memory of at least bi_attn_workspace_bytes(cfg, batch, max_seq_len);
 * its contents are undefined on return. max_seq_len >= every seq_lens[b].
 * Returns BI_EUNSUPPORTED, with nothing launched, when the partials of one (sequence, KV head)
 * would reach 2 GiB: Jmax * (Hq / Hkv) * D * 4 >= 2^31 (Jmax below; at S = 256, Hq / Hkv = 16,
 * D = 128 that is max_seq_len >= 2^26). Every decode entry point below shares this limit.
 */
int bi_attn_decode(const bi_attn_cfg* cfg, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* page_table, int32_t max_pages,
                   int32_t num_pages, const int32_t* seq_lens, int32_t batch,
                   int32_t max_seq_len, float* out, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * bi_attn_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and bits,
 * with the split partials in a static device array of BI_NOALLOC_SCRATCH_BYTES that the
 * library holds on each device it runs on until the process ends; nothing is allocated or
 * freed. Returns BI_EWORKSPACE, with nothing launched, when the call needs more than that
 * (bi_attn_workspace_bytes-sized partials for this batch and max_seq_len; 64 MiB holds, for
 * example, 64 sequences of up to 8192 tokens with 32 query heads). Every call on one device
 * shares the array: calls that overlap in time on one device (different streams, host
 * threads) race, so the caller must order them. Arguments otherwise as bi_attn_decode.
 */
#define BI_NOALLOC_SCRATCH_BYTES (64u << 20)
int bi_attn_decode_noalloc(const bi_attn_cfg* cfg, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* page_table, int32_t max_pages,
                           int32_t num_pages, const int32_t* seq_lens, int32_t batch,
                           int32_t max_seq_len, float* out, hipStream_t stream);

/*
 * The two phases of bi_attn_decode, for callers that move or inspect the split partials
 * between them (a context-parallel decode gathers partials from several devices and folds
 * them in ascending split order on the row's owner), and for per-kernel timing.
 * bi_attn_decode(...) == bi_attn_decode_partials(...) then bi_attn_decode_combine(...) on
 * the same stream, with the same cfg, seq_lens, batch, max_seq_len and workspace, bit for bit.
 * Partials layout in the workspace (fp32), G = Hq / Hkv: first (m, l) pairs
 * [batch*Hkv][Jmax][G], padded to 256 bytes, then accumulators [batch*Hkv][Jmax][G][D]; query
 * head h of sequence b is entry (b*Hkv + h/G, j, h%G). Jmax = ceil(max_seq_len / S) for
 * BI_SPLIT_FIXED. m is in base-2 units (max of q.k * scale * log2(e)).
 */
int bi_attn_decode_partials(const bi_attn_cfg* cfg, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* page_table, int32_t max_pages,
                            int32_t num_pages, const int32_t* seq_lens, int32_t batch,
                            int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);
int bi_attn_decode_combine(const bi_attn_cfg* cfg, const int32_t* seq_lens, int32_t batch,
                           int32_t max_seq_len, float* out, const void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Decode step with the page update folded in: the page update of the step's one new token per
 * sequence, then decode, in the decode's own launches (one fewer kernel per step than
 * bi_kv_page_update followed by bi_attn_decode). k_new, v_new: [batch][Hkv][D], row b the new
 * token of sequence b, at position seq_lens[b] - 1. The kernel that reads that position takes
 * the token's K and V rows from k_new / v_new (the bytes its slot receives) and writes them to
 * cache[page_table[b][pos / page_size]][kv_head][pos % page_size]. Outputs, partials and the
 * written slots are bit-identical to bi_kv_page_update (q_starts = 0, 1, ..., batch) followed by
 * bi_attn_decode with the same arguments (same neican.ai page and section as the page update and
 * decode above: the step writes the page before attention reads it), except that a sequence
 * whose length is outside [1, max_seq_len] has its slot left unwritten (its row is NaN either
 * way). No other sequence of the batch may read a new token's slot, as with the separate calls.
 * bi_attn_decode_append_partials is its first phase (page update and split partials), for
 * per-kernel timing; bi_attn_decode_combine completes it. Arguments otherwise as bi_attn_decode.
 */
int bi_attn_decode_append(const bi_attn_cfg* cfg, const void* q, const void* k_new,
                          const void* v_new, void* k_cache, void* v_cache,
                          const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                          const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);
int bi_attn_decode_append_partials(const bi_attn_cfg* cfg, const void* q, const void* k_new,
                                   const void* v_new, void* k_cache, void* v_cache,
                                   const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                                   const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Chunked prefill: n_new[b] = q_starts[b+1] - q_starts[b] new tokens per sequence (any
 * number, including 0 and 1), on top of a cached prefix; q [total_tokens][Hq][D]. Attention
 * reads all keys, prefix and chunk, through the page table (liuwei.blog post, section
 * 破解之道：重塑GPU内核: a token's reduction must not depend on whether its keys arrive as
 * a prefill block or from a full cache). max_q_len >= every n_new[b]; max_seq_len >= every
 * seq_lens[b]; q_starts non-decreasing from q_starts[0] >= 0 to q_starts[batch] <=
 * total_tokens. A sequence that breaks these (n_new[b] > max_q_len, q_starts[b+1] >
 * total_tokens, n_new[b] > seq_lens[b], seq_lens[b] > max_seq_len) gets NaN in its rows that
 * lie in q (rows q_starts[b] .. min(q_starts[b+1], total_tokens) - 1); a pair of q_starts
 * entries out of order gives the sequence no rows; the rows of every other sequence are
 * computed as usual (with q_starts out of order, rows claimed by two sequences are
 * unspecified). Nothing outside q, out and the caches is read or written.
 * workspace may be NULL (not used).
 */
int bi_attn_prefill(const bi_attn_cfg* cfg, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* page_table, int32_t max_pages,
                    int32_t num_pages, const int32_t* q_starts, const int32_t* seq_lens,
                    int32_t batch, int32_t total_tokens, int32_t max_q_len, int32_t max_seq_len,
                    float* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dense varlen attention, the trainer-side form of chunked prefill: K and V are contiguous
 * arrays [total_k][Hkv][D] (not a paged cache), sequence b owning rows k_starts[b] ..
 * k_starts[b+1] - 1 (k_starts ascending, k_starts[batch] <= total_k), so seq_len[b] =
 * k_starts[b+1] - k_starts[b]. Its n_new[b] = q_starts[b+1] - q_starts[b] queries (rows of q
 * [total_q][Hq][D]) are its last n_new positions, causal as in bi_attn_prefill. Sampling and
 * training must agree bit for bit for on-policy reinforcement learning (xitu-tech.com report,
 * section 强化学习的突破; neican.ai insight page, section 未来发展路径预测, true on-policy RL
 * item): this call runs the prefill kernel's arithmetic on the dense layout, so each output
 * row is bit-identical to bi_attn_prefill / bi_attn_decode on the same keys and values held
 * in a paged cache (any page placement, any batch, any chunking), within one build on one
 * device. A sequence whose k_starts entries are out of range, or with n_new > seq_len,
 * seq_len > max_seq_len, n_new > max_q_len or q_starts[b+1] > total_q, gets NaN rows (those
 * that lie in q), as in bi_attn_prefill. max_q_len >= every n_new[b]. No workspace.
 */
int bi_attn_varlen(const bi_attn_cfg* cfg, const void* q, const void* k, const void* v,
                   const int32_t* q_starts, const int32_t* k_starts, int32_t batch,
                   int32_t total_q, int32_t total_k, int32_t max_q_len, int32_t max_seq_len,
                   float* out, hipStream_t stream);

/* Static English text for a bi_status value (never NULL). */
const char* bi_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BI_ATTN_H_ */
