/*
 * starkv.h -- C ABI of the MI355X (gfx950) latent-KV decode-attention library.
 *
 * The library implements the decode-time data path of STAR-KV (Bhatnagar et al., "STAR-KV:
 * Low-Rank KV Cache Compression via Soft Thresholding for Adaptive Rank Control"): keys are
 * cached per head as pre-RoPE latents Z_k[h] (T x r_k[h]) with a constant up factor B_k[h]
 * (r_k[h] x d); values are cached as one joint latent Z_v (T x r_v) shared by all heads, with up
 * factor B_v (r_v x H*d). A decode step appends the new token's latents and attends from the
 * latents without ever writing a full-width K or V (Zhou, "STAR-KV reading notes", sections 2.2,
 * 5.1, 5.3 and Algorithm 2; gist.science explainer, "Technisches Resuemee", Methodik 2-3).
 *
 * Conventions shared by every entry point
 *  - All pointers to bulk data are DEVICE pointers owned by the caller; descriptor structs and
 *    key_ranks are HOST memory read during the call only. The library never allocates, frees or
 *    synchronises, and keeps no pointer after it returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is enqueued on it.
 *  - Validation runs on the host before anything is enqueued: a non-OK return means nothing was
 *    enqueued and no buffer was touched. A failed launch returns STARKV_ERR_DEVICE. Faults inside
 *    kernels surface at the caller's next synchronisation of the stream.
 *  - Shapes: num_heads in [1, 32]; head_dim 64 or 128; latent layers: 1 <= r_k[h] <= head_dim and
 *    1 <= r_v <= 2048, multiples of 16 for Q43 caches; capacity a multiple of 64.
 *  - Ranks and the 16-channel tile (Zhou notes, section 6.2: a kernel that rounds ranks to its
 *    tile stores more coordinates than the chosen rank): fp caches store each head's key latent
 *    and the value latent with their ranks rounded up to a multiple of 16; the extra channels are
 *    written as zeros by every append, and the cache sizes count them. Everything the caller
 *    passes or reads back (new rows, factors, read-back rows, down-projections) uses the true
 *    ranks; in the layouts below, R_k and r_v of the cache are the rounded sums.
 *  - Bulk pointers must be 16-byte aligned.
 *  - Calls that write the same buffers must not overlap in time (use one stream per cache).
 *
 * Cache layouts (element type = cache_dtype for F32/F16/BF16; fp16 tails for Q43):
 *  - latent layer, F32/F16/BF16: channel c of a latent (key: R_k = sum_h r_k[h] channels, the
 *      heads' latents concatenated in head order; value: r_v channels) at cache token t lives in
 *      64-token block t/64 and 16-channel group c/16, 1024 elements per (block, group):
 *      zk: [B][capacity/64][R_k/16][64][16]     element (t%64, c%16): tokens rows of 16 channels
 *      zv: [B][capacity/64][r_v/16][4][16][16]  element ((t%64)/16, c%16, t%16): runs of 16
 *          consecutive tokens per channel.
 *      Each lane load of 8 consecutive elements is one MFMA operand fragment. Use
 *      starkv_append_latents / starkv_dequant to write / read rows; the layout is an internal
 *      detail of this version.
 *      zk_meta, zv_meta, zk_tail, zv_tail: unused (may be NULL).
 *  - dense (exempt) layer, F32/F16/BF16: zk = K, zv = V, both [B][capacity][H*d] token-major;
 *      keys are stored pre-RoPE.
 *  - latent layer, Q43 (mixed 4/3-bit, see starkv_layer): for each latent (zk with C = R_k
 *      channels, the heads' latents concatenated; zv with C = r_v), channel j of a latent of
 *      width r (each head's key latent, the value latent) is "hi" (q_bits_hi = 4 bits) when
 *      j < ceil(q_top_fraction * r), else "lo" (q_bits_lo = 3 bits). Per 64-token block:
 *      zk:  [B][capacity/64][key_block_bytes]: 16-channel groups in channel order, group g
 *           holding 64 token rows of 48 + n_g bits (n_g = 4-bit channels at the start of the
 *           group); row t starts at bit t*(48 + n_g) of the group; bits 3e..3e+2 of a row are
 *           the low three bits of channel e of the group, bit 48+e the fourth bit of channel
 *           e < n_g. key_block_bytes = 24*R_k + 8*(number of 4-bit key channels).
 *      zv:  [B][capacity/64][value_block_bytes]: channel c's 64 codes at byte 32c when 4-bit,
 *           32*n_hi + 24*(c - n_hi) when 3-bit, as 32-bit words whose low 16 bits hold the
 *           even tokens of the word's span and whose high 16 bits the odd tokens. 4-bit: token t
 *           in word t/8 at bit 16*(t%2) + 4*((t/2)%4). 3-bit: words 0..3 the low two bits (token
 *           t in word t/16 at bit 16*(t%2) + 2*((t/2)%8)), words 4..5 the third bit (word
 *           4 + t/32, bit 16*(t%2) + (t/2)%16).
 *      Bits are little-endian in little-endian bytes; both code buffers carry 32 bytes of
 *      padding at the end (readers load aligned windows).
 *      zk_meta / zv_meta: [B][capacity/64][2][C] fp16: per block the scales of all channels,
 *           then their zero points.
 *      zk_tail / zv_tail: [B][64][C] fp16: rows of the unfinished last group.
 *    Use starkv_cache_bytes() for every buffer size.
 */
#ifndef STARKV_H
#define STARKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    STARKV_OK = 0,
    STARKV_ERR_NULL = 1,         /* a required pointer is NULL */
    STARKV_ERR_SHAPE = 2,        /* a size is negative, zero where it must not be, or inconsistent */
    STARKV_ERR_RANK_ALIGN = 3,   /* a rank is out of bounds, or not a multiple of 16 for Q43 */
    STARKV_ERR_DTYPE = 4,        /* unknown dtype or unsupported cache/factor combination */
    STARKV_ERR_MISALIGNED = 5,   /* a bulk pointer is not 16-byte aligned */
    STARKV_ERR_CAPACITY = 6,     /* capacity not a multiple of 64, or a range beyond capacity */
    STARKV_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than starkv_decode_workspace_bytes */
    STARKV_ERR_UNSUPPORTED = 8,  /* valid request outside what the kernels implement */
    STARKV_ERR_DEVICE = 9        /* a HIP call or kernel launch failed */
} starkv_status;

typedef enum { STARKV_F32 = 0, STARKV_F16 = 1, STARKV_BF16 = 2, STARKV_Q43 = 3 } starkv_dtype;

/* One attention layer. Host memory. */
typedef struct {
    int32_t num_heads;           /* H */
    int32_t head_dim;            /* d (64 or 128) */
    const int32_t *key_ranks;    /* [H] per-head key ranks r_k[h] (latent layers; NULL if dense) */
    int32_t value_rank;          /* joint value rank r_v (latent layers; ignored if dense) */
    int32_t dense;               /* 1: exempt layer with full-width K/V; 0: latent layer */
    int32_t cache_dtype;         /* starkv_dtype: F32, F16, BF16, or Q43 (latent layers only) */
    int32_t factor_dtype;        /* starkv_dtype of B_k, B_v: F32 with F32 caches, F16 with F16 and
                                    Q43 caches, BF16 with BF16 caches */
    double rope_base;            /* RoPE base (10000 for LLaMA); must be > 1 */
    float sm_scale;              /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
    float q_top_fraction;        /* Q43: fraction of each latent's leading channels at q_bits_hi */
    int32_t q_bits_hi;           /* Q43: 4 */
    int32_t q_bits_lo;           /* Q43: 3 */
    int32_t q_group;             /* Q43: tokens per quantisation group; must be 64 */
} starkv_layer;

/*
 * Caller-owned device buffers of one layer's cache (see layouts above).
 * Paged caches (block_table != NULL): every 64-token block of a sequence lives in a page of a
 * shared pool, as in paged KV caches for serving. Block blk of sequence b is page
 * block_table[b * table_stride + blk] (device int32, 4-byte aligned, table_stride >=
 * capacity / 64) of zk, zv, zk_meta and zv_meta, which then hold num_pages pages each: size them
 * with starkv_cache_bytes(layer, num_pages, 64) (fields 0-3). The tails stay per sequence
 * ([batch][64][C], fields 4-5 of starkv_cache_bytes(layer, batch, capacity)). capacity is the
 * per-sequence capacity in tokens. Page indices are read on the device and are not checked: each
 * must address a page of the pool, and two live blocks must not share a page.
 */
typedef struct {
    int32_t batch;               /* B */
    int32_t capacity;            /* tokens per sequence the buffers hold; multiple of 64 */
    void *zk, *zv;
    void *zk_meta, *zv_meta;     /* Q43 only */
    void *zk_tail, *zv_tail;     /* Q43 only */
    const int32_t *block_table;  /* NULL: contiguous per sequence; else [batch][table_stride] */
    int32_t table_stride;
} starkv_cache;

/* Byte sizes of the six cache buffers {zk, zv, zk_meta, zv_meta, zk_tail, zv_tail} for a layer,
 * batch and capacity (0 for buffers the layout does not use). Pure host arithmetic. */
starkv_status starkv_cache_bytes(const starkv_layer *layer, int32_t batch, int32_t capacity,
                                 size_t out_bytes[6]);

/*
 * Append n_new tokens per sequence at positions [pos, pos + n_new) (Zhou notes, Algorithm 2
 * steps 1-3: the new token's latents, already in the rotated basis when rotation is used, are
 * quantised if enabled and appended).
 *   zk_new: [B][n_new][R_k] (dense: [B][n_new][H*d]); zv_new: [B][n_new][r_v] (dense: H*d), in
 *   the cache element type (fp16 for Q43). Must not alias the cache.
 * Q43: a 64-token group is quantised when it completes (its earlier rows are read from the tail
 * buffer); rows of an unfinished group are written to the tail. Appends must therefore be made in
 * increasing, gap-free positions. fp caches accept any range.
 * Errors: NULL, SHAPE (pos < 0, n_new < 0), CAPACITY (pos + n_new > capacity), DTYPE, MISALIGNED.
 * n_new == 0 or batch == 0 returns OK without enqueuing.
 */
starkv_status starkv_append_latents(const starkv_layer *layer, const starkv_cache *cache,
                                    int64_t pos, int64_t n_new, const void *zk_new,
                                    const void *zv_new, void *stream);

/* Workspace bytes starkv_decode_attn needs for this layer, batch, seq_len and split request
 * (num_splits 0 = the library's choice). Returns 0 for invalid descriptors. */
size_t starkv_decode_workspace_bytes(const starkv_layer *layer, int32_t batch, int64_t seq_len,
                                     int32_t num_splits);

/*
 * Single-token decode attention over the first seq_len cached tokens of every sequence
 * (Zhou notes, Algorithm 2 steps 4-7, section 5.3):
 *   s_{h,n} = scale * q_h . RoPE_n(Z_k[h][n] B_k[h]),  p = softmax_n(s),
 *   out_h   = (sum_n p_{h,n} Z_v[n]) B_v[:, h*d:(h+1)*d]
 * (dense layers: out_h = sum_n p_{h,n} V_h[n] with K, V full width).
 * RoPE is LLaMA rotate-half: pair (i, i+d/2) of the key at cache position n is rotated by the
 * angle n * rope_base^(-2i/d). Split-K over the sequence with a log-sum-exp merge.
 *   q:   [B][H][d] fp32, already rotated to the query's own position.
 *   bk:  [R_k][d] factor_dtype (heads' factors stacked in head order); NULL for dense layers.
 *   bv:  [r_v][H*d] factor_dtype; NULL for dense layers.
 *   out: [B][H][d] fp32, per-head attention output before the output projection.
 *   num_splits: 0 = library choice; otherwise the requested number of sequence splits whose
 *   partial results are merged (raised when needed so that no split exceeds 256 blocks of 64
 *   tokens, lowered to the number of blocks).
 *   workspace: device scratch of at least starkv_decode_workspace_bytes(...) bytes; contents on
 *   entry are ignored and clobbered.
 * For Q43 caches seq_len must equal the number of tokens appended so far (the unfinished group is
 * read from the tail), or be a multiple of 64 not above it. out and workspace must not alias any input.
 * Errors: NULL, SHAPE (seq_len < 1), CAPACITY (seq_len > capacity), DTYPE, MISALIGNED, WORKSPACE,
 * UNSUPPORTED (among others: seq_len above 256 splits of 256 blocks, 4,194,304 tokens; the
 * workspace size is then 0). batch == 0 returns OK without enqueuing.
 */
starkv_status starkv_decode_attn(const starkv_layer *layer, const starkv_cache *cache,
                                 int64_t seq_len, const float *q, const void *bk, const void *bv,
                                 float *out, int32_t num_splits, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * Ragged batches (serving): every sequence of the batch has its own length. seq_lens is a device
 * array of batch int32 lengths (4-byte aligned); each is clamped to [0, max_seq_len], and
 * max_seq_len (host) plans the splits and sizes the workspace exactly as seq_len does for
 * starkv_decode_attn (use starkv_decode_workspace_bytes with max_seq_len). Sequence b attends to
 * its first seq_lens[b] cached tokens; splits past its end contribute nothing; a length of 0
 * gives an all-zero output row. For Q43 caches each length must equal the tokens appended to
 * that sequence or be a multiple of 64 not above it. Everything else is as starkv_decode_attn.
 * Errors: those of starkv_decode_attn with seq_len = max_seq_len; NULL (seq_lens), MISALIGNED.
 */
starkv_status starkv_decode_attn_ragged(const starkv_layer *layer, const starkv_cache *cache,
                                        int64_t max_seq_len, const int32_t *seq_lens,
                                        const float *q, const void *bk, const void *bv,
                                        float *out, int32_t num_splits, void *workspace,
                                        size_t workspace_bytes, void *stream);

/*
 * Several queries per cached sequence (speculative-decoding verification, a chunk of prefill
 * queries, parallel samples; Alg. 2 steps 4-7 for each query): query row i (q[i], out[i], both
 * [num_queries][H][d] fp32) reads cache sequence query_seq[i] and attends to its first
 * query_len[i] tokens (a causal query at position p uses p + 1). query_seq and query_len are
 * device int32 arrays of num_queries entries (4-byte aligned); a sequence index is clamped to
 * [0, batch) and a length to [0, max_len]; a length of 0 gives a zero row. max_len (host) plans
 * the splits; the workspace is starkv_decode_workspace_bytes(layer, num_queries, max_len,
 * num_splits). Each query runs the single-query kernels on its own row, so rows that read the
 * same sequence share no work beyond what the caches return (the latents are streamed once per
 * query). Q43: for each cache sequence, the longest length among the rows that read it must
 * equal the tokens appended to that sequence or be a multiple of 64 not above it; the groups
 * below that length are read from the codes by every row of the sequence, so shorter causal rows
 * may end anywhere (speculative verification across a group boundary). Errors: those of
 * starkv_decode_attn with seq_len = max_len; SHAPE (num_queries < 0, or queries on a batch-0
 * cache), NULL, MISALIGNED. num_queries == 0 returns OK.
 */
starkv_status starkv_decode_attn_queries(const starkv_layer *layer, const starkv_cache *cache,
                                         int32_t num_queries, const int32_t *query_seq,
                                         const int32_t *query_len, int64_t max_len,
                                         const float *q, const void *bk, const void *bv,
                                         float *out, int32_t num_splits, void *workspace,
                                         size_t workspace_bytes, void *stream);

/*
 * nq queries per cached sequence with one key rebuild and one latent stream for all of them
 * (speculative-decoding verification of nq drafted tokens, nq parallel samples; Alg. 2 steps 4-7
 * for each query): row b*nq + i of q and out ([batch*nq][H][d] fp32) is query i of sequence b.
 * The score kernel rotates each rebuilt key once and dots it with the nq queries; the value
 * kernel feeds each latent fragment to the nq rows' probability operands. q_lens: NULL (every row
 * attends to max_len tokens) or a device int32 array of batch*nq lengths (4-byte aligned,
 * clamped to [0, max_len]; a causal query at position p uses p + 1; 0 gives a zero row). The
 * workspace is starkv_decode_multi_workspace_bytes(layer, batch, nq, max_len, num_splits).
 * nq is 1, 2 or 4; latent layers with F16, BF16 or Q43 caches (nq = 1 also F32). Q43: the
 * longest of a sequence's nq lengths follows the starkv_decode_attn_queries rule. max_len is at
 * most 4,194,304 / nq tokens (256 splits of 256 / nq blocks; the workspace size is 0 above it).
 * Errors: those of starkv_decode_attn with seq_len = max_len; SHAPE (nq < 1), UNSUPPORTED (other
 * nq, dense layers, F32 with nq > 1, max_len above the limit), MISALIGNED.
 * Grouped query attention (G query heads per KV head; the reading notes' ledger counts KV heads):
 * describe the H_kv KV heads in the layer (their ranks, B_k rows and B_v columns) and pass the
 * query heads as rows: row b*G + g, head slot h holds query head h*G + g of sequence b, with
 * nq = G (2 or 4; other G go through starkv_decode_attn_queries, one row per (sequence, g)). Each
 * KV head's key is then rebuilt and rotated once for its G query heads, and its B_v slice applies
 * to each of them.
 */
size_t starkv_decode_multi_workspace_bytes(const starkv_layer *layer, int32_t batch, int32_t nq,
                                           int64_t max_len, int32_t num_splits);
starkv_status starkv_decode_attn_multi(const starkv_layer *layer, const starkv_cache *cache,
                                       int32_t nq, int64_t max_len, const int32_t *q_lens,
                                       const float *q, const void *bk, const void *bv, float *out,
                                       int32_t num_splits, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * One new token per sequence at its own position (the append step of a ragged decode batch,
 * Alg. 2 steps 1-3): positions is a device array of batch int32 positions (4-byte aligned);
 * sequence b's rows zk_new[b] ([batch][R_k] with the caller's ranks; dense: [batch][H*d]) and
 * zv_new[b] go to cache token positions[b]. A position outside [0, capacity) skips that sequence
 * (idle slots of a serving batch). Q43: the row is written to the tail and, when it is the last
 * token of its 64-token group, the group is quantised; each sequence must be appended in
 * increasing, gap-free positions. Errors: NULL, DTYPE, MISALIGNED; batch == 0 returns OK.
 */
starkv_status starkv_append_latents_ragged(const starkv_layer *layer, const starkv_cache *cache,
                                           const int32_t *positions, const void *zk_new,
                                           const void *zv_new, void *stream);

/*
 * starkv_decode_attn with kernel timing for profiling tools: event_begin, event_mid and event_end
 * (hipEvent_t passed as void*, created by the caller, each may be NULL) are recorded on `stream`
 * immediately before the kernel that streams the key latents, between it and the kernel that
 * streams the value latents, and after that one (dense layers: before and after the single
 * attention kernel, event_mid right after it). Everything else is identical to starkv_decode_attn
 * (same validation, same kernels, same results). Extra error: STARKV_ERR_DEVICE if recording an
 * event fails.
 */
starkv_status starkv_decode_attn_timed(const starkv_layer *layer, const starkv_cache *cache,
                                       int64_t seq_len, const float *q, const void *bk,
                                       const void *bv, float *out, int32_t num_splits,
                                       void *workspace, size_t workspace_bytes, void *stream,
                                       void *event_begin, void *event_mid, void *event_end);

/*
 * Decode attention followed by the output projection, in one call (Zhou notes, Algorithm 2 steps
 * 4-8; section 5.3 applies W_o after the latent value sum): y[b] = concat_h(out[b][h]) . W_o with
 * out as starkv_decode_attn computes it. wo, hidden: as starkv_output_projection (output-major
 * [hidden][H*d], the layer's factor type). y: [batch][hidden] fp32. The heads' outputs stay in the
 * workspace (starkv_decode_attn_project_workspace_bytes(layer, batch, seq_len, num_splits,
 * hidden)); W_o is read once per call. Results are bit for bit those of starkv_decode_attn
 * followed by starkv_output_projection. Errors: those of both calls, checked before anything is
 * enqueued.
 */
size_t starkv_decode_attn_project_workspace_bytes(const starkv_layer *layer, int32_t batch,
                                                  int64_t seq_len, int32_t num_splits,
                                                  int32_t hidden);
starkv_status starkv_decode_attn_project(const starkv_layer *layer, const starkv_cache *cache,
                                         int64_t seq_len, const float *q, const void *bk,
                                         const void *bv, const void *wo, int32_t hidden, float *y,
                                         int32_t num_splits, void *workspace,
                                         size_t workspace_bytes, void *stream);

/*
 * Prefill: a chunk of causal queries per sequence attends to the latent cache (a prompt chunk or
 * a long speculative draft; Zhou notes, Algorithm 2 steps 4-7 for every query of the chunk,
 * section 5.3 for the latent values; the model card times such a prefill kernel beside its decode
 * kernel). Query l of sequence b sits at position pos0 + l and attends to cached tokens
 * [0, pos0 + l] (its own token included): the chunk's latents must already be appended.
 *   chunk_lens: NULL (every sequence has `chunk` queries) or a device int32 array of batch chunk
 *     lengths (4-byte aligned, clamped to [0, chunk]); rows l >= chunk_lens[b] are empty (zero
 *     output).
 *   q:   [B][chunk][H][d] fp32, each query already rotated to its own position.
 *   bk, bv: as starkv_decode_attn.
 *   out: [B][chunk][H][d] fp32, per-head outputs before the output projection.
 * The keys (rotated to their positions in fp32) and the values of every head (Z_v B_v^h: for a
 * chunk of queries this order costs 2 d instead of 2 r_v flop per query, key and head) of each
 * 32-token tile up to pos0 + chunk_lens[b] are rebuilt once per call and kept in the workspace as
 * binary16 hi/lo parts; attention then runs 32 queries per wave on the matrix cores (query-key
 * products as hi/lo parts, an online softmax whose rescalings are exact powers of two) and writes
 * each output once. Latent layers with F16, BF16 or Q43 caches (Q43: sequence b must hold
 * pos0 + chunk_lens[b] appended tokens, or a multiple of 64 not above that). The workspace is
 * starkv_prefill_workspace_bytes(layer, batch, pos0, chunk), about
 * batch * (pos0 + chunk) * (2 r_v + 8 H d) bytes, plus batch * (pos0 + chunk) * 2 R_k for Q43
 * (16-bit key latents are read in place) (0 for invalid or unsupported requests); contents on
 * entry are ignored.
 * Errors: NULL, SHAPE (pos0 < 0, chunk < 1), CAPACITY (pos0 + chunk > capacity), DTYPE,
 * MISALIGNED, WORKSPACE, UNSUPPORTED (dense or F32 layers; pos0 + chunk above 4,194,304 tokens;
 * batch * chunk above 2^30). batch == 0 returns OK without enqueuing.
 */
size_t starkv_prefill_workspace_bytes(const starkv_layer *layer, int32_t batch, int64_t pos0,
                                      int32_t chunk);
starkv_status starkv_prefill_attn(const starkv_layer *layer, const starkv_cache *cache, int64_t pos0,
                                  int32_t chunk, const int32_t *chunk_lens, const float *q,
                                  const void *bk, const void *bv, float *out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * starkv_decode_attn without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). Same
 * arguments, validation, kernels and results as starkv_decode_attn with the same num_splits; the
 * workspace is a fixed device array of starkv_decode_attn_noalloc_max_bytes() bytes (64 MiB)
 * inside the library, one per GPU, looked up on the device current at the call (make the
 * stream's device current), and held until the process ends. Nothing is allocated or freed and
 * nothing needs to start at zero. Every call on a GPU shares that GPU's array, which keeps the
 * last call's contents: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.
 * Errors: those of starkv_decode_attn; WORKSPACE when starkv_decode_workspace_bytes(layer, batch,
 * seq_len, num_splits) exceeds the maximum (e.g. batch 16, 32 heads, r_v 1024 fits up to about
 * 43,000 tokens); DEVICE if the array's device address cannot be found.
 */
size_t starkv_decode_attn_noalloc_max_bytes(void);
starkv_status starkv_decode_attn_noalloc(const starkv_layer *layer, const starkv_cache *cache,
                                         int64_t seq_len, const float *q, const void *bk,
                                         const void *bv, float *out, int32_t num_splits,
                                         void *stream);

/*
 * Read cached tokens [t0, t1) back in token-major order (the dequantisation step of the decode
 * path: Zhou notes, section 6.1, which stores the cache as per-channel asymmetric 4/3-bit codes
 * with fp16 scales and zero points per group of 64 tokens, and Algorithm 2 step 4a, which
 * dequantises the latent tile before the keys are rebuilt): zk_out [B][t1-t0][R_k] (dense: H*d)
 * and zv_out [B][t1-t0][r_v] (dense: H*d). Element type: fp16 for Q43 (codes of complete groups
 * are dequantised as binary16(code * scale + zero), the exact value rounded once to
 * nearest-even; rows of the unfinished group come from the tail), otherwise the cache element
 * type (a plain gather). The decode kernels dequantise the same way in registers; this call
 * materialises the rows for inspection and tests. seq_len is the number of tokens appended so
 * far (Q43: decides which groups are complete). Either output may be NULL to skip it.
 * Errors: NULL (cache buffers), SHAPE (t0 < 0 or t0 > t1), CAPACITY (t1 > seq_len or seq_len >
 * capacity), DTYPE, MISALIGNED.
 */
starkv_status starkv_dequant(const starkv_layer *layer, const starkv_cache *cache,
                             int64_t seq_len, int64_t t0, int64_t t1, void *zk_out, void *zv_out,
                             void *stream);

/*
 * Offline preparation: absorb the blockwise Hadamard rotation (Zhou notes, section 6.1 / Fig. 5).
 * Each latent (every head's key latent for which = 0, the joint value latent for which = 1) is
 * split into its first ceil(q_top_fraction * r) channels and the rest; each part of width w is
 * rotated by blockdiag(H_b, ...) with b = min(64, largest power of two dividing w) and H_b the
 * normalised Sylvester-Hadamard matrix. kind 0 rotates latent rows (dst = src . H, src/dst
 * [n][C]); kind 1 rotates factor rows (dst = H^T . src, src/dst [C][n] with n = head_dim for keys,
 * H*d for values). fp16 in and out: each output is binary16 of (the exact signed sum of the
 * inputs) times the fp64 value of 1/sqrt(b). src and dst must not alias.
 * The layer's top fraction picks the split; src and dst are caller-owned device buffers of n * C
 * binary16 values (C = R_k for which = 0, r_v for which = 1), 2-byte aligned. n = 0 returns OK
 * without enqueuing. Errors (before anything is enqueued): NULL, SHAPE (which or kind not 0/1,
 * n < 0, or kind 1 with n other than the factor's column count), DTYPE (layer cache type not
 * F16 or Q43), UNSUPPORTED (dense layer), RANK_ALIGN, MISALIGNED.
 */
starkv_status starkv_hadamard_rotate(const starkv_layer *layer, int32_t which, int32_t kind,
                                     int64_t n, const void *src, void *dst, void *stream);

/*
 * Rows times weights on the matrix cores: the two dense products around decode attention share
 * one kernel pair (a split over the inner dimension, then a fixed-order sum of the split partials
 * fused with the store). Weights are output-major (row n holds output n's inputs contiguously,
 * the layout of a linear layer's weight). The fp32 input rows are split into two 16-bit parts
 * (hi = nearest 16-bit value, lo = nearest 16-bit value of the remainder) and both are
 * multiplied with fp32 accumulation, so results are within a few fp32 rounding errors of the
 * exact products; inputs must lie within the binary16 range for fp16 weights. Every workspace is
 * caller-owned device scratch of at least the queried size, 16-byte aligned; contents on entry
 * are ignored and clobbered.
 */

/* Workspace bytes for starkv_output_projection (0 for an invalid layer, batch < 1 or hidden < 1). */
size_t starkv_output_projection_workspace_bytes(const starkv_layer *layer, int32_t batch,
                                               int32_t hidden);

/*
 * Output projection of the layer (Zhou notes, Algorithm 2 step 8; section 5.3 applies W_o after
 * the value step): y[b] = concat_h(out[b][h]) . W_o, i.e. y[b][n] = sum_{h,j} out[b][h][j] *
 * wo[n][h*d + j].
 *   o:  [batch][H*d] fp32, the per-head outputs of starkv_decode_attn (its `out`).
 *   wo: [hidden][H*d] output-major (W_o transposed), the layer's factor type (latent layers) or
 *       cache type (dense layers).
 *   y:  [batch][hidden] fp32, 4-byte aligned; o, wo and the workspace 16-byte aligned.
 * y must not alias o, wo or the workspace. batch == 0 returns OK without enqueuing.
 * Errors (before anything is enqueued): NULL, SHAPE (batch < 0, hidden < 1), DTYPE, MISALIGNED,
 * WORKSPACE.
 */
starkv_status starkv_output_projection(const starkv_layer *layer, int32_t batch, const float *o,
                                      const void *wo, int32_t hidden, float *y, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* Workspace bytes for starkv_append_tokens (0 for an invalid layer, batch < 1, n_new < 1 or
 * model_dim < 64). Does not depend on pos. */
size_t starkv_append_tokens_workspace_bytes(const starkv_layer *layer, int32_t batch,
                                            int64_t n_new, int32_t model_dim);

/*
 * Fused append front-end (Zhou notes, Algorithm 2 steps 1-3): project the new tokens' hidden
 * states to their key and value latents and append them, without writing the latents anywhere
 * but the cache:
 *   zk_new[b][t] = x[b][t] . A_k (A_k: the heads' key down-projections side by side, R_k columns)
 *   zv_new[b][t] = x[b][t] . A_v (r_v columns)
 * each output rounded once (nearest-even) to the cache element type (binary16 for Q43), then
 * stored exactly as starkv_append_latents stores zk_new / zv_new (Q43: rows go to the tail and a
 * group this call completes is quantised). For Q43 layers the blockwise rotation is absorbed into
 * the weights by the caller (section 6.1: the down-projection takes the rotation), so A_k and A_v
 * here are the rotated ones. Dense layers: A_k, A_v are the full key and value projections
 * (H*d columns each) and the keys are stored pre-RoPE.
 *   x:   [batch][n_new][model_dim] fp32 hidden states; model_dim a multiple of 64.
 *   a_k: [R_k][model_dim] output-major (A_k transposed; dense: [H*d][model_dim]), a_v:
 *        [r_v][model_dim] (dense: [H*d][model_dim]); factor type (latent) or cache type (dense).
 * Q43 appends are processed one 64-token group at a time (a call spanning g groups makes about
 * 2g launches); as with starkv_append_latents, Q43 appends must be made in increasing, gap-free
 * positions. Errors (before anything is enqueued): NULL, SHAPE (pos < 0, n_new < 0,
 * model_dim < 1), CAPACITY (pos + n_new > capacity), DTYPE, MISALIGNED, WORKSPACE, UNSUPPORTED
 * (model_dim not a multiple of 64). n_new == 0 or batch == 0 returns OK without enqueuing.
 */
starkv_status starkv_append_tokens(const starkv_layer *layer, const starkv_cache *cache,
                                   int64_t pos, int64_t n_new, const float *x, int32_t model_dim,
                                   const void *a_k, const void *a_v, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* Static description of a status code (never NULL). */
const char *starkv_status_string(starkv_status status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t starkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STARKV_H */
