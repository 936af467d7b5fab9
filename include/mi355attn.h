/*
 * mi355attn — exact fused attention forward and split-KV decode for MI355X
 * (gfx950 / CDNA4). C ABI.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, row-major, in device memory owned by the caller. The
 *    library allocates nothing, keeps no workspace and no mutable global state
 *    (apart from a per-device cache of the compute-unit count, which the split
 *    kernels size their grid by, the fixed device array of attn_bwd_noalloc
 *    with its per-device address, and the launch-log switch below), and may be
 *    called from several host threads at once.
 *  - Launch log: with the environment variable MI355ATTN_LOG set to anything
 *    but "" or "0" when the first kernel is launched, every launch prints one
 *    line to stderr, "mi355attn: " then the kernel (dtype, head dim, variant),
 *    its grid and block, the problem's shape and the stream. The variable is
 *    read once per process; logging changes nothing that runs.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    Every call only enqueues work on that stream and returns at once.
 *  - The return value covers argument checks and the launch itself
 *    (hipGetLastError after the launch), never the completion of the kernels.
 *    Argument checks run before any HIP call, so a rejected call touches no GPU
 *    state. No call aborts or throws.
 *  - `dtype` selects the 16-bit element type of q, k, v and o:
 *    MI355ATTN_BF16 (0) or MI355ATTN_FP16 (1). LSE values are always fp32.
 *  - q, k, v, o, the caches and part_o must be 16-byte aligned (the kernels use
 *    128-bit loads and stores); lse, part_lse and seq_lens 4-byte aligned.
 *  - Offsets are computed in 64 bits; a single tensor may exceed 2^31 elements.
 *  - `scale` multiplies q.k before the mask and the exponential; it must be
 *    finite and > 0 (the usual value is 1/sqrt(d)).
 *  - The LSE is the natural log of sum_j exp(scale * q.k_j) over the allowed keys
 *    (as in the rustytorch "flash_attention_forward.cu" page,
 *    OnlineSoftmaxState::get_log_sum_exp). A row with no allowed key gets O = 0
 *    and LSE = -inf.
 */
#ifndef MI355ATTN_H
#define MI355ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element type codes. */
#define MI355ATTN_BF16 0
#define MI355ATTN_FP16 1

/* Status codes. */
#define MI355ATTN_OK 0
#define MI355ATTN_ERR_NULL_PTR (-1)    /* a required pointer is NULL */
#define MI355ATTN_ERR_BAD_SHAPE (-2)   /* a size <= 0, Hq % Hkv != 0, a sequence longer than
                                          2^23 (Nq, Nk, max_len), or a grid too large */
#define MI355ATTN_ERR_UNSUPPORTED (-3) /* d not in {64, 128}, unknown dtype, Hq/Hkv > 32 in decode */
#define MI355ATTN_ERR_MISALIGNED (-4)  /* a pointer breaks the alignment rule above */
#define MI355ATTN_ERR_BAD_ARG (-5)     /* scale not finite or <= 0, causal not 0/1 */
#define MI355ATTN_ERR_HIP (-6)         /* the HIP runtime reported an error at launch */
#define MI355ATTN_ERR_SCRATCH (-7)     /* larger than the fixed scratch of attn_bwd_noalloc */

/*
 * attn_fwd — exact attention forward with per-row log-sum-exp.
 *
 *   O = softmax(scale * Q K^T + mask) V,   LSE_i = log sum_j exp(scale * q_i.k_j)
 *
 * computed tile by tile with the online-softmax rescale, so the Nq x Nk score
 * matrix never exists in memory (the algorithm described in the module
 * documentation of the abaddon "attention.rs" page: Q tile resident, K/V tiles
 * streamed, running max and sum, final division by the sum).
 *
 *   q   [B, Hq,  Nq, d]   dtype        (read)
 *   k   [B, Hkv, Nk, d]   dtype        (read)
 *   v   [B, Hkv, Nk, d]   dtype        (read)
 *   o   [B, Hq,  Nq, d]   dtype        (written, rounded to nearest even)
 *   lse [B, Hq,  Nq]      float        (written)
 *
 * Query head h reads key/value head floor(h * Hkv / Hq) (grouped-query
 * attention, as in the abaddon page's flash_attention_f16); Hq must be a
 * multiple of Hkv. d must be 64 or 128. causal = 1 allows key j for query row i
 * iff j <= i + (Nk - Nq) (aligned to the bottom-right corner; for Nq == Nk this
 * is the pages' j <= i); causal = 0 allows every key.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype, void* stream);

/*
 * attn_fwd_qkvpacked — attn_fwd reading q, k and v straight out of one packed
 * projection output, with no permute (the llm.c page's attention_forward first
 * permutes a [B, N, 3, H, d] qkv tensor into separate q, k, v; here the kernel
 * addresses the packed rows directly), and writing o token-major, ready for the
 * output projection:
 *
 *   qkv [B, N, 3, H, d]  dtype  (read: q = qkv[:, :, 0], k = [:, :, 1], v = [:, :, 2])
 *   o   [B, N, H, d]     dtype  (written, rounded to nearest even)
 *   lse [B, H, N]        float  (written)
 *
 * Hq = Hkv = H; causal, d, dtype and scale as in attn_fwd.
 */
int attn_fwd_qkvpacked(const void* qkv, void* o, float* lse, int B, int N, int H, int d,
                       float scale, int causal, int dtype, void* stream);

/*
 * attn_fwd_local — attn_fwd with a local (sliding-window) mask, the "local"
 * mode that the flash-attention page's kernel traits carry as a flag: key j is
 * allowed for query row i iff
 *
 *   i + (Nk - Nq) - window_left <= j <= i + (Nk - Nq) + window_right
 *
 * (aligned to the bottom-right corner, as the causal mask of attn_fwd); a
 * negative window_left or window_right puts no bound on that side, so (-1, 0)
 * is attn_fwd's causal mask and (-1, -1) no mask. Only the key tiles a row's
 * window touches are read. Tensors, head mapping, d, dtype and scale as in
 * attn_fwd; a row with no allowed key gets O = 0 and LSE = -inf.
 */
int attn_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, int window_left,
                   int window_right, int dtype, void* stream);

/*
 * attn_bwd — gradients of attn_fwd: given dout = dL/dO, writes dq, dk, dv, with
 * the probabilities recomputed from the forward's LSE rather than stored (the
 * backward of the flash-attention page's "flash_bwd_kernel" and the llm.c
 * page's attention_backward compute the same quantities):
 *
 *   D_i = sum_t dout_it o_it,  P_ij = exp(scale q_i.k_j - lse_i) (0 if masked),
 *   dS_ij = P_ij (dout_i.v_j - D_i),
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i
 *
 * where dk and dv of a key/value head sum over the query heads that read it.
 *
 *   q, o, dout [B, Hq,  Nq, d]  dtype  (read; o and lse as attn_fwd wrote them)
 *   k, v       [B, Hkv, Nk, d]  dtype  (read)
 *   lse        [B, Hq,  Nq]     float  (read)
 *   delta      [B, Hq,  Nq]     float  (workspace owned by the caller: written
 *                                       with D, then read)
 *   dq         [B, Hq,  Nq, d]  dtype  (written, rounded to nearest even)
 *   dk, dv     [B, Hkv, Nk, d]  dtype  (written, rounded to nearest even)
 *
 * Shapes, head mapping, causal alignment, d, dtype and scale as in attn_fwd. A
 * query row with no allowed key contributes nothing and gets dq = 0. Two
 * kernels run in order on `stream` (dq, which also writes delta, then dk and
 * dv); the result does not depend on scheduling (no atomics).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int Hq, int Hkv,
             int Nq, int Nk, int d, float scale, int causal, int dtype, void* stream);

/*
 * attn_bwd_ds — attn_bwd with the score gradient dS stored once instead of
 * recomputed (the llm.c page's attention_backward keeps the whole score
 * gradient matrix in memory; here it is written once, rounded to dtype, and
 * read once): D from dout and o, then dk and dv (which also write dS^T to `ds`),
 * then dq = scale * dS k from `ds`, so S and dP are formed once per (row, key)
 * pair instead of twice.
 *
 *   arguments as attn_bwd, plus
 *   ds        workspace owned by the caller, 256-byte aligned, ds_bytes long,
 *             at least attn_bwd_ds_workspace(B, Hq, Nq, Nk) bytes (written,
 *             then read; its contents on entry do not matter)
 *
 * The workspace holds dS^T in blocks of 64 keys x 128 query rows (16 KiB each,
 * one per (batch, head, 64-key tile, 128-row block)): B * Hq * ceil(Nk / 64) *
 * ceil(Nq / 128) * 16384 bytes (1 GiB at B=4, Hq=32, Nq=Nk=2048), so this form
 * suits moderate lengths; attn_bwd needs no such buffer. Three kernels run in order on `stream`; no atomics. ds_bytes below
 * the requirement returns MI355ATTN_ERR_BAD_ARG, a misaligned ds
 * MI355ATTN_ERR_MISALIGNED.
 */
int attn_bwd_ds(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, float* delta, void* ds, long long ds_bytes, void* dq,
                void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                int causal, int dtype, void* stream);

/* Bytes attn_bwd_ds needs in `ds` (MI355ATTN_ERR_BAD_SHAPE for sizes <= 0 or
 * lengths above 2^23). */
long long attn_bwd_ds_workspace(int B, int Hq, int Nq, int Nk);

/*
 * attn_bwd_noalloc — attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * it): the same kernels and the same result, with D kept in a fixed scratch
 * array inside the library instead of the caller's delta buffer. Nothing is
 * allocated by the call.
 *
 *   arguments as attn_bwd, without delta.
 *
 * The scratch holds 4194304 floats (16 MiB) on each GPU the library runs on,
 * from the first call there until the process ends; B * Hq * Nq above that
 * returns MI355ATTN_ERR_SCRATCH before any HIP call. Every call on one GPU
 * uses the same scratch (each call rewrites what it reads), so calls that
 * overlap in time on one GPU (other streams, other host threads) race and
 * must be serialised by the caller.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                     int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
                     void* stream);

/*
 * attn_fwd_varlen — attn_fwd over a packed batch of sequences of different
 * lengths (the variable-length mode that the flash-attention page's kernel
 * traits carry as a flag): no padding, each sequence attends only to its own
 * keys, with its own causal alignment.
 *
 *   q            [total_q, Hq,  d]   dtype  (read)
 *   k            [total_k, Hkv, d]   dtype  (read)
 *   v            [total_k, Hkv, d]   dtype  (read)
 *   o            [total_q, Hq,  d]   dtype  (written, rounded to nearest even)
 *   lse          [Hq, total_q]       float  (written)
 *   cu_seqlens_q [B + 1]             int32, device memory (read)
 *   cu_seqlens_k [B + 1]             int32, device memory (read)
 *
 * Sequence b owns query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]); both arrays must start at 0, never
 * decrease and end at total_q / total_k (values are clamped into [0, total]
 * and a decrease counts as an empty sequence, so the kernel never reads or
 * writes outside the tensors). With Nq_b and Nk_b its lengths, causal = 1
 * allows key j for query row i iff j <= i + (Nk_b - Nq_b) (bottom-right, as in
 * attn_fwd); a row with no allowed key gets O = 0 and LSE = -inf. max_seqlen_q
 * sizes the grid and must be >= every Nq_b: rows of a longer sequence past
 * max_seqlen_q are not written. Head mapping, d, dtype and scale as attn_fwd.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                    int total_q, int total_k, int max_seqlen_q, int d, float scale, int causal,
                    int dtype, void* stream);

/*
 * attn_decode_split — first half of split-KV ("flash decoding") decode: one new
 * query token per sequence against a padded KV cache, split into chunks of
 * `chunk` keys; each chunk emits its own normalised partial output and LSE
 * (the partials that the aprender-gpu "flash_decoding/reduce_kernel.rs" page's
 * reduction consumes, stored here as O_c and LSE_c = m_c + log l_c instead of
 * the unnormalised sum with separate max and sum; the two carry the same
 * information).
 *
 *   q        [B, Hq, d]                dtype  (read)
 *   k_cache  [B, Hkv, max_len, d]      dtype  (read: rows < seq_lens[b] only)
 *   v_cache  [B, Hkv, max_len, d]      dtype  (read: rows < seq_lens[b] only)
 *   seq_lens [B]                       int32, device memory (read); values are
 *                                      clamped to [0, max_len]
 *   part_o   [B, Hq, C, d]             float  (written for chunks c < ceil(L_b/chunk))
 *   part_lse [B, Hq, C]                float  (written for every c; -inf past the end)
 *
 * with C = ceil(max_len / chunk). Chunk c of sequence b covers keys
 * [c*chunk, min((c+1)*chunk, L_b)). d must be 64 or 128 and Hq/Hkv <= 32.
 */
int attn_decode_split(const void* q, const void* k_cache, const void* v_cache,
                      const int* seq_lens, float* part_o, float* part_lse, int B, int Hq,
                      int Hkv, int max_len, int d, int chunk, float scale, int dtype,
                      void* stream);

/*
 * attn_decode_split_paged — attn_decode_split over a paged KV cache (block
 * tables), the cache layout of the aprender-gpu page's
 * "attention/paged/flash_decoding" module: the keys of a sequence live in
 * fixed-size pages anywhere in a shared pool, and a per-sequence table lists
 * the pages in order.
 *
 *   q           [B, Hq, d]                         dtype  (read)
 *   k_pages     [num_pages, page_size, Hkv, d]     dtype  (read: rows a sequence uses)
 *   v_pages     [num_pages, page_size, Hkv, d]     dtype  (read: rows a sequence uses)
 *   block_table [B, max_pages]                     int32, device memory (read)
 *   seq_lens    [B]                                int32, device memory (read); values
 *                                                  clamped to [0, max_pages * page_size]
 *   part_o      [B, Hq, C, d]                      float  (written as in attn_decode_split)
 *   part_lse    [B, Hq, C]                         float  (written as in attn_decode_split)
 *
 * with C = ceil(max_pages * page_size / chunk). Logical key j of sequence b is
 * row j % page_size of page block_table[b][j / page_size]; pages may be shared
 * between sequences (read only). The result is that of attn_decode_split on the
 * cache these lookups describe, and attn_decode_combine (with max_chunks = C)
 * merges it. page_size and chunk must be multiples of 16 and one chunk may span
 * at most 16 pages (chunk / page_size <= 16 when chunk is a multiple of
 * page_size, else (chunk + page_size - 2) / page_size + 1 <= 16), else
 * MI355ATTN_ERR_UNSUPPORTED.
 * Table entries a sequence uses must lie in [0, num_pages); the kernel never
 * reads outside k_pages / v_pages: an entry out of range reads as zero keys
 * and values (the result for that sequence is then meaningless).
 */
int attn_decode_split_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int* block_table, const int* seq_lens, float* part_o,
                            float* part_lse, int B, int Hq, int Hkv, int num_pages, int page_size,
                            int max_pages, int d, int chunk, float scale, int dtype, void* stream);

/*
 * attn_decode_combine — second half of split-KV decode: merges the partials of
 * each (b, h) with the rescaling combine (the two passes of the aprender-gpu
 * reduce kernel: global maximum M of the chunk LSEs, then weights
 * exp(LSE_c - M), weighted mean of the chunk outputs):
 *
 *   O = sum_c w_c O_c / sum_c w_c,   LSE = M + log(sum_c w_c)
 *
 * over the first ceil(L_b / chunk) chunks (capped at max_chunks); chunks whose
 * LSE is -inf carry no weight.
 *
 *   part_o   [B, Hq, max_chunks, d]  float  (read)
 *   part_lse [B, Hq, max_chunks]     float  (read)
 *   seq_lens [B]                     int32, device memory (read, clamped at 0)
 *   o        [B, Hq, d]              dtype  (written, rounded to nearest even)
 *   lse      [B, Hq]                 float  (written)
 *
 * max_chunks and chunk must be the C and chunk used for attn_decode_split.
 */
int attn_decode_combine(const float* part_o, const float* part_lse, const int* seq_lens,
                        void* o, float* lse, int B, int Hq, int max_chunks, int d, int chunk,
                        int dtype, void* stream);

/*
 * attn_decode — single-token decode in one call: the library picks the chunk
 * length from the shape and runs attn_decode_split (+ attn_decode_combine) with
 * it, or, when one chunk covers max_len and the (sequence, kv-head) pairs
 * already fill the GPU, a single pass whose split kernel writes o and lse
 * itself (no partials, no combine; the unsplit short-context regime of the
 * abaddon page's cached-decode kernel, done with one read of K and V and no
 * atomics). The chunk is about eight work items per resident wave if every
 * sequence had max_len keys, clamped to [256, 2048] keys.
 *
 *   q, k_cache, v_cache, seq_lens  as attn_decode_split
 *   o          [B, Hq, d]   dtype  (written, rounded to nearest even)
 *   lse        [B, Hq]      float  (written)
 *   workspace  float array of workspace_floats elements, 16-byte aligned,
 *              owned by the caller; it must hold at least
 *              attn_decode_workspace(B, Hq, Hkv, max_len, d) floats (NULL is
 *              allowed when that is 0). Its contents are scratch.
 *
 * The result equals attn_decode_split + attn_decode_combine at any chunk (up to
 * rounding). A too-small workspace returns MI355ATTN_ERR_BAD_ARG.
 */
int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                void* o, float* lse, float* workspace, long long workspace_floats, int B, int Hq,
                int Hkv, int max_len, int d, float scale, int dtype, void* stream);

/*
 * attn_decode_workspace — the number of floats attn_decode needs as workspace
 * for this shape on the current device (0: a single pass needs none), or a
 * negative status code for a shape attn_decode would reject. The chunk choice
 * depends on the device's compute-unit count, so query it on the device that
 * will run the decode.
 */
long long attn_decode_workspace(int B, int Hq, int Hkv, int max_len, int d);

/*
 * attn_decode_fused — split-KV decode in a single launch: the combine of the
 * aprender-gpu "flash_decoding/reduce_kernel.rs" page (global maximum of the
 * chunk LSEs, weights exp(LSE_c - M), weighted mean) runs inside the split
 * kernel, started by the chunk that finishes last (a last-block-done counter
 * per (sequence, kv-head) pair), so there is no second kernel and no pass over
 * every partial by a separate launch. A sequence that fits one chunk writes
 * its final output directly.
 *
 *   q, k_cache, v_cache, seq_lens  as attn_decode_split (chunk keys per chunk)
 *   o          [B, Hq, d]   dtype  (written, rounded to nearest even)
 *   lse        [B, Hq]      float  (written; a sequence of length 0 gets O = 0
 *                                   and LSE = -inf)
 *   workspace  attn_decode_fused_workspace(B, Hq, Hkv, max_len, d, chunk)
 *              floats (workspace_floats given), 256-byte aligned, owned by the
 *              caller: B*Hkv int32 counters first, then the chunk partials.
 *              The counters must be zero the first time a workspace is used
 *              (e.g. memory allocated zeroed); every call that runs to its end
 *              leaves them zero again, so the workspace can be reused call
 *              after call. Calls that overlap in time must not share one.
 *
 * The result equals attn_decode_split + attn_decode_combine with the same
 * chunk (up to rounding). Needs (Hq/Hkv) * ceil(max_len/chunk) * d * 4 < 2^32
 * (else MI355ATTN_ERR_UNSUPPORTED); a too-small workspace returns
 * MI355ATTN_ERR_BAD_ARG.
 */
int attn_decode_fused(const void* q, const void* k_cache, const void* v_cache,
                      const int* seq_lens, void* o, float* lse, float* workspace,
                      long long workspace_floats, int B, int Hq, int Hkv, int max_len, int d,
                      int chunk, float scale, int dtype, void* stream);

/*
 * attn_decode_fused_paged — attn_decode_fused over a paged KV cache; q,
 * k_pages, v_pages, block_table, seq_lens, page_size and chunk as in
 * attn_decode_split_paged (max_len = max_pages * page_size), o, lse and the
 * workspace as in attn_decode_fused.
 */
int attn_decode_fused_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int* block_table, const int* seq_lens, void* o, float* lse,
                            float* workspace, long long workspace_floats, int B, int Hq, int Hkv,
                            int num_pages, int page_size, int max_pages, int d, int chunk,
                            float scale, int dtype, void* stream);

/*
 * attn_decode_fused_workspace — floats of workspace attn_decode_fused (and
 * attn_decode_fused_paged, with max_len = max_pages * page_size) needs for
 * this shape and chunk, or a negative status code for a shape it rejects.
 */
long long attn_decode_fused_workspace(int B, int Hq, int Hkv, int max_len, int d, int chunk);

/* A static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MI355ATTN_H */
