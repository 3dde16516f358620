/*
 * dsa.h -- C ABI of libdsa, the MI355X (gfx950) DeepSeek-Sparse-Attention
 * decode path of GLM-5.3-Flash.
 *
 * The calls follow the pipeline diagram of the Atlas docs page
 * "spark_model/layers/glm5next_dsa/mod.rs", section "Shape of the pipeline":
 *
 *   k,gate,valid,ape -> kpool_compress -> pool keys / starts / validity
 *                    -> index_scores   -> [Q, P] scores + candidate validity
 *                    -> topk_pools     -> [Q, select_k] pool ids
 *                    -> expand_selection -> [Q, out_width] token ids (-1 = none)
 *                    -> sparse_mla_decode (NoPE MLA over those tokens)
 *
 * plus the fp32 indexer head-gate w = hidden @ W of stkernel pull request
 * #227 ("indexer fp32 head-gate split-K"), whose output weights the heads of
 * index_scores.
 *
 * Conventions shared by every call:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  Arrays are
 *    dense, row-major, with the element types named in each comment; bf16
 *    values travel as uint16_t bit patterns, fp8 as uint8_t codes.
 *  - Every tensor pointer (workspaces included) is 16-byte aligned, as
 *    hipMalloc's and torch's allocations are; the kernels use 16-byte vector
 *    accesses.  A misaligned pointer is INVALID_ARG.
 *  - The library never allocates, frees, synchronizes, or reads device memory
 *    on the host.  Each call validates its host arguments first and, if they
 *    are bad, returns an error before launching anything; otherwise it
 *    enqueues its kernels on `stream` and returns DSA_OK (or DSA_ERR_LAUNCH if
 *    the runtime refused a launch).  Calls are safe to capture in a HIP graph.
 *  - Every per-request length lives in a device array, so a captured graph
 *    replays correctly over changed lengths.  Host integers only bound sizes.
 *  - A missing or unsupported path is an error, never a silent fallback onto
 *    another computation.
 *  - dsa_last_error() returns a thread-local message for the last failing call
 *    of the calling thread.
 *  - Calls on one stream are ordered; two calls that share a workspace must
 *    not run concurrently.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 4

typedef int dsa_status;
#define DSA_OK 0
#define DSA_ERR_INVALID_ARG 1 /* an argument breaks the documented contract */
#define DSA_ERR_UNSUPPORTED 2 /* a legal shape the library has no kernel for */
#define DSA_ERR_LAUNCH 3      /* the HIP runtime refused a launch */

/* latent cache element types for dsa_sparse_mla_decode */
#define DSA_LATENT_BF16 0
#define DSA_LATENT_FP8_E4M3 1 /* OCP E4M3FN codes, one f32 scale per row */

/* Largest kpool: the Atlas page's validate() refuses index_kpool above the
 * 8 pool slots its compression kernel keeps in registers. */
#define DSA_MAX_KPOOL 8
/* The latent width: validate() refuses a kv_lora_rank other than 512 (NoPE, so
 * the cache row is exactly kv_lora_rank wide). */
#define DSA_KV_LORA 512
/* Most indexer heads one head-gate row / index_scores call supports. */
#define DSA_MAX_INDEX_HEADS 16

int dsa_abi_version(void);
const char* dsa_last_error(void);

/* ---------------------------------------------------------------------------
 * a1. Indexer head-gate   [stkernel PR #227]
 *
 *   w[m, n] = sum_k hidden[m, k] * W[k, n]        (fp32 in, fp32 accumulate)
 *
 * hidden [M, K] f32, W [K, N] f32, w [M, N] f32.  1 <= N <= 16, K >= 1,
 * M >= 0 (M = 0 is a no-op).  For M <= 512 (decode, and small batches)
 * every row gets its own workgroup that spreads K over 1024 threads and adds
 * the partial sums in a fixed order, so the result is deterministic and the
 * same bits for a row whatever the batch (up to 512 rows).  For M > 512 one
 * workgroup per 16 rows splits K over 16 waves (fp32 MFMA when K % 16 == 0)
 * and adds the waves' partial sums in a fixed order, so those rows are
 * deterministic too.  No
 * workspace is needed at present (dsa_head_gate_workspace_size returns 0; ws
 * may be NULL).
 * Errors: INVALID_ARG for N outside [1,16], K < 1, M < 0, or a NULL or
 * misaligned pointer with M > 0.
 * ------------------------------------------------------------------------- */
size_t dsa_head_gate_workspace_size(int M, int K, int N);
dsa_status dsa_head_gate(const float* hidden, const float* W, float* w, int M, int K, int N,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * a2. Gated pool compression with k_norm   [Atlas page, "Traps carried from
 *     Slice 8" and the k_norm field of Glm5NextDsaKernels]
 *
 * Request r owns rows tok_off[r] .. tok_off[r+1]-1 of k, gate and valid, and
 * pool slots pool_off[r] .. pool_off[r+1]-1 of keys, pool_start, pool_valid
 * (its capacity cap_r).  With f_r its first valid row (request-local) and
 * P_r = floor((T_r - f_r) / kpool) its full pools (0 if no row is valid):
 *   pool p covers rows f_r + p*kpool + s, s < kpool;
 *   alpha[s, c] = softmax over s of (gate[row_s, c] + ape[s, c]), per channel;
 *   x[c] = sum_s alpha[s, c] * k[row_s, c];
 *   keys[p] = bf16_rne( (x - mean x) / sqrt(var x + eps) * ln_w + ln_b )
 *             (biased variance; LayerNorm with bias, not an RMSNorm);
 *   pool_start[p] = f_r + p*kpool;  pool_valid[p] = 1 iff every slot row is
 *   valid.  Slots p in [P_r, cap_r) get start -1, valid 0, key 0.
 *   n_pools[r] = P_r.
 * Left padding is skipped, and a trailing partial pool is not a pool.
 *
 * T_r is the region's size tok_off[r+1] - tok_off[r], or, when seq_len [B]
 * i32 is given, the live length seq_len[r] (clamped to [0, region]): a
 * request's region may hold more rows than it has written (rows past the live
 * length are not read).  ln_w = ln_b = NULL: the k rows were normalised when
 * stored (dsa_indexer_store with a LayerNorm, the per-token k_normed form) and
 * keys[p] = bf16_rne(x), with no LayerNorm.
 *
 * k, gate [sumT, D] bf16; ape [kpool, D] bf16; valid [sumT] u8 (0/1);
 * tok_off [B+1] i32; pool_off [B+1] i32 with cap_r >= floor(T_r / kpool);
 * ln_w, ln_b [D] f32 (or both NULL); keys [sum cap, D] bf16; pool_start [sum cap] i32;
 * pool_valid [sum cap] u8; n_pools [B] i32.  max_cap >= every cap_r (host
 * bound that sizes the grid).
 *
 * Incremental mode (a decode step that appended rows): new_from [B] i32 is the
 * first request-local row that changed in request r, and max_new >= T_r -
 * new_from[r] for every r.  Then only the pools holding a row at or after
 * new_from[r] (p in [floor((new_from[r] - f_r)/kpool), P_r)) are written,
 * with n_pools; all other slots keep their contents (the sentinels and pools
 * of an earlier full call).  The slots must hold the result of an earlier call
 * on the same rows before new_from[r] with the same pool_off: slot 0 of a
 * request, when it holds a pool starting before new_from[r], supplies f_r.
 * new_from = NULL recomputes every slot.
 * Errors: INVALID_ARG for kpool outside [1, 8] (never truncated), B < 0, NULL
 * pointers, exactly one of ln_w / ln_b NULL, max_cap < 0, max_new < 1 with
 * new_from; UNSUPPORTED for D not in {32, 64, 128, 256} or more than 65535
 * requests.
 * ------------------------------------------------------------------------- */
dsa_status dsa_kpool_compress(const uint16_t* k, const uint16_t* gate, const uint16_t* ape,
                              const uint8_t* valid, const int32_t* tok_off, const int32_t* pool_off,
                              const int32_t* seq_len, const float* ln_w, const float* ln_b,
                              float eps, int B, int D,
                              int kpool, int max_cap, const int32_t* new_from, int max_new,
                              uint16_t* keys, int32_t* pool_start, uint8_t* pool_valid,
                              int32_t* n_pools, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * a3. Index scores   [Atlas page, "Shape of the pipeline": [Q, P] scores +
 *     candidate validity]
 *
 * For query q of request r = q_req[q] and request-local pool p < pstride:
 *   score[q, p] = sum_h w[q, h] * max(0, <qi[q, h, :], keys[pool_off[r] + p, :]>)
 * (bf16 products, fp32 accumulation, a -0 result stored as +0) when p is a
 * candidate: p < n_pools[r], pool_valid, and pool_start + kpool - 1 <=
 * q_pos[q].  Otherwise score = -inf and cand = 0.  Every element of the
 * [Q, pstride] rows is written.
 * qi [Q, H, D] bf16; w [Q, H] f32 (the head-gate output); keys, pool_start,
 * pool_valid, pool_off, n_pools as written by dsa_kpool_compress; q_req,
 * q_pos [Q] i32; scores [Q, pstride] f32; cand [Q, pstride] u8.
 * pstride >= every cap_r.
 * Performance: with Q >= 256 and at least 256 (8-query block, 256-pool block)
 * pairs (prefill-sized calls) the call reads each 256-pool block of keys once
 * per 8 consecutive queries, so queries of one request should be consecutive
 * in q_req; any order gives the same bits, only slower.
 * Errors: INVALID_ARG for H outside [1, 16], kpool outside [1, 8], pstride < 1,
 * Q < 0, NULL pointers; UNSUPPORTED for D not in {32, 64, 128, 256} or
 * Q > 65535.
 * ------------------------------------------------------------------------- */
dsa_status dsa_index_scores(const uint16_t* qi, const float* w, const uint16_t* keys,
                            const int32_t* pool_start, const uint8_t* pool_valid,
                            const int32_t* pool_off, const int32_t* n_pools, const int32_t* q_req,
                            const int32_t* q_pos, int Q, int H, int D, int kpool, int pstride,
                            float* scores, uint8_t* cand, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * a4. Pool top-k   [Atlas page, "Shape of the pipeline": [Q, select_k] pool
 *     ids; Glm5NextDsaConfig::select_k caps the budget by the pools there are]
 *
 * Row q keeps the k_eff = min(select_k, #candidates) candidates with the
 * largest score, ties to the lower pool id, and lists their ids in ascending
 * order in sel[q, 0 .. k_eff-1]; sel[q, k_eff ..] = -1.  The ordering is exact
 * (fp32 keys compared as ordered integers), so the result is a pure function
 * of the scores.
 * scores [Q, pstride] f32, cand [Q, pstride] u8, sel [Q, select_k] i32.
 * row_len [Q] i32 or NULL: only entries p < row_len[q] of row q count
 * (clamped to [0, pstride]; NULL means pstride), for rows shorter than the
 * batch's widest.
 * Any row length is taken: rows of up to 16384 entries stay in registers.
 * A longer row is selected in two stages when ws holds
 * dsa_topk_pools_workspace_size bytes: each 16384-entry block of the row
 * keeps its own top select_k (the row's top select_k is among them), then one
 * workgroup selects among those candidates; this needs at most 16384
 * candidates per row (blocks x select_k).  Otherwise (ws NULL or smaller, or
 * too many candidates) the row is read again from memory on each pass of a
 * one-workgroup select.  A row of 4096 to 16384 entries with
 * 8 * select_k <= 2048 takes the two stages too, in 2048-entry blocks, when
 * ws is large enough (else one pass).  All give the same result.
 * Workspace: Q x candidates x 4 bytes for rows that take two stages (0
 * otherwise); ws may be NULL.
 * Errors: INVALID_ARG for select_k < 1, pstride < 1, Q < 0, NULL pointers.
 * ------------------------------------------------------------------------- */
size_t dsa_topk_pools_workspace_size(int Q, int pstride, int select_k);
dsa_status dsa_topk_pools(const float* scores, const uint8_t* cand, const int32_t* row_len, int Q,
                          int pstride, int select_k, int32_t* sel, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------
 * a5. Selection expansion   [Atlas page, "Shape of the pipeline" and "Traps":
 *     the -1 sentinel destination must be fully written]
 *
 *   tok[q, j*kpool + s] = pool_start[pool_off[q_req[q]] + sel[q, j]] + s
 * for sel[q, j] >= 0 and s < kpool; every other element of the [Q, out_width]
 * row is -1.  Ids are request-local row positions.
 * sel [Q, select_k] i32; pool_start, pool_off, q_req as above; tok
 * [Q, out_width] i32.  flags must be 0 (bit 0 is reserved: the
 * always_select_tail slots are written by dsa_select_tail afterwards).
 * Errors: INVALID_ARG for out_width < select_k * kpool (the page's
 * topk-multiple-of-kpool rule), kpool outside [1, 8], select_k < 1, unknown
 * flag bits, NULL pointers; UNSUPPORTED for flag bit 0 or Q > 65535.
 * ------------------------------------------------------------------------- */
dsa_status dsa_expand_selection(const int32_t* sel, const int32_t* pool_start,
                                const int32_t* pool_off, const int32_t* q_req, int Q, int select_k,
                                int kpool, int out_width, int flags, int32_t* tok,
                                hipStream_t stream);

/* ---------------------------------------------------------------------------
 * always_select_tail   [Atlas page, Glm5NextDsaConfig::out_width: the tail adds
 *     kpool - 1 slots to the emitted row]
 *
 * Run after dsa_expand_selection or dsa_topk_expand on the same tok rows.  For
 * query q at request-local position t = q_pos[q] of request r = q_req[q], with
 * first valid row f_r: the pools that count for q are the full pools ending at
 * or before t, P_t = floor((t + 1 - f_r) / kpool) of them; the rows after them
 * up to t (fewer than kpool) are q's tail.  Its valid rows, in ascending
 * order, are written to tok[q, select_k*kpool + i]; the rest of those kpool-1
 * slots get -1.  No other element of the row is touched; a query before f_r
 * has no tail.  f_r is read as pool_start of the request's pool 0 when
 * n_pools[r] > 0 (so pool_start and n_pools must be this step's compression
 * output).
 * valid [sumT] u8; tok_off [B+1], pool_start, pool_off [B+1], n_pools [B],
 * q_req, q_pos [Q] i32; tok [Q, out_width] i32.
 * Errors: INVALID_ARG for kpool outside [1, 8], select_k < 1, out_width <
 * select_k*kpool + kpool - 1, Q < 0, NULL pointers.  kpool = 1 has no tail
 * slots and launches nothing.
 * ------------------------------------------------------------------------- */
dsa_status dsa_select_tail(const uint8_t* valid, const int32_t* tok_off, const int32_t* pool_start,
                           const int32_t* pool_off, const int32_t* n_pools, const int32_t* q_req,
                           const int32_t* q_pos, int Q, int kpool, int select_k, int out_width,
                           int32_t* tok, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * a6. NoPE sparse MLA decode   [Atlas page, "Traps" (NoPE: the latent is both
 *     key and value, kv_cache_dim = kv_lora_rank = 512) and the
 *     MASKED_ATTN_MAX_KEYS note (a per-row gather of the selected ids equals
 *     the dense set-membership mask; online softmax, no full score row kept)]
 *
 * For query q, head h, over the ids j with tok[q, j] >= 0 and latent row
 * c_j = ckv[kv_off[q_req[q]] + tok[q, j]] (times ckv_scale of that row for
 * fp8):  l_j = sm_scale * <q[q, h, :], c_j>,  out[q, h] = sum_j softmax(l)_j
 * c_j (rounded to bf16),  lse[q, h] = log sum_j exp(l_j).  A row with no
 * selected id gives out = 0, lse = -inf.
 * q [Q, Hm, L] bf16; ckv [rows, L] bf16 or fp8 codes; ckv_scale [rows] f32
 * (fp8 only, else NULL); kv_off [B] i32; q_req [Q] i32; tok [Q, out_width]
 * i32; out [Q, Hm, L] bf16; lse [Q, Hm] f32 or NULL.
 * The selected ids of a row are split into chunks processed by separate
 * workgroups and merged in a fixed order; the workspace
 * dsa_sparse_mla_decode_workspace_size(Q, Hm, L, out_width, latent_dtype)
 * holds the per-chunk partial results (its contents need no initialisation).
 * Errors: UNSUPPORTED for L != 512 (the latent width is fixed, as the page's
 * validate() demands); INVALID_ARG for Hm < 1, out_width < 1, Q < 0, an
 * unknown latent_dtype, fp8 without ckv_scale, NULL pointers, or ws_bytes
 * below the size; UNSUPPORTED for Q > 65535.
 * ------------------------------------------------------------------------- */
size_t dsa_sparse_mla_decode_workspace_size(int Q, int Hm, int L, int out_width,
                                            int latent_dtype);
dsa_status dsa_sparse_mla_decode(const uint16_t* q, const void* ckv, const float* ckv_scale,
                                 int latent_dtype, const int32_t* kv_off, const int32_t* q_req,
                                 const int32_t* tok, int Q, int Hm, int L, int out_width,
                                 float sm_scale, uint16_t* out, float* lse, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * a6 over a paged latent cache   [Atlas page, the MASKED_ATTN_MAX_KEYS note
 *     (the serving decode is a block-table paged, online-softmax MLA that walks
 *     a selected-index row) and the step taps (the logical selection and the
 *     physical indices are kept apart)]
 *
 * As dsa_sparse_mla_decode, with the rows found through a block table instead
 * of kv_off: the cache is n_pages pages of page_rows rows each (ckv
 * [n_pages * page_rows, L], ckv_scale the same rows for fp8), and request r's
 * logical row x is physical row
 *     block_table[r * bt_stride + x / page_rows] * page_rows + x % page_rows.
 * block_table [B, bt_stride] i32, row-major (entries past a request's blocks
 * are never read as pages; any value).  kvidx [Q, out_width] i32 or NULL:
 * receives the physical row of every selected id, -1 where tok is -1.
 * The workspace is dsa_sparse_mla_decode_workspace_size's.
 * Ids must lie inside their request's blocks and table entries inside the
 * cache; out-of-range block numbers and page numbers are clamped (to the table
 * row, to the cache), so a bad table gives wrong rows, never an access outside
 * block_table or ckv.
 * Errors: those of dsa_sparse_mla_decode; INVALID_ARG for bt_stride,
 * page_rows or n_pages < 1; UNSUPPORTED for n_pages * page_rows > 2^31 - 1.
 * ------------------------------------------------------------------------- */
dsa_status dsa_sparse_mla_decode_paged(const uint16_t* q, const void* ckv, const float* ckv_scale,
                                       int latent_dtype, const int32_t* block_table,
                                       int bt_stride, int page_rows, int n_pages,
                                       const int32_t* q_req, const int32_t* tok, int Q, int Hm,
                                       int L, int out_width, float sm_scale, uint16_t* out,
                                       float* lse, int32_t* kvidx, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* -------------------------------------------------------------------------
 * dsa_sparse_mla_decode_noalloc -- dsa_sparse_mla_decode without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, kernels, results (bit for bit) and errors as
 * dsa_sparse_mla_decode, except ws / ws_bytes: the per-chunk partials go to a
 * fixed array of DSA_MLA_SCRATCH_BYTES inside the library, one per GPU,
 * allocated when the library's code is loaded on that GPU and held until the
 * process ends.  The call itself allocates and frees nothing.  Its device
 * address is looked up (hipGetSymbolAddress) on the first call on each device,
 * with that device current.
 * Every call on one GPU shares that GPU's array, and the array keeps what the
 * last call wrote (nothing in it needs to start at zero): calls that overlap
 * on one GPU (two streams, two threads) race and give wrong results.
 * Errors: those of dsa_sparse_mla_decode; UNSUPPORTED when
 * dsa_sparse_mla_decode_workspace_size(Q, Hm, L, out_width, latent_dtype)
 * exceeds DSA_MLA_SCRATCH_BYTES (nothing is launched); INVALID_ARG when the
 * stream belongs to a device other than the current one; LAUNCH when the
 * array's address cannot be found.
 * ------------------------------------------------------------------------- */
#define DSA_MLA_SCRATCH_BYTES (32u << 20)
dsa_status dsa_sparse_mla_decode_noalloc(const uint16_t* q, const void* ckv,
                                         const float* ckv_scale, int latent_dtype,
                                         const int32_t* kv_off, const int32_t* q_req,
                                         const int32_t* tok, int Q, int Hm, int L, int out_width,
                                         float sm_scale, uint16_t* out, float* lse,
                                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The cache-write side of a decode step   [Atlas page, Glm5NextDsaKernels:
 *     write_geom (the step's selector geometry derived on the device from
 *     seq_len, so a captured graph replays over the live context) and
 *     indexer_store (the staged indexer row placed at a device-side position
 *     and marked valid; the page's per-token k_normed row)]
 *
 * dsa_write_geom: one decode query per request, from the live lengths
 * seq_len [B] i32 (a negative length counts as 0):
 *   q_req[r] = r;  q_pos[r] = seq_len[r] - 1 (-1 for an empty request: no
 *   candidate pool and no tail);  new_from[r] = max(seq_len[r] - 1, 0) (the
 *   row the step writes, where dsa_kpool_compress's incremental mode starts);
 *   slot[r] = the physical latent row of position seq_len[r] - 1 under the
 *   block table, as dsa_sparse_mla_decode_paged maps it (-1 when empty).
 * q_req, new_from and slot may be NULL (not written); slot needs block_table
 * [B, bt_stride], page_rows and n_pages as in dsa_sparse_mla_decode_paged.
 * Errors: INVALID_ARG for B < 0, NULL seq_len / q_pos, slot without a valid
 * table geometry.
 *
 * dsa_indexer_store: for each request r with 0 <= pos[r] < tok_off[r+1] -
 * tok_off[r], row tok_off[r] + pos[r] of k and gate receives k_new[r] and
 * gate_new[r], and valid of that row becomes 1; other positions store nothing.
 * With ln_w / ln_b the stored k row is k_norm of the staged row (LayerNorm
 * with bias, biased variance, eps), rounded once to bf16; use then
 * dsa_kpool_compress without ln_w / ln_b.  k_new, gate_new [B, D] bf16; pos
 * [B] i32 (for a decode step, dsa_write_geom's new_from); tok_off [B+1] i32;
 * ln_w, ln_b [D] f32 or both NULL; k, gate [rows, D] bf16, valid [rows] u8.
 * Errors: INVALID_ARG for B < 0, NULL pointers, exactly one of ln_w / ln_b
 * NULL, eps < 0; UNSUPPORTED for D not in {32, 64, 128, 256}.
 *
 * dsa_gate_compress_live: the start of a decode step in one launch, with the
 * results of dsa_write_geom (q_req, q_pos, new_from; no slot), then
 * dsa_indexer_store (pos = new_from), then dsa_gate_compress in incremental
 * mode (new_from, max_new = 1, seq_len).  ln_w / ln_b are required;
 * normed_rows = 0 applies them after pooling (the stored row is raw),
 * normed_rows = 1 to the stored row only (the per-token k_normed form).  The
 * pool that the stored row completes takes that row from registers.  k, gate
 * and valid are written (the stored row); every other argument as in those
 * calls.  Errors: the union of theirs.
 * ------------------------------------------------------------------------- */
dsa_status dsa_write_geom(const int32_t* seq_len, int B, const int32_t* block_table, int bt_stride,
                          int page_rows, int n_pages, int32_t* q_req, int32_t* q_pos,
                          int32_t* new_from, int32_t* slot, hipStream_t stream);
dsa_status dsa_indexer_store(const uint16_t* k_new, const uint16_t* gate_new, const int32_t* pos,
                             const int32_t* tok_off, const float* ln_w, const float* ln_b,
                             float eps, int B, int D, uint16_t* k, uint16_t* gate,
                             uint8_t* valid, hipStream_t stream);
dsa_status dsa_gate_compress_live(const float* hidden, const float* W, int M, int K, int N,
                                  float* gate_part, size_t gate_part_bytes, uint16_t* k,
                                  uint16_t* gate, const uint16_t* ape, uint8_t* valid,
                                  const int32_t* tok_off, const int32_t* pool_off,
                                  const int32_t* seq_len, const uint16_t* k_new,
                                  const uint16_t* gate_new, const float* ln_w, const float* ln_b,
                                  int normed_rows, float eps, int B, int D, int kpool,
                                  int max_cap, uint16_t* keys, int32_t* pool_start,
                                  uint8_t* pool_valid, int32_t* n_pools, int32_t* q_req,
                                  int32_t* q_pos, int32_t* new_from, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Fused decode calls   [stkernel pull request #290 measures what each launch
 *     of a serving step costs; the Atlas page's pipeline order is kept]
 *
 * Three calls that compute a1-a5 with two launches fewer on the critical path;
 * with dsa_sparse_mla_decode they make one decode step:
 *
 *   dsa_gate_compress       a1 (as split-K partials) and a2 in one launch
 *   dsa_index_scores_gated  a3, adding the a1 partials first (writes w)
 *   dsa_topk_expand         a4 and a5 in one launch
 *
 * Results equal those of the separate calls up to the summation order of the
 * head-gate (fixed, so deterministic); every output of the separate calls is
 * still written (w, keys, pool_start, pool_valid, n_pools, scores, cand, sel,
 * tok).
 *
 * dsa_gate_split_count(M, K, N): the number of head-gate partials ns that
 * dsa_gate_compress writes: K / 128 when 1 <= M <= 64, K is a multiple of 128
 * and K / 128 <= 64; otherwise 1, and then the "partials" buffer receives w
 * itself from the dense head-gate.  Returns 0 for N outside [1, 16], M < 0 or
 * K < 1.
 * dsa_gate_compress_workspace_size(M, K, N) = ns * M * N * 4 bytes.
 *
 * dsa_gate_compress: hidden, W, M, K, N as in dsa_head_gate; gate_part
 * [M, ns, N] f32, part[m][s][n] = sum over k in slice s of hidden[m][k] W[k][n]
 * (query-major, so the partials of a run of queries are contiguous; contents
 * on entry are ignored); every other argument as in
 * dsa_kpool_compress (B = 0 runs the head-gate alone).  Errors: those of
 * dsa_kpool_compress and dsa_head_gate, and INVALID_ARG for gate_part_bytes
 * below the size.
 *
 * dsa_index_scores_gated: as dsa_index_scores, with the head weights given as
 * gate_part and nslices = ns (1 <= ns <= 64): w[q, h] = sum over s of
 * gate_part[q][s][h], added in a fixed order, and stored to w [Q, H] f32
 * unless w is NULL.  The gate call's rows are the queries: a call on queries
 * q0 .. q0+Q-1 of a batch passes gate_part + q0*ns*H (and the other per-query
 * arrays offset alike).
 *
 * dsa_topk_expand: dsa_topk_pools followed by dsa_expand_selection on the same
 * rows (arguments as there; sel and tok both written in full).  A row that
 * takes two stages (as there) and whose first-stage candidates (blocks x
 * select_k) fit its tok row keeps them there between the stages (no
 * workspace).  Errors:
 * the union of theirs.
 * ------------------------------------------------------------------------- */
int dsa_gate_split_count(int M, int K, int N);
size_t dsa_gate_compress_workspace_size(int M, int K, int N);
dsa_status dsa_gate_compress(const float* hidden, const float* W, int M, int K, int N,
                             float* gate_part, size_t gate_part_bytes, const uint16_t* k,
                             const uint16_t* gate, const uint16_t* ape, const uint8_t* valid,
                             const int32_t* tok_off, const int32_t* pool_off,
                             const int32_t* seq_len, const float* ln_w,
                             const float* ln_b, float eps, int B, int D, int kpool, int max_cap,
                             const int32_t* new_from, int max_new, uint16_t* keys,
                             int32_t* pool_start, uint8_t* pool_valid, int32_t* n_pools,
                             hipStream_t stream);
dsa_status dsa_index_scores_gated(const uint16_t* qi, const float* gate_part, int nslices,
                                  float* w, const uint16_t* keys, const int32_t* pool_start,
                                  const uint8_t* pool_valid, const int32_t* pool_off,
                                  const int32_t* n_pools, const int32_t* q_req,
                                  const int32_t* q_pos, int Q, int H, int D, int kpool,
                                  int pstride, float* scores, uint8_t* cand, hipStream_t stream);
dsa_status dsa_topk_expand(const float* scores, const uint8_t* cand, const int32_t* row_len,
                           int Q, int pstride, int select_k, const int32_t* pool_start,
                           const int32_t* pool_off, const int32_t* q_req, int kpool,
                           int out_width, int flags, int32_t* sel, int32_t* tok,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * One decode step from one host call   [Atlas page, "Shape of the pipeline"
 *     (the stages and their order); stkernel pull request #227 (the fp32
 *     head-gate whose weights the index scores take)]
 *
 * dsa_decode_step(a, stream) enqueues on `stream`, in this order:
 *   dsa_gate_compress       (N = H, M = Q)
 *   dsa_index_scores_gated  (nslices = dsa_gate_split_count(Q, K, H))
 *   dsa_topk_expand
 *   dsa_select_tail         only when select_tail is nonzero
 *   dsa_sparse_mla_decode   or dsa_sparse_mla_decode_paged when block_table
 *                           is not NULL (kv_off is then unused)
 * with the arguments held in *a, which lives in host memory and is read
 * during the call only (its tensor pointers are device pointers, as in every
 * call).  The results are those of the same calls made one by one, bit for
 * bit.  The step costs one host call instead of four or five, so a host
 * thread keeps the stream's queue ahead of the kernels without a graph.
 * Every argument of every call is checked before anything is launched (each
 * call first runs as a dry run): an error from any of them returns with
 * nothing enqueued, and dsa_last_error() names the call.
 * struct_bytes must be sizeof(dsa_decode_step_args), which
 * dsa_decode_step_args_size() reports, so a binding that lays the struct out
 * itself can check its layout.  Errors: INVALID_ARG for a NULL a, a
 * struct_bytes that differs, or M != Q; then those of the calls.
 * ------------------------------------------------------------------------- */
typedef struct dsa_decode_step_args {
  size_t struct_bytes;
  /* dsa_gate_compress */
  const float* hidden;
  const float* W;
  int M, K, H;
  float* gate_part;
  size_t gate_part_bytes;
  const uint16_t* k;
  const uint16_t* gate;
  const uint16_t* ape;
  const uint8_t* valid;
  const int32_t* tok_off;
  const int32_t* pool_off;
  const int32_t* seq_len;
  const float* ln_w;
  const float* ln_b;
  float eps;
  int B, D, kpool, max_cap;
  const int32_t* new_from;
  int max_new;
  uint16_t* keys;
  int32_t* pool_start;
  uint8_t* pool_valid;
  int32_t* n_pools;
  /* dsa_index_scores_gated */
  const uint16_t* qi;
  float* w;
  const int32_t* q_req;
  const int32_t* q_pos;
  int Q, pstride;
  float* scores;
  uint8_t* cand;
  /* dsa_topk_expand, then dsa_select_tail when select_tail != 0 */
  const int32_t* row_len;
  int select_k, out_width, topk_flags, select_tail;
  int32_t* sel;
  int32_t* tok;
  /* dsa_sparse_mla_decode, or dsa_sparse_mla_decode_paged */
  const uint16_t* q_mla;
  const void* ckv;
  const float* ckv_scale;
  int latent_dtype, Hm, L;
  float sm_scale;
  const int32_t* kv_off;
  uint16_t* out;
  float* lse;
  void* mla_ws;
  size_t mla_ws_bytes;
  const int32_t* block_table;
  int bt_stride, page_rows, n_pages;
  int32_t* kvidx;
} dsa_decode_step_args;
size_t dsa_decode_step_args_size(void);
dsa_status dsa_decode_step(const dsa_decode_step_args* a, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Measurement: the HBM read lane   [stkernel pull request #290, its
 *     measurement ledger: a bandwidth-bound kernel is compared with the rate
 *     of a plain streaming kernel on the same part, and counts as at the
 *     bandwidth floor at 90 % of it or more]
 *
 * dsa_lane_read: reads `bytes` bytes at src (device memory, 16-byte aligned)
 * once with coalesced 16-byte loads; writes at most one word to sink (device,
 * 4 bytes) and only for a value no ordinary fill produces.  Its duration over
 * `bytes` is the lane.  Errors: INVALID_ARG for bytes not a multiple of 16 or
 * NULL pointers with bytes > 0.
 * ------------------------------------------------------------------------- */
dsa_status dsa_lane_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
