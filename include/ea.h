/*
 * ea.h -- C ABI of libea.so: routed hybrid-attention prefill (Elastic Attention) on AMD
 * MI355X (gfx950).
 *
 * The method (web pages on "Elastic Attention: Test-time Adaptive Sparsity Ratios for
 * Efficient Transformers", arXiv:2601.17367):
 *   - Elastic Attention blog post, section 2.1 "Attention Router": a light router reads
 *     the current key hidden states and an MLP emits one routing signal r per head;
 *     r = 0 runs Full Attention, r = 1 runs Sparse Attention; the per-mode outputs are
 *     concatenated.
 *   - same post, section 1: hybrid schemes let some heads attend globally and others only
 *     to a local or sliding window; gist.science explanation, section "问题所在": sparse
 *     reading looks at the first and the last pages only.  This library fixes the sparse
 *     pattern as an attention sink (the first `sink` keys of each sequence) united with a
 *     causal sliding window of `window` keys that ends at the query (diagonal included).
 *   - same post, section 3 "Fused Kernel": the routing decision is handed to a single
 *     kernel as metadata and one launch serves full and sparse heads together.
 *
 * Conventions shared by every entry point
 *   Pointers are DEVICE pointers unless their name ends in _host.  `stream` is a
 *   hipStream_t passed as void* (NULL = the null stream).  Work is enqueued
 *   asynchronously on `stream`; no entry point synchronises the host unless it writes a
 *   *_host output.
 *   Layout is packed token-major ("THD"): sequence b owns tokens
 *   [cu_seqlens[b], cu_seqlens[b+1]) and positions restart at 0 in every sequence;
 *   no token attends across a sequence boundary.  Q and O are [T, n_heads_q, head_dim],
 *   K and V are [T, n_heads_kv, head_dim], contiguous, 16-byte aligned.  Query head h
 *   reads KV head h / (n_heads_q / n_heads_kv).  The output of head h for token t is
 *   written to O[t, h, :], so O viewed as [T, n_heads_q * head_dim] is the concatenation
 *   of the heads.
 *   The caller owns every buffer.  The library allocates no device memory; all scratch
 *   lives in the caller's `workspace` (size from ea_workspace_size).  Calls that share a
 *   workspace must be ordered on one stream.
 *   Errors: every argument check runs on the host before anything is enqueued; on an
 *   error nothing is launched and no output is touched.  HIP failures return
 *   EA_ERR_HIP.  ea_last_error() gives a detail string for the calling thread.
 */
#ifndef EA_H
#define EA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EA_OK = 0,
  EA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned buffer, bad cu_seqlens */
  EA_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement            */
  EA_ERR_WORKSPACE = 3,   /* workspace smaller than ea_workspace_size() demands       */
  EA_ERR_HIP = 4          /* a HIP runtime call failed (detail in ea_last_error())    */
} ea_status;

typedef enum { EA_BF16 = 0, EA_F32 = 1 } ea_dtype;

/*
 * Bytes of workspace that suffice for every entry point below called with these sizes
 * (any dtype, any head_dim).  batch >= 1, max_seqlen >= 0, n_heads_q >= 1; kv_dim and
 * hidden are the router's input and hidden widths (0 if ea_route is not used).
 * Returns 0 if the sizes are invalid.
 */
size_t ea_workspace_size(int32_t batch, int32_t max_seqlen, int32_t n_heads_q, int32_t kv_dim,
                         int32_t hidden);

/*
 * Tile shape of the attention kernel for (dt, head_dim): *bm query rows per work item
 * and *bn keys per key tile.  These fix the work-list items and their costs.
 * Unsupported combinations set both to 0.
 */
void ea_tile_config(ea_dtype dt, int32_t head_dim, int32_t* bm, int32_t* bn);

/* Static text for a status code; never NULL. */
const char* ea_status_string(ea_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char* ea_last_error(void);

/*
 * Attention Router (blog post section 2.1; 0.27M parameters per layer for an 8B model,
 * section 2.2).  For every sequence b:
 *   x_b = mean over the sequence's tokens of key_states[t, :]   (zero vector if empty)
 *   z_b = W2 * SiLU(W1 * x_b + b1) + b2,   SiLU(u) = u / (1 + exp(-u))
 *   route_out[b, h] = (z_b[h] > 0) ? 1 : 0    (1 = sparse, 0 = full; z == 0 is full)
 * key_states  [T, kv_dim], dtype kdt (EA_BF16 or EA_F32); a layer's K viewed as
 *             [T, n_heads_kv * head_dim] is a valid input
 * cu_seqlens  [batch + 1] int32, device
 * w1 [hidden, kv_dim], b1 [hidden], w2 [n_heads_q, hidden], b2 [n_heads_q]: fp32, row-major
 * logits_out  [batch, n_heads_q] fp32 (nullable), route_out [batch, n_heads_q] uint8
 * The mean is accumulated in fp32 in a fixed order (deterministic); the MLP runs in fp32.
 */
ea_status ea_route(const void* key_states, ea_dtype kdt, int32_t kv_dim,
                   const int32_t* cu_seqlens, int32_t batch,
                   const float* w1, const float* b1, int32_t hidden,
                   const float* w2, const float* b2, int32_t n_heads_q,
                   float* logits_out, uint8_t* route_out,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * Work list of the fused launch (blog post section 3: routing reaches the kernel as
 * metadata).  One item per (sequence b, query head h, q-tile j of bm rows), as four
 * int32 {b, h, j, cost}, where cost is the number of bn-key tiles that hold at least one
 * visible (query, key) pair for the item's rows: tiles 0..(m1-1)/bn for a full head,
 * the sink tiles united with the window tiles for a sparse head (rows [m0, m1)).
 * Order: cost descending, ties by (b, j, h) ascending -- longest first, so long full-head
 * items start early and short sparse items fill the tail; sibling heads of one q-tile
 * are adjacent.  The order is unique, so the list is reproducible bit for bit.
 * Limits (the planner runs in one workgroup): batch <= 1024, n_heads_q <= 128 and
 * 2 * batch * ceil(max_seqlen / bm) <= 8192; beyond them EA_ERR_UNSUPPORTED.
 * worklist_out       [worklist_capacity, 4] int32; worklist_capacity (in items) must be at
 *                    least batch * n_heads_q * ceil(max_seqlen / bm), else EA_ERR_INVALID_ARG
 * n_items_out   device int32 (nullable): item count.  n_items_host (nullable): if given,
 *               the call synchronises `stream` and stores the count there.
 * dt, head_dim select (bm, bn) as ea_tile_config.  max_seqlen bounds every sequence.
 */
ea_status ea_build_worklist(const uint8_t* route, const int32_t* cu_seqlens, int32_t batch,
                            int32_t max_seqlen, int32_t n_heads_q, int32_t sink, int32_t window,
                            ea_dtype dt, int32_t head_dim,
                            int32_t* worklist_out, int64_t worklist_capacity,
                            int32_t* n_items_out, int32_t* n_items_host,
                            void* workspace, size_t ws_bytes, void* stream);

/*
 * Routed hybrid-attention prefill in one persistent launch (blog post sections 2.1 and 3).
 * For sequence b, head h, position i (0-based in the sequence), with g the KV head of h:
 *   visible(i) = { j : j <= i }                                     if route[b, h] == 0
 *              = { j : j <= i and (j < sink or j > i - window) }     otherwise
 *   o = sum_{j in visible} softmax_j(scale * <q_i, k_j>) v_j   -> O[cu_seqlens[b] + i, h, :]
 *   lse = log sum_{j in visible} exp(scale * <q_i, k_j>)        -> lse_out[h, cu_seqlens[b] + i]
 * q, k, v, o   dtype dt: EA_BF16 (bf16 MFMA, fp32 accumulation and softmax, P rounded to
 *              bf16 for P*V, O rounded to nearest even) or EA_F32 (fp32 throughout)
 * cu_seqlens       [batch + 1] int32 device; cu_seqlens_host: nullable host copy that
 *                  enables the host-side checks (monotone, starts at 0, lengths <=
 *                  max_seqlen) and the exact aliasing check of o against q, k, v
 * head_dim 64 or 128; n_heads_q % n_heads_kv == 0; sink >= 0; window >= 1;
 * scale <= 0 selects 1/sqrt(head_dim)
 * route        [batch, n_heads_q] uint8 (0 full, nonzero sparse)
 * lse_out      nullable, [n_heads_q, T] fp32
 * worklist_out nullable, receives the work list (see ea_build_worklist) for inspection;
 *              worklist_capacity is its size in items (same bound as ea_build_worklist)
 * o must not overlap q, k or v.  Results do not depend on scheduling: every output
 * element is written by exactly one work item.
 */
ea_status ea_hybrid_attn_prefill(const void* q, const void* k, const void* v, void* o,
                                 ea_dtype dt, const int32_t* cu_seqlens,
                                 const int32_t* cu_seqlens_host, int32_t batch,
                                 int32_t max_seqlen, int32_t n_heads_q, int32_t n_heads_kv,
                                 int32_t head_dim, const uint8_t* route, int32_t sink,
                                 int32_t window, float scale, float* lse_out,
                                 int32_t* worklist_out, int64_t worklist_capacity,
                                 void* workspace, size_t ws_bytes, void* stream);

/*
 * ea_hybrid_attn_prefill for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The same arguments
 * without workspace / ws_bytes, and the same kernels and results.  The queue counters and
 * the internal work list live in a device array of the library (4 MiB per GPU, held until
 * the process ends), whose address is taken once per device; the call allocates nothing.
 * Limit: batch * n_heads_q * ceil(max_seqlen / 64) <= 262128 work items (EA_ERR_UNSUPPORTED
 * beyond it; e.g. 32 heads x 256K tokens x 2 sequences fits).  Every call on one GPU shares
 * the array: calls that overlap on one GPU (other streams, other host threads) race and
 * must be ordered by the caller.  Each call's planner resets what the attention kernel
 * reads, so nothing an earlier call left there is used.
 */
ea_status ea_hybrid_attn_prefill_noalloc(const void* q, const void* k, const void* v, void* o,
                                         ea_dtype dt, const int32_t* cu_seqlens,
                                         const int32_t* cu_seqlens_host, int32_t batch,
                                         int32_t max_seqlen, int32_t n_heads_q,
                                         int32_t n_heads_kv, int32_t head_dim,
                                         const uint8_t* route, int32_t sink, int32_t window,
                                         float scale, float* lse_out, int32_t* worklist_out,
                                         int64_t worklist_capacity, void* stream);

/*
 * Chunked prefill over a KV prefix: the same routed attention when each sequence's queries
 * are only its newest tokens.  Sequence b has Lk = cu_seqlens_k[b+1] - cu_seqlens_k[b]
 * positions whose keys and values are k, v [Tk, n_heads_kv, head_dim] (an earlier prefix,
 * e.g. cached, followed by the new chunk), and Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] <= Lk
 * queries q [Tq, n_heads_q, head_dim], the last Lq positions: query row r of the chunk sits
 * at position i = Lk - Lq + r and sees, under its head's mode, the keys j <= i visible to
 * position i exactly as in ea_hybrid_attn_prefill.  o [Tq, n_heads_q, head_dim];
 * lse_out [n_heads_q, Tq].  With cu_seqlens_k equal to cu_seqlens_q this is
 * ea_hybrid_attn_prefill.  max_seqlen_q <= max_seqlen_k bound the two packings (per-sequence
 * key windows need max_seqlen_k * n_heads_kv * head_dim * elem < 2^31).
 * cu_seqlens_q_host / cu_seqlens_k_host: give both (host copies, checked: monotone, within
 * the bounds, Lq <= Lk per sequence, o not overlapping q, k, v) or neither.  On the device
 * a sequence with Lk < Lq gets no work and its output rows are not written.  Other
 * arguments and worklist_out as for ea_hybrid_attn_prefill, with max_seqlen_q in place of
 * max_seqlen for the work list bound.  workspace: at least
 * ea_prefill_chunked_workspace_size(batch, max_seqlen_q, n_heads_q, head_dim) bytes.
 * bf16 runs split-KV: a work item whose key-tile cost exceeds a budget set from the total
 * cost and the device's workgroup count runs as up to 16 pieces over consecutive parts of its
 * tiles, on different workgroups, and a third launch merges their fp32 partial results; the
 * work list (worklist_out) is the same as without splitting.
 */
/*
 * Bytes of workspace ea_hybrid_attn_prefill_chunked needs: the work list and its counters
 * plus, for split-KV, 512 partial-result slots of 256 rows x head_dim fp32 (64 MiB at
 * head_dim 128).  0 if the sizes overflow.
 */
size_t ea_prefill_chunked_workspace_size(int32_t batch, int32_t max_seqlen_q, int32_t n_heads_q,
                                         int32_t head_dim);

ea_status ea_hybrid_attn_prefill_chunked(
    const void* q, const void* k, const void* v, void* o, ea_dtype dt,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* cu_seqlens_q_host,
    const int32_t* cu_seqlens_k_host, int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, const uint8_t* route, int32_t sink,
    int32_t window, float scale, float* lse_out, int32_t* worklist_out,
    int64_t worklist_capacity, void* workspace, size_t ws_bytes, void* stream);

/*
 * The attention half of ea_hybrid_attn_prefill on a work list made by ea_build_worklist
 * (same dt, head_dim, sink, window, route and cu_seqlens).  worklist and n_items are
 * device pointers; worklist_capacity is the work list's size in items (the kernels never
 * read past min(*n_items, worklist_capacity), and skip items that name a sequence, head
 * or q-tile outside the call's sizes).  grid_blocks sets the number of persistent workgroups (0 = one per
 * resident slot on the device); the output does not depend on it.
 * The workgroups take items through two queue counters kept in the workspace: they are
 * zeroed by ea_build_worklist and ea_hybrid_attn_prefill and left at zero by every
 * completed run, so pass a workspace that has been through one of those calls.  No other
 * entry point writes them (ea_route's scratch lies past them), so ea_route may run on the
 * same workspace between ea_build_worklist and this call.  A queue head outside
 * [0, n_items) ends every workgroup's loop: nothing is read outside the work list.
 */
ea_status ea_hybrid_attn_run(const void* q, const void* k, const void* v, void* o, ea_dtype dt,
                             const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                             int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                             const uint8_t* route, int32_t sink, int32_t window, float scale,
                             float* lse_out, const int32_t* worklist,
                             int64_t worklist_capacity, const int32_t* n_items,
                             int32_t grid_blocks, void* workspace, size_t ws_bytes,
                             void* stream);

/*
 * Bytes of workspace ea_hybrid_attn_decode needs for these sizes: per-split partial
 * results, batch * n_heads_q * ceil(max_seqlen / 256) * (head_dim + 2) floats.
 * batch >= 1, max_seqlen >= 1, n_heads_q >= 1, head_dim >= 1; 0 if the sizes overflow.
 */
size_t ea_decode_workspace_size(int32_t batch, int32_t max_seqlen, int32_t n_heads_q,
                                int32_t head_dim);

/*
 * One decode step of the routed hybrid attention (blog post section 2.1: r = 0 runs Full
 * Attention, r = 1 Sparse Attention; sparse pattern as above).  Sequence b holds
 * L = seqlens[b] tokens in its KV cache, the newest being the query's own token, and every
 * query head attends from position i = L - 1 exactly as a prefill row at position i:
 *   visible = { j < L }                                   if route[b, h] == 0
 *           = { j < L : j < sink or j > i - window }       otherwise
 *   o = sum_{j in visible} softmax_j(scale * <q, k_j>) v_j   -> O[b, h, :]
 *   lse = log sum_{j in visible} exp(scale * <q, k_j>)      -> lse_out[b, h]
 * q, o         [batch, n_heads_q, head_dim], dtype dt (EA_BF16 or EA_F32; fp32
 *              arithmetic, O rounded once to dt)
 * k_cache, v_cache  [batch, cache_capacity, n_heads_kv, head_dim], dtype dt; only the
 *              first seqlens[b] slots of sequence b are read (and of them, for a KV head
 *              whose query heads are all sparse, only the visible ones)
 * seqlens      [batch] int32 device; each must lie in [1, min(cache_capacity, max_seqlen)]
 *              (a sequence outside that range gets NaN outputs and no cache reads beyond
 *              its slots).  seqlens_host: nullable host copy that enables the host check.
 * head_dim 64 or 128; n_heads_q % n_heads_kv == 0 with at most 8 query heads per KV head;
 * sink >= 0; window >= 1; scale <= 0 selects 1/sqrt(head_dim)
 * route        [batch, n_heads_q] uint8 (0 full, nonzero sparse)
 * lse_out      nullable, [batch, n_heads_q] fp32
 * workspace    at least ea_decode_workspace_size(batch, max_seqlen, n_heads_q, head_dim)
 *              bytes, 256-byte aligned; o must not overlap q or the caches
 * Two launches: per (KV-cache split of 256 keys, KV head, sequence) partial results, then
 * their combination; results do not depend on scheduling.
 */
ea_status ea_hybrid_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                void* o, ea_dtype dt, const int32_t* seqlens,
                                const int32_t* seqlens_host, int32_t batch,
                                int32_t cache_capacity, int32_t max_seqlen, int32_t n_heads_q,
                                int32_t n_heads_kv, int32_t head_dim, const uint8_t* route,
                                int32_t sink, int32_t window, float scale, float* lse_out,
                                void* workspace, size_t ws_bytes, void* stream);

/*
 * Pooled KV cache for decode.  A KV head whose query heads are all sparse only ever needs
 * the sink keys and the last `window` keys (the sparse pattern above), so its cache can be a
 * sink + ring buffer of sink + window rows instead of a full history; this is where the
 * hybrid routing saves decode memory.  The pool is one array of rows per tensor,
 * k_pool / v_pool [pool_rows, head_dim], dtype dt; the rows of (sequence b, KV head h) form
 * the region region_base[b * n_heads_kv + h] .. + region_rows[...] (int64 / int32, device
 * for the kernels):
 *   linear region (some query head of h is full, route == 0): position j at row j;
 *   ring region (every query head of h is sparse): position j < sink at row j, position
 *     j >= sink at row sink + (j - sink) % window; it needs sink + window rows.
 * The routing must be the one the regions were laid out for.
 */

/*
 * Host-only layout of a pool: for route_host [batch, n_heads_q] (uint8, host), linear
 * regions of `capacity` rows and ring regions of sink + window rows, packed in (b, h) order
 * from row 0.  Writes region_base_host / region_rows_host [batch * n_heads_kv] and
 * *total_rows_host (the pool_rows to allocate).  batch >= 1, capacity >= 1, sink >= 0,
 * window >= 1, n_heads_q a multiple of n_heads_kv.
 */
ea_status ea_decode_pool_layout(const uint8_t* route_host, int32_t batch, int32_t n_heads_q,
                                int32_t n_heads_kv, int32_t capacity, int32_t sink,
                                int32_t window, int64_t* region_base_host,
                                int32_t* region_rows_host, int64_t* total_rows_host);

/*
 * Prefill K/V into the pool: k, v [T, n_heads_kv, head_dim] packed as cu_seqlens [batch+1]
 * (max_seqlen >= every length).  A linear region receives every position (those past its
 * rows are dropped); a ring region receives the positions a decode query at position L can
 * see besides its own: j < sink and j >= L - window, L the sequence length.  A region outside
 * the pool or beyond 2^31 bytes is skipped (the decode then gives NaN for it).  head_dim 64
 * or 128; at most 8 query heads per KV head; k, v, pools 16-byte aligned.
 */
ea_status ea_decode_pool_fill(const void* k, const void* v, ea_dtype dt, const int32_t* cu_seqlens,
                              int32_t batch, int32_t max_seqlen, int32_t n_heads_q,
                              int32_t n_heads_kv, int32_t head_dim, const uint8_t* route,
                              int32_t sink, int32_t window, const int64_t* region_base,
                              const int32_t* region_rows, int64_t pool_rows, void* k_pool,
                              void* v_pool, void* stream);

/*
 * Append one token per sequence: k_new, v_new [batch, n_heads_kv, head_dim] go to position
 * positions[b] (int32 device; the new length minus one) of every region of sequence b; in a
 * ring the row of position j - window is reused, which no later query can see.  A negative
 * position, a row past the region or an unusable region writes nothing.  Call it before
 * ea_hybrid_attn_decode_pool for that token (the query's own key is part of its cache).
 */
ea_status ea_decode_pool_append(const void* k_new, const void* v_new, ea_dtype dt,
                                const int32_t* positions, int32_t batch, int32_t n_heads_q,
                                int32_t n_heads_kv, int32_t head_dim, const uint8_t* route,
                                int32_t sink, int32_t window, const int64_t* region_base,
                                const int32_t* region_rows, int64_t pool_rows, void* k_pool,
                                void* v_pool, void* stream);

/*
 * ea_hybrid_attn_decode over a pooled cache: the same outputs (O and LSE of position
 * seqlens[b] - 1 of every query head) with keys read from the regions above.  A region that
 * cannot serve its query (outside the pool, over 2^31 bytes, a linear region shorter than
 * the sequence, a ring shorter than sink + window) gives NaN outputs for that KV head's
 * query heads and is not read; lengths outside [1, max_seqlen] give NaN for the sequence.
 * Workspace: ea_decode_workspace_size(batch, max_seqlen, n_heads_q, head_dim) bytes,
 * 256-byte aligned.  Other arguments as for ea_hybrid_attn_decode.
 */
ea_status ea_hybrid_attn_decode_pool(const void* q, const void* k_pool, const void* v_pool,
                                     void* o, ea_dtype dt, const int32_t* seqlens,
                                     const int32_t* seqlens_host, int32_t batch,
                                     int32_t max_seqlen, int32_t n_heads_q, int32_t n_heads_kv,
                                     int32_t head_dim, const int64_t* region_base,
                                     const int32_t* region_rows, int64_t pool_rows,
                                     const uint8_t* route, int32_t sink, int32_t window,
                                     float scale, float* lse_out, void* workspace,
                                     size_t ws_bytes, void* stream);

/*
 * Training: backward of the routed attention (blog post section 2.1, "training trick": the
 * model learns through its routed attention, so gradients flow through the full heads and
 * the sparse heads alike; masks as in ea_hybrid_attn_prefill).  With P the forward's softmax
 * (recomputed from lse: P_ij = exp(scale <q_i, k_j> - lse_i)) and dO the gradient of O,
 *   D_i = <dO_i, O_i>,  dS_ij = P_ij (<dO_i, v_j> - D_i)   for visible (i, j),
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dO_i,
 * dk and dv summed over the query heads of a KV head.  The hard routing passes gradients
 * only through the branch each head took.
 * q, o, dout   [Tq, n_heads_q, head_dim] and k, v [Tk, n_heads_kv, head_dim], dtype dt
 *              (EA_BF16 or EA_F32), packed as cu_seqlens_q / cu_seqlens_k [batch + 1]
 *              (device int32; cu_seqlens_k NULL = cu_seqlens_q, a plain prefill; else chunk
 *              row r of sequence b sits at position Lk - Lq + r, as in
 *              ea_hybrid_attn_prefill_chunked)
 * lse          [n_heads_q, Tq] fp32, the forward's lse_out for the same inputs
 * cu_seqlens_q_host / cu_seqlens_k_host: nullable host copies (both or neither; with
 *              cu_seqlens_k NULL, pass cu_seqlens_q_host alone) that enable the host checks
 *              of the packings and of buffer overlaps
 * dq [Tq, n_heads_q, head_dim], dk, dv [Tk, n_heads_kv, head_dim]: fp32 outputs, every
 *              element written (a key no row can see gets 0); they must not overlap the
 *              inputs or each other
 * head_dim 64 or 128; sink >= 0; window >= 1; scale <= 0 selects 1/sqrt(head_dim);
 * batch and n_heads_q at most 65535; all tensors 16-byte aligned; for EA_BF16 one
 * sequence's rows of q at most 2^31 bytes (max_seqlen_k * n_heads_q * head_dim * 2; 256K
 * tokens at 32 x 128), else EA_ERR_UNSUPPORTED
 * workspace    ea_attn_backward_workspace_size(dt, batch, max_seqlen_q, max_seqlen_k,
 *              n_heads_q, n_heads_kv, head_dim) bytes, 256-byte aligned: the D_i values; for
 *              EA_BF16 also lse in base-2 units and, with several query heads per KV head, the
 *              per-query-head fp32 partials of dk and dv (2 * batch * max_seqlen_k * n_heads_q
 *              * head_dim * 4 bytes)
 * EA_BF16: products on the matrix cores (bf16 operands: the inputs, and P and dS rounded to
 * bf16; fp32 accumulation); EA_F32: fp32 arithmetic throughout.  Fixed summation orders
 * (deterministic, no atomics).  Launches: D; dq per (q-tile, query head, sequence); dk and dv
 * per (key tile, KV head or, for EA_BF16, query head, sequence); for EA_BF16 with several
 * query heads per KV head a reduce adding the partials in head order.  A device packing that breaks the bounds above (a sequence longer than
 * its max_seqlen, a chunk longer than its keys) leaves that sequence's gradients unwritten;
 * the host copies turn it into EA_ERR_INVALID_ARG.
 */
size_t ea_attn_backward_workspace_size(ea_dtype dt, int32_t batch, int32_t max_seqlen_q,
                                       int32_t max_seqlen_k, int32_t n_heads_q,
                                       int32_t n_heads_kv, int32_t head_dim);

ea_status ea_hybrid_attn_backward(
    const void* q, const void* k, const void* v, const void* o, const void* dout, ea_dtype dt,
    const float* lse, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host, int32_t batch,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_heads_q, int32_t n_heads_kv,
    int32_t head_dim, const uint8_t* route, int32_t sink, int32_t window, float scale,
    float* dq, float* dk, float* dv, void* workspace, size_t ws_bytes, void* stream);

/*
 * Training: gradient of the Attention Router through its straight-through decision (blog
 * post section 2.1, "training trick": Gumbel-Softmax with a straight-through estimator).
 * The forward routes with the hard r = (z + g > 0) and head h outputs
 * r O_sparse + (1 - r) O_full; the backward uses r_soft = sigmoid((z + g) / tau):
 *   dr[b, h] = sum over the rows t of sequence b of <dout[t, h], O_sparse[t, h] - O_full[t, h]>
 *   dz = dr r_soft (1 - r_soft) / tau
 * then the router MLP of ea_route (z = W2 SiLU(W1 x + b1) + b2, x the mean of the key states)
 * backward: dw2 = dz^T hs, db2 = sum_b dz, du = (dz W2) SiLU'(u), dw1 = du^T x,
 * db1 = sum_b du, and dkey_states[t] = (du W1)[b] / n_b for the n_b rows t of sequence b
 * (an empty sequence gets no rows).
 * key_states, cu_seqlens, w1, b1, w2, b2, kv_dim, hidden, n_heads_q: as for ea_route
 * o_full, o_sparse, dout  [T, n_heads_q, head_dim], dtype odt: the layer's output with every
 *              head full (route all 0) and every head sparse (route all 1), and the gradient
 *              of the routed output; head_dim 64 or 128
 * noise        nullable [batch, n_heads_q] fp32: the logistic noise g of the draw (NULL = 0)
 * tau          temperature, > 0
 * dr_out       nullable [batch, n_heads_q]; dz_out [batch, n_heads_q]; dw1 [hidden, kv_dim];
 *              db1 [hidden]; dw2 [n_heads_q, hidden]; db2 [n_heads_q]: fp32 outputs
 * dkey_states  nullable [T, kv_dim] fp32 (needs kv_dim % 4 == 0 and 16-byte alignment)
 * workspace    ea_route_backward_workspace_size(batch, kv_dim, hidden, n_heads_q, head_dim)
 *              bytes, 256-byte aligned
 * Ten short launches in fixed summation orders (deterministic); the dr reduction streams the
 * three [T, n_heads_q, head_dim] tensors once.
 */
size_t ea_route_backward_workspace_size(int32_t batch, int32_t kv_dim, int32_t hidden,
                                        int32_t n_heads_q, int32_t head_dim);

ea_status ea_route_backward(const void* key_states, ea_dtype kdt, int32_t kv_dim,
                            const int32_t* cu_seqlens, int32_t batch, const float* w1,
                            const float* b1, int32_t hidden, const float* w2, const float* b2,
                            int32_t n_heads_q, const void* o_full, const void* o_sparse,
                            const void* dout, ea_dtype odt, int32_t head_dim, const float* noise,
                            float tau, float* dr_out, float* dz_out, float* dw1, float* db1,
                            float* dw2, float* db2, float* dkey_states, void* workspace,
                            size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EA_H */
