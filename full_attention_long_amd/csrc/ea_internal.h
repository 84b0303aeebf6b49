// ea_internal.h -- shared declarations of libea's host layer and its HIP kernels.
// Not installed; the public ABI is include/ea.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ea {

// ---------------------------------------------------------------- tile shapes
// bf16 path: 8 wavefronts x 32 query rows = 256-row q-tiles, 64-key tiles.
// fp32 path: 64-row q-tiles, 32-key tiles.
constexpr int kBf16BM = 256;
constexpr int kBf16BN = 64;
constexpr int kF32BM = 64;
constexpr int kF32BN = 32;
constexpr int kMinBM = 64;           // smallest q-tile over all paths (sizes the work list)
// The planner keeps its whole state in the LDS of one workgroup:
constexpr int kPlanMaxCells = 8192;  // 2 cells per (sequence, q-tile)
constexpr int kPlanMaxBatch = 1024;  // sequences per call
constexpr int kPlanMaxHeads = 128;   // query heads
// Split-KV for the bf16 chunked prefill: a work item whose key-tile cost exceeds a budget is
// run as up to kSplitMaxPieces pieces over consecutive parts of its tile plan, each writing
// fp32 partial results to one of kSplitSlots slots, merged afterwards.
constexpr int kSplitMaxPieces = 16;
constexpr int kSplitSlots = 512;
constexpr int kSplitMinTiles = 32;   // smallest budget (tiles per piece)

// ---------------------------------------------------------------- workspace
struct WsLayout {
  // the router's scratch overlays the start of the workspace (see ws_layout)
  int router_chunks = 0;
  size_t router_partial = 0;  // float [batch][router_chunks][kv_dim]
  size_t router_x = 0;        // float [batch][kv_dim]   pooled key states
  size_t router_h = 0;        // float [batch][hidden]   SiLU(W1 x + b1)
  size_t items = 0;           // int4 [batch * n_heads_q * qt_max] (internal work list)
  size_t counters = 0;        // int32 [16]: 0 n_items, 1 queue head, 2 workgroups done,
                              // 3 pieces (split-KV), 4 split items
  // split-KV (only laid out by ws_layout_split)
  size_t piece_prefix = 0;    // int32 [item_cap + 1]: first piece of every item
  size_t slot_base = 0;       // int32 [item_cap]: first partial slot of a split item, else -1
  size_t split_list = 0;      // int32 [kSplitSlots]: the split items
  size_t o_part = 0;          // float [kSplitSlots][BM][head_dim] unnormalised partial O
  size_t ml_part = 0;         // float [kSplitSlots][BM][2] partial row max (score units), sum
  size_t total = 0;
  int64_t item_cap = 0;
};

// Returns false if the sizes overflow what the layout can describe.
bool ws_layout(int32_t batch, int32_t max_seqlen, int32_t n_heads_q, int32_t kv_dim,
               int32_t hidden, WsLayout* out);
// ws_layout plus the split-KV buffers of the bf16 chunked prefill.
bool ws_layout_split(int32_t batch, int32_t max_seqlen_q, int32_t n_heads_q, int32_t head_dim,
                     WsLayout* out);

int router_chunks(int32_t batch);

// ---------------------------------------------------------------- launches
// Each returns the hipError_t of its launch.
hipError_t launch_route(const void* ks, int kdt, int kv_dim, const int32_t* cu, int batch,
                        const float* w1, const float* b1, int hidden, const float* w2,
                        const float* b2, int n_heads_q, float* logits, uint8_t* route,
                        float* partial, int chunks, float* x, float* hv, hipStream_t stream);

struct PlanArgs {
  const uint8_t* route;
  const int32_t* cu;
  // nullable: key packing of a chunked prefill over a KV prefix (sequence b's cu[b+1]-cu[b]
  // queries are the last of its cu_k[b+1]-cu_k[b] positions); null = cu
  const int32_t* cu_k;
  int batch, n_heads_q, sink, window, bm, bn;
  int4* items;
  int32_t item_cap;       // items the list can hold
  int32_t* counters;      // [0] n_items, [1] queue head, [2] workgroups done (both zeroed)
  int32_t* n_items_out;   // nullable
  // split-KV (split_workers > 0): budget from the total cost and this many workgroups
  int split_workers;
  int32_t* piece_prefix;  // [n_items + 1]
  int32_t* slot_base;     // [n_items]
  int32_t* split_list;    // [kSplitSlots]
};
hipError_t launch_plan(const PlanArgs& a, hipStream_t stream);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* cu;
  const int32_t* cu_k;    // nullable, as in PlanArgs
  const uint8_t* route;
  const int4* items;
  const int32_t* n_items;
  int32_t item_cap;       // never read items[item_cap] or beyond
  int32_t* queue;         // [0] queue head, [1] workgroups done; zero on entry, re-zeroed
                          // by the last workgroup to finish
  float* lse;
  int batch, n_heads_q, n_heads_kv, head_dim, sink, window;
  float scale;
  // split-KV (piece_prefix non-null; bf16 kernel only): the queue hands out pieces, counters
  // [3] = number of pieces; piece p of item i (p - piece_prefix[i] of the item's
  // piece_prefix[i+1] - piece_prefix[i]) runs its share of the item's tile plan and, when the
  // item has more than one piece, writes partial results to slot slot_base[i] + piece
  const int32_t* piece_prefix;
  const int32_t* slot_base;
  const int32_t* n_pieces;
  float* o_part;
  float* ml_part;
};
hipError_t launch_attn_bf16(const AttnArgs& a, int grid, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs& a, int grid, hipStream_t stream);
// Merge of the split items' partial results (after launch_attn_bf16 with split-KV): one
// workgroup per split item (counters[4] of them), O rounded to bf16 and the LSE written.
hipError_t launch_split_combine(const AttnArgs& a, const int32_t* split_list,
                                const int32_t* n_split, hipStream_t stream);
// One decode step (ea_decode.hip): per-split partial results in the workspace, then a
// combine.  kDecodeSplit keys per split; group sizes up to kDecodeMaxGroup.
constexpr int kDecodeSplit = 256;
constexpr int kDecodeMaxGroup = 8;
struct DecodeArgs {
  const void* q;          // [batch, n_heads_q, head_dim]
  const void* kc;         // dense: [batch, cap, n_heads_kv, head_dim]; pooled: [pool_rows, head_dim]
  const void* vc;
  // pooled cache (pooled != 0): the rows of (sequence b, KV head h) start at row
  // region_base[b * n_heads_kv + h] of the pool and number region_rows[...]; a KV head with a
  // full query head keeps position j at row j, one whose query heads are all sparse keeps
  // the sink and a ring of `window` rows (position j >= sink at row sink + (j - sink) % window)
  const int64_t* region_base;
  const int32_t* region_rows;
  int64_t pool_rows;
  int pooled;
  void* o;                // [batch, n_heads_q, head_dim]
  const int32_t* seqlens; // [batch]
  const uint8_t* route;   // [batch, n_heads_q]
  float* o_part;          // [batch, n_heads_q, max_splits, head_dim]
  float* ml_part;         // [batch, n_heads_q, max_splits, 2]: split max (log2 units), sum
  float* lse;             // [batch, n_heads_q] or null
  int batch, cap, max_seqlen, max_splits, n_heads_q, n_heads_kv, head_dim, sink, window;
  float scale;
};
hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream);
// Pooled cache writers (ea_decode.hip).  fill: prefill K/V [T, n_heads_kv, head_dim] of
// packed sequences (cu) into their regions, every row the next decode step can see;
// append: one new row per (sequence, KV head) at position positions[b].
struct PoolWriteArgs {
  const void* k;          // fill: [T, n_heads_kv, head_dim]; append: [batch, n_heads_kv, head_dim]
  const void* v;
  const int32_t* cu;      // fill: [batch + 1]
  const int32_t* positions;  // append: [batch]
  const uint8_t* route;   // [batch, n_heads_q]
  const int64_t* region_base;
  const int32_t* region_rows;
  void* k_pool;
  void* v_pool;
  int64_t pool_rows;
  int batch, max_seqlen, n_heads_q, n_heads_kv, head_dim, sink, window;
};
// Backward of the router through its straight-through decision (ea_router.hip).
struct RouteBwdArgs {
  const void* key_states;  // [T, kv_dim], kdt
  const int32_t* cu;       // [batch + 1]
  const float *w1, *b1, *w2, *b2;
  const void *o_full, *o_sparse, *dout;  // [T, n_heads_q, head_dim], odt
  const float* noise;      // nullable [batch, n_heads_q]
  float tau;
  int kdt, odt, batch, kv_dim, hidden, n_heads_q, head_dim, pool_chunks, dr_chunks;
  // workspace
  float *pool_partial, *x, *u, *hs, *dr_partial, *du, *dx;
  // outputs
  float *dr, *dz, *dw1, *db1, *dw2, *db2, *dkey_states;
};
int route_bwd_chunks(int32_t batch, int32_t width);
hipError_t launch_route_backward(const RouteBwdArgs& a, hipStream_t stream);

// Backward of the routed attention (ea_backward.hip).
struct BwdArgs {
  const void* q;          // [Tq, n_heads_q, head_dim]
  const void* k;          // [Tk, n_heads_kv, head_dim]
  const void* v;
  const void* o;          // forward output [Tq, n_heads_q, head_dim]
  const void* dout;       // [Tq, n_heads_q, head_dim]
  const float* lse;       // forward log-sum-exp [n_heads_q, Tq]
  const int32_t* cu_q;    // [batch + 1]
  const int32_t* cu_k;    // [batch + 1] (the same as cu_q for a plain prefill)
  const uint8_t* route;   // [batch, n_heads_q]
  float* delta;           // workspace [n_heads_q, Tq]
  float* lse2;            // workspace [n_heads_q, Tq]: lse * log2(e) (bf16 path; else null)
  float* dq;              // [Tq, n_heads_q, head_dim]
  float* dk;              // [Tk, n_heads_kv, head_dim]
  float* dv;
  int64_t tq_cap;         // rows the delta workspace holds per head (batch * max_seqlen_q)
  int64_t tk_cap;         // key rows a dk/dv partial holds (batch * max_seqlen_k)
  float* dk_part;         // bf16 path with n_heads_q > n_heads_kv: per-query-head partials
  float* dv_part;         // [group][tk_cap][n_heads_kv][head_dim], summed by a reduce kernel
  int batch, max_seqlen_q, max_seqlen_k, n_heads_q, n_heads_kv, head_dim, sink, window;
  float scale;
};
hipError_t launch_attn_backward(const BwdArgs& a, bool bf16, hipStream_t stream);
// dq and dk/dv of bf16 inputs on the matrix cores (ea_backward_bf16.hip); D already computed.
hipError_t launch_attn_backward_bf16_mfma(const BwdArgs& a, hipStream_t stream);

hipError_t launch_pool_fill(const PoolWriteArgs& a, int elem_bytes, hipStream_t stream);
hipError_t launch_pool_append(const PoolWriteArgs& a, int elem_bytes, hipStream_t stream);

// Workgroups of each attention kernel that fit on one CU at once.
int attn_bf16_blocks_per_cu();
int attn_f32_blocks_per_cu();

}  // namespace ea
