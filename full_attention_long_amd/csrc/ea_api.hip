// ea_api.hip -- host side of libea.so: the C ABI declared in include/ea.h.
//
// Every argument is checked here, on the host, before anything is enqueued, so a
// rejected call launches nothing and leaves every output untouched.  The library never
// allocates device memory: the router partial sums, the planner's cells and the work
// list live in the caller's workspace, carved by ws_layout().
#include <atomic>
#include <math.h>
#include <mutex>
#include <string.h>

#include <string>

#include "../../include/ea.h"
#include "ea_internal.h"

namespace ea {

namespace {

thread_local std::string g_last_error;

ea_status fail(ea_status s, const std::string& why) {
  g_last_error = why;
  return s;
}

ea_status hip_fail(hipError_t e, const char* where) {
  return fail(EA_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// A window longer than every sequence hides nothing: clamping it to max_len + 1 keeps the
// mask and keeps the kernels' position arithmetic (i - window, j + window) inside 32 bits.
int32_t clamp_window(int32_t window, int64_t max_len) {
  return (int32_t)(window < max_len + 1 ? window : max_len + 1);
}

bool tile_shape(ea_dtype dt, int32_t head_dim, int* bm, int* bn) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (dt == EA_BF16) {
    *bm = kBf16BM;
    *bn = kBf16BN;
    return true;
  }
  if (dt == EA_F32) {
    *bm = kF32BM;
    *bn = kF32BN;
    return true;
  }
  return false;
}

constexpr int kMaxDevices = 64;
// per-device compute-unit count, filled on first use; calls from several host threads may
// race to fill an entry, all with the same value, so relaxed atomics suffice
std::atomic<int> g_cu_count[kMaxDevices];

hipError_t cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *out = cached;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return hipSuccess;
}

// Upper bound on the number of work items for these sizes.
int64_t item_bound(int32_t batch, int32_t max_seqlen, int32_t n_heads_q, int bm) {
  return (int64_t)batch * n_heads_q * ceil_div64(max_seqlen, bm);
}

// The planner holds its state in one workgroup's LDS: bound the cells, sequences, heads.
ea_status check_plan_limits(int32_t batch, int32_t max_seqlen, int32_t n_heads_q, int bm) {
  if (batch > kPlanMaxBatch) return fail(EA_ERR_UNSUPPORTED, "more than 1024 sequences");
  if (n_heads_q > kPlanMaxHeads) return fail(EA_ERR_UNSUPPORTED, "more than 128 query heads");
  if (2 * (int64_t)batch * ceil_div64(max_seqlen, bm) > kPlanMaxCells)
    return fail(EA_ERR_UNSUPPORTED, "batch * ceil(max_seqlen / bm) exceeds 4096 q-tiles");
  return EA_OK;
}

// Checks shared by the attention entry points.  Fills bm/bn.  max_seqlen bounds the key
// sequences (32-bit per-sequence addressing); plan_seqlen bounds the query rows the planner
// tiles (the chunk length of a chunked prefill, else max_seqlen).
ea_status check_attn_args(const void* q, const void* k, const void* v, void* o, ea_dtype dt,
                          const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                          int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                          const uint8_t* route, int32_t sink, int32_t window, float scale,
                          void* workspace, int* bm, int* bn, int32_t plan_seqlen = -1) {
  if (!q || !k || !v || !o || !cu_seqlens || !route || !workspace)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (dt != EA_BF16 && dt != EA_F32) return fail(EA_ERR_INVALID_ARG, "unknown dtype");
  if (batch < 1 || max_seqlen < 0) return fail(EA_ERR_INVALID_ARG, "batch < 1 or max_seqlen < 0");
  if (n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv != 0)
    return fail(EA_ERR_INVALID_ARG, "n_heads_q must be a positive multiple of n_heads_kv");
  if (sink < 0 || window < 1) return fail(EA_ERR_INVALID_ARG, "need sink >= 0 and window >= 1");
  if (isnan(scale) || isinf(scale)) return fail(EA_ERR_INVALID_ARG, "scale is not finite");
  if (!tile_shape(dt, head_dim, bm, bn))
    return fail(EA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(EA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (o == q || o == k || o == v) return fail(EA_ERR_INVALID_ARG, "o aliases q, k or v");
  const int64_t elem = dt == EA_BF16 ? 2 : 4;
  // per-sequence K/V windows and per-item Q/O windows use 32-bit byte offsets
  if ((int64_t)max_seqlen * n_heads_kv * head_dim * elem >= ((int64_t)1 << 31) ||
      (int64_t)(*bm + 1) * n_heads_q * head_dim * elem >= ((int64_t)1 << 31))
    return fail(EA_ERR_UNSUPPORTED, "sequence too long for 32-bit per-sequence addressing");
  return check_plan_limits(batch, plan_seqlen < 0 ? max_seqlen : plan_seqlen, n_heads_q, *bm);
}

ea_status check_cu_host(const int32_t* cu, int32_t batch, int32_t max_seqlen) {
  if (cu[0] != 0) return fail(EA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = (int64_t)cu[b + 1] - cu[b];
    if (len < 0) return fail(EA_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing");
    if (len > max_seqlen) return fail(EA_ERR_INVALID_ARG, "a sequence is longer than max_seqlen");
  }
  return EA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

ea_status enqueue_plan(const uint8_t* route, const int32_t* cu, int32_t batch,
                       int32_t max_seqlen, int32_t n_heads_q, int32_t sink, int32_t window,
                       int bm, int bn, int4* items, int64_t item_cap, int32_t* n_items_out,
                       const WsLayout& L, char* ws, hipStream_t stream,
                       const int32_t* cu_k = nullptr, int split_workers = 0) {
  PlanArgs p{};
  // the planner writes nothing past this many items (nor past its LDS cells): device lengths
  // beyond max_seqlen give an empty work list instead
  if (split_workers > 0 && item_cap > L.item_cap) item_cap = L.item_cap;
  p.item_cap = (int32_t)(item_cap < INT32_MAX ? item_cap : INT32_MAX);
  if (split_workers > 0) {
    p.split_workers = split_workers;
    p.piece_prefix = (int32_t*)(ws + L.piece_prefix);
    p.slot_base = (int32_t*)(ws + L.slot_base);
    p.split_list = (int32_t*)(ws + L.split_list);
  }
  p.route = route;
  p.cu = cu;
  p.cu_k = cu_k;
  p.batch = batch;
  p.n_heads_q = n_heads_q;
  p.sink = sink;
  p.window = window;
  p.bm = bm;
  p.bn = bn;
  p.items = items;
  p.counters = (int32_t*)(ws + L.counters);
  p.n_items_out = n_items_out;
  hipError_t e = launch_plan(p, stream);
  if (e != hipSuccess) return hip_fail(e, "planner launch");
  return EA_OK;
}

ea_status enqueue_attn(const void* q, const void* k, const void* v, void* o, ea_dtype dt,
                       const int32_t* cu, int32_t batch, int32_t n_heads_q, int32_t n_heads_kv,
                       int32_t head_dim, const uint8_t* route, int32_t sink, int32_t window,
                       float scale, float* lse, const int4* items, const int32_t* n_items,
                       int64_t item_cap, int32_t* queue, int grid_blocks, hipStream_t stream,
                       const int32_t* cu_k = nullptr, const WsLayout* split = nullptr,
                       char* ws = nullptr) {
  AttnArgs a{};
  if (split) {  // split-KV: pieces from the planner's split phase, then the combine launch
    a.piece_prefix = (const int32_t*)(ws + split->piece_prefix);
    a.slot_base = (const int32_t*)(ws + split->slot_base);
    a.n_pieces = (const int32_t*)(ws + split->counters) + 3;
    a.o_part = (float*)(ws + split->o_part);
    a.ml_part = (float*)(ws + split->ml_part);
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.cu = cu;
  a.cu_k = cu_k;
  a.route = route;
  a.items = items;
  a.n_items = n_items;
  a.item_cap = (int32_t)(item_cap < INT32_MAX ? item_cap : INT32_MAX);
  a.queue = queue;
  a.lse = lse;
  a.batch = batch;
  a.n_heads_q = n_heads_q;
  a.n_heads_kv = n_heads_kv;
  a.head_dim = head_dim;
  a.sink = sink;
  a.window = window;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)head_dim);
  int grid = grid_blocks;
  if (grid <= 0) {
    int ncu = 0;
    hipError_t e = cu_count(&ncu);
    if (e != hipSuccess) return hip_fail(e, "device query");
    grid = ncu * (dt == EA_BF16 ? attn_bf16_blocks_per_cu() : attn_f32_blocks_per_cu());
  }
  hipError_t e = dt == EA_BF16 ? launch_attn_bf16(a, grid, stream) : launch_attn_f32(a, grid, stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (split) {
    const int32_t* counters = (const int32_t*)(ws + split->counters);
    e = launch_split_combine(a, (const int32_t*)(ws + split->split_list), counters + 4, stream);
    if (e != hipSuccess) return hip_fail(e, "split combine launch");
  }
  return EA_OK;
}

// Workspace of the attention backward: D [n_heads_q][batch * max_seqlen_q]; for bf16 then
// lse * log2(e) of the same shape and, with several query heads per KV head, the per-head dk
// and dv partials
// [group][batch * max_seqlen_k][n_heads_kv][head_dim] (fp32 each).
struct BwdLayout {
  size_t delta = 0, lse2 = 0, dk_part = 0, dv_part = 0, total = 0;
  bool parts = false;
};
bool bwd_layout(ea_dtype dt, int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, BwdLayout* L) {
  if ((dt != EA_BF16 && dt != EA_F32) || batch < 1 || max_seqlen_q < 0 ||
      max_seqlen_k < max_seqlen_q || n_heads_q < 1 || n_heads_kv < 1 || head_dim < 1 ||
      n_heads_q % n_heads_kv != 0)
    return false;
  const int64_t rows_q = (int64_t)batch * max_seqlen_q, rows_k = (int64_t)batch * max_seqlen_k;
  if (rows_q > ((int64_t)1 << 31) - 1 || rows_k > ((int64_t)1 << 31) - 1) return false;
  const double bytes = (double)rows_k * n_heads_q * head_dim * 8.0 + (double)rows_q * n_heads_q * 4.0;
  if (bytes > 1.0e12) return false;  // beyond any device
  L->delta = 0;
  size_t at = align256((size_t)rows_q * n_heads_q * 4) + 256;
  if (dt == EA_BF16) {  // lse in base-2 units, staged by the matrix-core kernels
    L->lse2 = at;
    at += align256((size_t)rows_q * n_heads_q * 4) + 256;
  }
  L->parts = dt == EA_BF16 && n_heads_q > n_heads_kv;
  if (L->parts) {
    const size_t part = align256((size_t)rows_k * n_heads_q * head_dim * 4);  // G slices
    L->dk_part = at;
    L->dv_part = at + part;
    at += 2 * part;
  }
  L->total = at;
  return true;
}

}  // namespace

bool ws_layout(int32_t batch, int32_t max_seqlen, int32_t n_heads_q, int32_t kv_dim,
               int32_t hidden, WsLayout* out) {
  if (batch < 1 || max_seqlen < 0 || n_heads_q < 1 || kv_dim < 0 || hidden < 0) return false;
  WsLayout L;
  const int64_t qt_max = ceil_div64(max_seqlen, kMinBM);
  L.item_cap = (int64_t)batch * n_heads_q * qt_max;
  if (L.item_cap > INT32_MAX / 4) return false;
  size_t at = 0;
  L.counters = at;   at = align256(at + 16 * sizeof(int32_t));
  L.items = at;      at = align256(at + 16 * (size_t)L.item_cap);
  // The router's scratch overlays the internal work list (not the counters, which must
  // stay zero between calls): it is dead once ea_route has written its bits, and calls
  // that share a workspace are ordered on one stream.
  L.router_chunks = router_chunks(batch);
  size_t r = L.items;
  L.router_partial = r;
  r = align256(r + sizeof(float) * (size_t)batch * L.router_chunks * (size_t)kv_dim);
  L.router_x = r;
  r = align256(r + sizeof(float) * (size_t)batch * (size_t)kv_dim);
  L.router_h = r;
  r = align256(r + sizeof(float) * (size_t)batch * (size_t)hidden);
  L.total = at > r ? at : r;
  *out = L;
  return true;
}

bool ws_layout_split(int32_t batch, int32_t max_seqlen_q, int32_t n_heads_q, int32_t head_dim,
                     WsLayout* out) {
  if (head_dim < 1) return false;
  WsLayout L;
  if (!ws_layout(batch, max_seqlen_q, n_heads_q, 0, 0, &L)) return false;
  size_t at = align256(L.total);
  L.piece_prefix = at;  at = align256(at + sizeof(int32_t) * (size_t)(L.item_cap + 1));
  L.slot_base = at;     at = align256(at + sizeof(int32_t) * (size_t)L.item_cap);
  L.split_list = at;    at = align256(at + sizeof(int32_t) * (size_t)kSplitSlots);
  L.o_part = at;        at = align256(at + sizeof(float) * (size_t)kSplitSlots * kBf16BM * head_dim);
  L.ml_part = at;       at = align256(at + sizeof(float) * (size_t)kSplitSlots * kBf16BM * 2);
  L.total = at;
  *out = L;
  return true;
}

}  // namespace ea

namespace ea {
namespace {

// Device-resident workspace of ea_hybrid_attn_prefill_noalloc: the queue counters and the
// internal work list, for callers that cannot allocate.  Every GPU the library runs on
// holds its own copy until the process ends; all calls on one GPU share it.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The array's device address on each device, taken once with that device current (the
// host-side name of a __device__ array is a stand-in, not a device address).
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace ea

using namespace ea;

extern "C" {

ea_status ea_hybrid_attn_prefill_noalloc(const void* q, const void* k, const void* v, void* o,
                                         ea_dtype dt, const int32_t* cu_seqlens,
                                         const int32_t* cu_seqlens_host, int32_t batch,
                                         int32_t max_seqlen, int32_t n_heads_q,
                                         int32_t n_heads_kv, int32_t head_dim,
                                         const uint8_t* route, int32_t sink, int32_t window,
                                         float scale, float* lse_out, int32_t* worklist_out,
                                         int64_t worklist_capacity, void* stream) {
  g_last_error.clear();
  WsLayout L;
  if (batch < 1 || max_seqlen < 0 || n_heads_q < 1 ||
      !ws_layout(batch, max_seqlen, n_heads_q, 0, 0, &L))
    return fail(EA_ERR_INVALID_ARG, "batch < 1, max_seqlen < 0, n_heads_q < 1 or sizes overflow");
  if (L.total > kNoAllocScratchBytes)
    return fail(EA_ERR_UNSUPPORTED,
                "the work list needs " + std::to_string(L.total) +
                    " bytes; the no-allocation entry point holds 4194304 (batch * n_heads_q * "
                    "ceil(max_seqlen / 64) <= 262128)");
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "device scratch address");
  // the planner launched by the call below zeroes the queue counters before the
  // attention kernel reads them, so nothing left by an earlier call is read
  return ea_hybrid_attn_prefill(q, k, v, o, dt, cu_seqlens, cu_seqlens_host, batch, max_seqlen,
                                n_heads_q, n_heads_kv, head_dim, route, sink, window, scale,
                                lse_out, worklist_out, worklist_capacity, ws,
                                kNoAllocScratchBytes, stream);
}

size_t ea_workspace_size(int32_t batch, int32_t max_seqlen, int32_t n_heads_q, int32_t kv_dim,
                         int32_t hidden) {
  WsLayout L;
  if (!ws_layout(batch, max_seqlen, n_heads_q, kv_dim, hidden, &L)) return 0;
  return L.total;
}

size_t ea_prefill_chunked_workspace_size(int32_t batch, int32_t max_seqlen_q, int32_t n_heads_q,
                                         int32_t head_dim) {
  WsLayout L;
  if (!ws_layout_split(batch, max_seqlen_q, n_heads_q, head_dim, &L)) return 0;
  return L.total;
}

void ea_tile_config(ea_dtype dt, int32_t head_dim, int32_t* bm, int32_t* bn) {
  int m = 0, n = 0;
  if (!tile_shape(dt, head_dim, &m, &n)) m = n = 0;
  if (bm) *bm = m;
  if (bn) *bn = n;
}

const char* ea_status_string(ea_status s) {
  switch (s) {
    case EA_OK: return "ok";
    case EA_ERR_INVALID_ARG: return "invalid argument";
    case EA_ERR_UNSUPPORTED: return "unsupported configuration";
    case EA_ERR_WORKSPACE: return "workspace too small";
    case EA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* ea_last_error(void) { return g_last_error.c_str(); }

ea_status ea_route(const void* key_states, ea_dtype kdt, int32_t kv_dim,
                   const int32_t* cu_seqlens, int32_t batch, const float* w1, const float* b1,
                   int32_t hidden, const float* w2, const float* b2, int32_t n_heads_q,
                   float* logits_out, uint8_t* route_out, void* workspace, size_t ws_bytes,
                   void* stream) {
  g_last_error.clear();
  if (!key_states || !cu_seqlens || !w1 || !b1 || !w2 || !b2 || !route_out || !workspace)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (kdt != EA_BF16 && kdt != EA_F32) return fail(EA_ERR_INVALID_ARG, "unknown dtype");
  if (batch < 1 || kv_dim < 1 || hidden < 1 || n_heads_q < 1)
    return fail(EA_ERR_INVALID_ARG, "batch, kv_dim, hidden and n_heads_q must be >= 1");
  if (!aligned16(key_states)) return fail(EA_ERR_INVALID_ARG, "key_states must be 16-byte aligned");
  WsLayout L;
  if (!ws_layout(batch, 0, n_heads_q, kv_dim, hidden, &L))
    return fail(EA_ERR_INVALID_ARG, "sizes overflow the workspace layout");
  if (ws_bytes < L.total) return fail(EA_ERR_WORKSPACE, "workspace smaller than ea_workspace_size()");
  char* ws = (char*)workspace;
  hipError_t e = launch_route(key_states, kdt == EA_BF16 ? 0 : 1, kv_dim, cu_seqlens, batch, w1,
                              b1, hidden, w2, b2, n_heads_q, logits_out, route_out,
                              (float*)(ws + L.router_partial), L.router_chunks,
                              (float*)(ws + L.router_x), (float*)(ws + L.router_h),
                              (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  return EA_OK;
}

ea_status ea_build_worklist(const uint8_t* route, const int32_t* cu_seqlens, int32_t batch,
                            int32_t max_seqlen, int32_t n_heads_q, int32_t sink, int32_t window,
                            ea_dtype dt, int32_t head_dim, int32_t* worklist_out,
                            int64_t worklist_capacity, int32_t* n_items_out,
                            int32_t* n_items_host, void* workspace, size_t ws_bytes,
                            void* stream) {
  g_last_error.clear();
  if (!route || !cu_seqlens || !worklist_out || !workspace)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (batch < 1 || max_seqlen < 0 || n_heads_q < 1)
    return fail(EA_ERR_INVALID_ARG, "batch < 1, max_seqlen < 0 or n_heads_q < 1");
  if (sink < 0 || window < 1) return fail(EA_ERR_INVALID_ARG, "need sink >= 0 and window >= 1");
  int bm = 0, bn = 0;
  if (dt != EA_BF16 && dt != EA_F32) return fail(EA_ERR_INVALID_ARG, "unknown dtype");
  if (!tile_shape(dt, head_dim, &bm, &bn))
    return fail(EA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  ea_status s = check_plan_limits(batch, max_seqlen, n_heads_q, bm);
  if (s != EA_OK) return s;
  window = clamp_window(window, max_seqlen);
  if (worklist_capacity < item_bound(batch, max_seqlen, n_heads_q, bm))
    return fail(EA_ERR_INVALID_ARG, "worklist_capacity below batch * n_heads_q * ceil(max_seqlen / bm)");
  WsLayout L;
  if (!ws_layout(batch, max_seqlen, n_heads_q, 0, 0, &L))
    return fail(EA_ERR_INVALID_ARG, "sizes overflow the workspace layout");
  if (ws_bytes < L.total) return fail(EA_ERR_WORKSPACE, "workspace smaller than ea_workspace_size()");
  char* ws = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  s = enqueue_plan(route, cu_seqlens, batch, max_seqlen, n_heads_q, sink, window, bm, bn,
                   (int4*)worklist_out, worklist_capacity, n_items_out, L, ws, st);
  if (s != EA_OK) return s;
  if (n_items_host) {
    hipError_t e = hipMemcpyAsync(n_items_host, ws + L.counters, sizeof(int32_t),
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "item count copy");
  }
  return EA_OK;
}

ea_status ea_hybrid_attn_prefill(const void* q, const void* k, const void* v, void* o,
                                 ea_dtype dt, const int32_t* cu_seqlens,
                                 const int32_t* cu_seqlens_host, int32_t batch,
                                 int32_t max_seqlen, int32_t n_heads_q, int32_t n_heads_kv,
                                 int32_t head_dim, const uint8_t* route, int32_t sink,
                                 int32_t window, float scale, float* lse_out,
                                 int32_t* worklist_out, int64_t worklist_capacity,
                                 void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int bm = 0, bn = 0;
  ea_status s = check_attn_args(q, k, v, o, dt, cu_seqlens, batch, max_seqlen, n_heads_q,
                                n_heads_kv, head_dim, route, sink, window, scale, workspace,
                                &bm, &bn);
  if (s != EA_OK) return s;
  window = clamp_window(window, max_seqlen);
  if (worklist_out && worklist_capacity < item_bound(batch, max_seqlen, n_heads_q, bm))
    return fail(EA_ERR_INVALID_ARG, "worklist_capacity below batch * n_heads_q * ceil(max_seqlen / bm)");
  if (cu_seqlens_host) {
    s = check_cu_host(cu_seqlens_host, batch, max_seqlen);
    if (s != EA_OK) return s;
    const int64_t T = cu_seqlens_host[batch];
    const size_t elem = dt == EA_BF16 ? 2 : 4;
    const size_t nq = (size_t)T * n_heads_q * head_dim * elem;
    const size_t nkv = (size_t)T * n_heads_kv * head_dim * elem;
    if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv))
      return fail(EA_ERR_INVALID_ARG, "o overlaps q, k or v");
  }
  WsLayout L;
  if (!ws_layout(batch, max_seqlen, n_heads_q, 0, 0, &L))
    return fail(EA_ERR_INVALID_ARG, "sizes overflow the workspace layout");
  if (ws_bytes < L.total) return fail(EA_ERR_WORKSPACE, "workspace smaller than ea_workspace_size()");
  char* ws = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  int4* items = worklist_out ? (int4*)worklist_out : (int4*)(ws + L.items);
  int32_t* counters = (int32_t*)(ws + L.counters);
  const int64_t cap = worklist_out ? worklist_capacity : L.item_cap;
  s = enqueue_plan(route, cu_seqlens, batch, max_seqlen, n_heads_q, sink, window, bm, bn, items,
                   cap, nullptr, L, ws, st);
  if (s != EA_OK) return s;
  return enqueue_attn(q, k, v, o, dt, cu_seqlens, batch, n_heads_q, n_heads_kv, head_dim, route,
                      sink, window, scale, lse_out, items, counters, cap, counters + 1, 0, st);
}

ea_status ea_hybrid_attn_prefill_chunked(
    const void* q, const void* k, const void* v, void* o, ea_dtype dt,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* cu_seqlens_q_host,
    const int32_t* cu_seqlens_k_host, int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
    int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, const uint8_t* route, int32_t sink,
    int32_t window, float scale, float* lse_out, int32_t* worklist_out,
    int64_t worklist_capacity, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!cu_seqlens_k) return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (max_seqlen_q < 0 || max_seqlen_q > max_seqlen_k)
    return fail(EA_ERR_INVALID_ARG, "need 0 <= max_seqlen_q <= max_seqlen_k");
  int bm = 0, bn = 0;
  // key windows are sized by max_seqlen_k; the planner tiles the chunk's max_seqlen_q rows
  ea_status s = check_attn_args(q, k, v, o, dt, cu_seqlens_q, batch, max_seqlen_k, n_heads_q,
                                n_heads_kv, head_dim, route, sink, window, scale, workspace,
                                &bm, &bn, max_seqlen_q);
  if (s != EA_OK) return s;
  window = clamp_window(window, max_seqlen_k);
  if (o == k || o == v || q == k) return fail(EA_ERR_INVALID_ARG, "o aliases q, k or v");
  if (worklist_out && worklist_capacity < item_bound(batch, max_seqlen_q, n_heads_q, bm))
    return fail(EA_ERR_INVALID_ARG, "worklist_capacity below batch * n_heads_q * ceil(max_seqlen_q / bm)");
  if ((cu_seqlens_q_host == nullptr) != (cu_seqlens_k_host == nullptr))
    return fail(EA_ERR_INVALID_ARG, "give both host copies of the packings or neither");
  if (cu_seqlens_q_host) {
    s = check_cu_host(cu_seqlens_q_host, batch, max_seqlen_q);
    if (s != EA_OK) return s;
    s = check_cu_host(cu_seqlens_k_host, batch, max_seqlen_k);
    if (s != EA_OK) return s;
    for (int32_t b = 0; b < batch; ++b)
      if (cu_seqlens_k_host[b + 1] - cu_seqlens_k_host[b] <
          cu_seqlens_q_host[b + 1] - cu_seqlens_q_host[b])
        return fail(EA_ERR_INVALID_ARG, "a chunk is longer than its key sequence");
    const size_t elem = dt == EA_BF16 ? 2 : 4;
    const size_t nq = (size_t)cu_seqlens_q_host[batch] * n_heads_q * head_dim * elem;
    const size_t nkv = (size_t)cu_seqlens_k_host[batch] * n_heads_kv * head_dim * elem;
    if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv))
      return fail(EA_ERR_INVALID_ARG, "o overlaps q, k or v");
  }
  // bf16: long items run split over several workgroups (split-KV); fp32: one per item
  const bool split = dt == EA_BF16;
  WsLayout L;
  if (!(split ? ws_layout_split(batch, max_seqlen_q, n_heads_q, head_dim, &L)
              : ws_layout(batch, max_seqlen_q, n_heads_q, 0, 0, &L)))
    return fail(EA_ERR_INVALID_ARG, "sizes overflow the workspace layout");
  if (ws_bytes < L.total)
    return fail(EA_ERR_WORKSPACE, "workspace smaller than ea_prefill_chunked_workspace_size()");
  char* ws = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  int4* items = worklist_out ? (int4*)worklist_out : (int4*)(ws + L.items);
  int32_t* counters = (int32_t*)(ws + L.counters);
  int workers = 0;
  if (split) {
    int ncu = 0;
    const hipError_t e = cu_count(&ncu);
    if (e != hipSuccess) return hip_fail(e, "device query");
    workers = ncu * attn_bf16_blocks_per_cu();
  }
  const int64_t cap = worklist_out ? worklist_capacity : L.item_cap;
  s = enqueue_plan(route, cu_seqlens_q, batch, max_seqlen_q, n_heads_q, sink, window, bm, bn,
                   items, cap, nullptr, L, ws, st, cu_seqlens_k, workers);
  if (s != EA_OK) return s;
  return enqueue_attn(q, k, v, o, dt, cu_seqlens_q, batch, n_heads_q, n_heads_kv, head_dim,
                      route, sink, window, scale, lse_out, items, counters, cap, counters + 1, 0,
                      st, cu_seqlens_k, split ? &L : nullptr, ws);
}

ea_status ea_hybrid_attn_run(const void* q, const void* k, const void* v, void* o, ea_dtype dt,
                             const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                             int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                             const uint8_t* route, int32_t sink, int32_t window, float scale,
                             float* lse_out, const int32_t* worklist,
                             int64_t worklist_capacity, const int32_t* n_items,
                             int32_t grid_blocks, void* workspace, size_t ws_bytes,
                             void* stream) {
  g_last_error.clear();
  int bm = 0, bn = 0;
  ea_status s = check_attn_args(q, k, v, o, dt, cu_seqlens, batch, max_seqlen, n_heads_q,
                                n_heads_kv, head_dim, route, sink, window, scale, workspace,
                                &bm, &bn);
  if (s != EA_OK) return s;
  window = clamp_window(window, max_seqlen);
  if (!worklist || !n_items) return fail(EA_ERR_INVALID_ARG, "null work list or item count");
  if (grid_blocks < 0) return fail(EA_ERR_INVALID_ARG, "grid_blocks < 0");
  if (worklist_capacity < 0) return fail(EA_ERR_INVALID_ARG, "worklist_capacity < 0");
  WsLayout L;
  if (!ws_layout(batch, max_seqlen, n_heads_q, 0, 0, &L))
    return fail(EA_ERR_INVALID_ARG, "sizes overflow the workspace layout");
  if (ws_bytes < L.total) return fail(EA_ERR_WORKSPACE, "workspace smaller than ea_workspace_size()");
  char* ws = (char*)workspace;
  int32_t* counters = (int32_t*)(ws + L.counters);
  return enqueue_attn(q, k, v, o, dt, cu_seqlens, batch, n_heads_q, n_heads_kv, head_dim, route,
                      sink, window, scale, lse_out, (const int4*)worklist, n_items,
                      worklist_capacity, counters + 1, grid_blocks, (hipStream_t)stream);
}

size_t ea_decode_workspace_size(int32_t batch, int32_t max_seqlen, int32_t n_heads_q,
                                int32_t head_dim) {
  if (batch < 1 || max_seqlen < 1 || n_heads_q < 1 || head_dim < 1) return 0;
  const int64_t splits = ceil_div64(max_seqlen, kDecodeSplit);
  const int64_t slots = (int64_t)batch * n_heads_q * splits;
  if (slots > ((int64_t)1 << 40) / (head_dim + 2)) return 0;
  return align256((size_t)slots * head_dim * 4) + align256((size_t)slots * 2 * 4);
}

ea_status ea_hybrid_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                void* o, ea_dtype dt, const int32_t* seqlens,
                                const int32_t* seqlens_host, int32_t batch,
                                int32_t cache_capacity, int32_t max_seqlen, int32_t n_heads_q,
                                int32_t n_heads_kv, int32_t head_dim, const uint8_t* route,
                                int32_t sink, int32_t window, float scale, float* lse_out,
                                void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k_cache || !v_cache || !o || !seqlens || !route || !workspace)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (dt != EA_BF16 && dt != EA_F32) return fail(EA_ERR_INVALID_ARG, "unknown dtype");
  if (batch < 1 || cache_capacity < 1 || max_seqlen < 1)
    return fail(EA_ERR_INVALID_ARG, "need batch >= 1, cache_capacity >= 1, max_seqlen >= 1");
  if (max_seqlen > cache_capacity) return fail(EA_ERR_INVALID_ARG, "max_seqlen > cache_capacity");
  if (n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv != 0)
    return fail(EA_ERR_INVALID_ARG, "n_heads_q must be a positive multiple of n_heads_kv");
  if (n_heads_q / n_heads_kv > kDecodeMaxGroup)
    return fail(EA_ERR_UNSUPPORTED, "more than 8 query heads per KV head");
  if (head_dim != 64 && head_dim != 128) return fail(EA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (sink < 0 || window < 1) return fail(EA_ERR_INVALID_ARG, "need sink >= 0 and window >= 1");
  if (isnan(scale) || isinf(scale)) return fail(EA_ERR_INVALID_ARG, "scale is not finite");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(EA_ERR_INVALID_ARG, "q, caches and o must be 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0) return fail(EA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const int64_t elem = dt == EA_BF16 ? 2 : 4;
  // each sequence's KV-head window of the cache uses 32-bit byte offsets
  if ((int64_t)cache_capacity * n_heads_kv * head_dim * elem >= ((int64_t)1 << 31))
    return fail(EA_ERR_UNSUPPORTED, "cache too long for 32-bit per-sequence addressing");
  const size_t qo_bytes = (size_t)batch * n_heads_q * head_dim * elem;
  const size_t cache_bytes = (size_t)batch * cache_capacity * n_heads_kv * head_dim * elem;
  if (overlaps(o, qo_bytes, q, qo_bytes) || overlaps(o, qo_bytes, k_cache, cache_bytes) ||
      overlaps(o, qo_bytes, v_cache, cache_bytes))
    return fail(EA_ERR_INVALID_ARG, "o overlaps q or a cache");
  if (seqlens_host)
    for (int32_t b = 0; b < batch; ++b)
      if (seqlens_host[b] < 1 || seqlens_host[b] > max_seqlen)
        return fail(EA_ERR_INVALID_ARG, "seqlens must lie in [1, max_seqlen]");
  const size_t need = ea_decode_workspace_size(batch, max_seqlen, n_heads_q, head_dim);
  if (need == 0) return fail(EA_ERR_INVALID_ARG, "sizes overflow the workspace layout");
  if (ws_bytes < need) return fail(EA_ERR_WORKSPACE, "workspace smaller than ea_decode_workspace_size()");
  const int64_t splits = ceil_div64(max_seqlen, kDecodeSplit);
  if (splits > 2147483647 / 2) return fail(EA_ERR_UNSUPPORTED, "too many splits");
  window = clamp_window(window, max_seqlen);
  DecodeArgs a{};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.o = o;
  a.seqlens = seqlens;
  a.route = route;
  a.o_part = (float*)workspace;
  a.ml_part = (float*)((char*)workspace +
                       align256((size_t)batch * n_heads_q * splits * head_dim * 4));
  a.lse = lse_out;
  a.batch = batch;
  a.cap = cache_capacity;
  a.max_seqlen = max_seqlen;
  a.max_splits = (int)splits;
  a.n_heads_q = n_heads_q;
  a.n_heads_kv = n_heads_kv;
  a.head_dim = head_dim;
  a.sink = sink;
  a.window = window;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)head_dim);
  const hipError_t e = launch_decode(a, dt == EA_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return EA_OK;
}

ea_status ea_decode_pool_layout(const uint8_t* route_host, int32_t batch, int32_t n_heads_q,
                                int32_t n_heads_kv, int32_t capacity, int32_t sink,
                                int32_t window, int64_t* region_base_host,
                                int32_t* region_rows_host, int64_t* total_rows_host) {
  g_last_error.clear();
  int64_t* const region_base = region_base_host;
  int32_t* const region_rows = region_rows_host;
  int64_t* const total_rows = total_rows_host;
  if (!route_host || !region_base || !region_rows || !total_rows)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (batch < 1 || capacity < 1) return fail(EA_ERR_INVALID_ARG, "need batch >= 1 and capacity >= 1");
  if (n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv != 0)
    return fail(EA_ERR_INVALID_ARG, "n_heads_q must be a positive multiple of n_heads_kv");
  if (sink < 0 || window < 1) return fail(EA_ERR_INVALID_ARG, "need sink >= 0 and window >= 1");
  if ((int64_t)sink + window > 2147483647) return fail(EA_ERR_INVALID_ARG, "sink + window overflows");
  const int G = n_heads_q / n_heads_kv;
  int64_t next = 0;
  for (int32_t b = 0; b < batch; ++b)
    for (int32_t h = 0; h < n_heads_kv; ++h) {
      bool any_full = false;
      for (int g = 0; g < G; ++g) any_full |= route_host[(int64_t)b * n_heads_q + h * G + g] == 0;
      const int32_t rows = any_full ? capacity : sink + window;
      region_base[(int64_t)b * n_heads_kv + h] = next;
      region_rows[(int64_t)b * n_heads_kv + h] = rows;
      next += rows;
    }
  *total_rows = next;
  return EA_OK;
}

// checks shared by the pooled-cache entry points
static ea_status check_pool_args(ea_dtype dt, int32_t batch, int32_t n_heads_q, int32_t n_heads_kv,
                                 int32_t head_dim, int32_t sink, int32_t window, int64_t pool_rows,
                                 const void* k_pool, const void* v_pool) {
  if (dt != EA_BF16 && dt != EA_F32) return fail(EA_ERR_INVALID_ARG, "unknown dtype");
  if (batch < 1) return fail(EA_ERR_INVALID_ARG, "need batch >= 1");
  if (n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv != 0)
    return fail(EA_ERR_INVALID_ARG, "n_heads_q must be a positive multiple of n_heads_kv");
  if (n_heads_q / n_heads_kv > kDecodeMaxGroup)
    return fail(EA_ERR_UNSUPPORTED, "more than 8 query heads per KV head");
  if (head_dim != 64 && head_dim != 128) return fail(EA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (sink < 0 || window < 1) return fail(EA_ERR_INVALID_ARG, "need sink >= 0 and window >= 1");
  if ((int64_t)sink + window > 2147483647) return fail(EA_ERR_INVALID_ARG, "sink + window overflows");
  if (pool_rows < 1) return fail(EA_ERR_INVALID_ARG, "need pool_rows >= 1");
  if (!aligned16(k_pool) || !aligned16(v_pool))
    return fail(EA_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  const int64_t row_bytes = (int64_t)head_dim * (dt == EA_BF16 ? 2 : 4);
  if (overlaps(k_pool, (size_t)(pool_rows * row_bytes), v_pool, (size_t)(pool_rows * row_bytes)))
    return fail(EA_ERR_INVALID_ARG, "k_pool and v_pool overlap");
  return EA_OK;
}

ea_status ea_decode_pool_fill(const void* k, const void* v, ea_dtype dt, const int32_t* cu_seqlens,
                              int32_t batch, int32_t max_seqlen, int32_t n_heads_q,
                              int32_t n_heads_kv, int32_t head_dim, const uint8_t* route,
                              int32_t sink, int32_t window, const int64_t* region_base,
                              const int32_t* region_rows, int64_t pool_rows, void* k_pool,
                              void* v_pool, void* stream) {
  g_last_error.clear();
  if (!k || !v || !cu_seqlens || !route || !region_base || !region_rows || !k_pool || !v_pool)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  const ea_status st = check_pool_args(dt, batch, n_heads_q, n_heads_kv, head_dim, sink, window,
                                       pool_rows, k_pool, v_pool);
  if (st != EA_OK) return st;
  if (max_seqlen < 1) return fail(EA_ERR_INVALID_ARG, "need max_seqlen >= 1");
  if (!aligned16(k) || !aligned16(v)) return fail(EA_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  PoolWriteArgs a{};
  a.k = k;
  a.v = v;
  a.cu = cu_seqlens;
  a.route = route;
  a.region_base = region_base;
  a.region_rows = region_rows;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.pool_rows = pool_rows;
  a.batch = batch;
  a.max_seqlen = max_seqlen;
  a.n_heads_q = n_heads_q;
  a.n_heads_kv = n_heads_kv;
  a.head_dim = head_dim;
  a.sink = sink;
  a.window = window;
  const hipError_t e = launch_pool_fill(a, dt == EA_BF16 ? 2 : 4, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pool fill launch");
  return EA_OK;
}

ea_status ea_decode_pool_append(const void* k_new, const void* v_new, ea_dtype dt,
                                const int32_t* positions, int32_t batch, int32_t n_heads_q,
                                int32_t n_heads_kv, int32_t head_dim, const uint8_t* route,
                                int32_t sink, int32_t window, const int64_t* region_base,
                                const int32_t* region_rows, int64_t pool_rows, void* k_pool,
                                void* v_pool, void* stream) {
  g_last_error.clear();
  if (!k_new || !v_new || !positions || !route || !region_base || !region_rows || !k_pool || !v_pool)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  const ea_status st = check_pool_args(dt, batch, n_heads_q, n_heads_kv, head_dim, sink, window,
                                       pool_rows, k_pool, v_pool);
  if (st != EA_OK) return st;
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(EA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  PoolWriteArgs a{};
  a.k = k_new;
  a.v = v_new;
  a.positions = positions;
  a.route = route;
  a.region_base = region_base;
  a.region_rows = region_rows;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.pool_rows = pool_rows;
  a.batch = batch;
  a.n_heads_q = n_heads_q;
  a.n_heads_kv = n_heads_kv;
  a.head_dim = head_dim;
  a.sink = sink;
  a.window = window;
  const hipError_t e = launch_pool_append(a, dt == EA_BF16 ? 2 : 4, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pool append launch");
  return EA_OK;
}

ea_status ea_hybrid_attn_decode_pool(const void* q, const void* k_pool, const void* v_pool,
                                     void* o, ea_dtype dt, const int32_t* seqlens,
                                     const int32_t* seqlens_host, int32_t batch,
                                     int32_t max_seqlen, int32_t n_heads_q, int32_t n_heads_kv,
                                     int32_t head_dim, const int64_t* region_base,
                                     const int32_t* region_rows, int64_t pool_rows,
                                     const uint8_t* route, int32_t sink, int32_t window,
                                     float scale, float* lse_out, void* workspace,
                                     size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k_pool || !v_pool || !o || !seqlens || !route || !workspace || !region_base ||
      !region_rows)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  const ea_status st = check_pool_args(dt, batch, n_heads_q, n_heads_kv, head_dim, sink, window,
                                       pool_rows, k_pool, v_pool);
  if (st != EA_OK) return st;
  if (max_seqlen < 1) return fail(EA_ERR_INVALID_ARG, "need max_seqlen >= 1");
  if (isnan(scale) || isinf(scale)) return fail(EA_ERR_INVALID_ARG, "scale is not finite");
  if (!aligned16(q) || !aligned16(o)) return fail(EA_ERR_INVALID_ARG, "q and o must be 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0) return fail(EA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const int64_t elem = dt == EA_BF16 ? 2 : 4;
  const size_t qo_bytes = (size_t)batch * n_heads_q * head_dim * elem;
  const size_t pool_bytes = (size_t)pool_rows * head_dim * elem;
  if (overlaps(o, qo_bytes, q, qo_bytes) || overlaps(o, qo_bytes, k_pool, pool_bytes) ||
      overlaps(o, qo_bytes, v_pool, pool_bytes))
    return fail(EA_ERR_INVALID_ARG, "o overlaps q or a pool");
  if (seqlens_host)
    for (int32_t b = 0; b < batch; ++b)
      if (seqlens_host[b] < 1 || seqlens_host[b] > max_seqlen)
        return fail(EA_ERR_INVALID_ARG, "seqlens must lie in [1, max_seqlen]");
  const size_t need = ea_decode_workspace_size(batch, max_seqlen, n_heads_q, head_dim);
  if (need == 0) return fail(EA_ERR_INVALID_ARG, "sizes overflow the workspace layout");
  if (ws_bytes < need) return fail(EA_ERR_WORKSPACE, "workspace smaller than ea_decode_workspace_size()");
  const int64_t splits = ceil_div64(max_seqlen, kDecodeSplit);
  DecodeArgs a{};
  a.q = q;
  a.kc = k_pool;
  a.vc = v_pool;
  a.o = o;
  a.seqlens = seqlens;
  a.route = route;
  a.region_base = region_base;
  a.region_rows = region_rows;
  a.pool_rows = pool_rows;
  a.pooled = 1;
  a.o_part = (float*)workspace;
  a.ml_part = (float*)((char*)workspace +
                       align256((size_t)batch * n_heads_q * splits * head_dim * 4));
  a.lse = lse_out;
  a.batch = batch;
  a.cap = max_seqlen;  // lengths are bounded by max_seqlen; each region's size by its own check
  a.max_seqlen = max_seqlen;
  a.max_splits = (int)splits;
  a.n_heads_q = n_heads_q;
  a.n_heads_kv = n_heads_kv;
  a.head_dim = head_dim;
  a.sink = sink;
  a.window = window;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)head_dim);
  const hipError_t e = launch_decode(a, dt == EA_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pooled decode launch");
  return EA_OK;
}


size_t ea_attn_backward_workspace_size(ea_dtype dt, int32_t batch, int32_t max_seqlen_q,
                                       int32_t max_seqlen_k, int32_t n_heads_q,
                                       int32_t n_heads_kv, int32_t head_dim) {
  BwdLayout L;
  return bwd_layout(dt, batch, max_seqlen_q, max_seqlen_k, n_heads_q, n_heads_kv, head_dim, &L)
             ? L.total
             : 0;
}

ea_status ea_hybrid_attn_backward(
    const void* q, const void* k, const void* v, const void* o, const void* dout, ea_dtype dt,
    const float* lse, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host, int32_t batch,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_heads_q, int32_t n_heads_kv,
    int32_t head_dim, const uint8_t* route, int32_t sink, int32_t window, float scale,
    float* dq, float* dk, float* dv, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !dout || !lse || !cu_seqlens_q || !route || !dq || !dk || !dv ||
      !workspace)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if (dt != EA_BF16 && dt != EA_F32) return fail(EA_ERR_INVALID_ARG, "unknown dtype");
  if (batch < 1 || batch > 65535) return fail(EA_ERR_INVALID_ARG, "need 1 <= batch <= 65535");
  if (max_seqlen_q < 0 || max_seqlen_q > max_seqlen_k)
    return fail(EA_ERR_INVALID_ARG, "need 0 <= max_seqlen_q <= max_seqlen_k");
  if (n_heads_kv < 1 || n_heads_q < n_heads_kv || n_heads_q % n_heads_kv != 0 ||
      n_heads_q > 65535)
    return fail(EA_ERR_INVALID_ARG, "n_heads_q must be a positive multiple of n_heads_kv");
  if (sink < 0 || window < 1) return fail(EA_ERR_INVALID_ARG, "need sink >= 0 and window >= 1");
  if (isnan(scale) || isinf(scale)) return fail(EA_ERR_INVALID_ARG, "scale is not finite");
  if (head_dim != 64 && head_dim != 128)
    return fail(EA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(EA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0)
    return fail(EA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  // the matrix-core kernels address one sequence's q / dO rows (all query heads; k and v are
  // no larger) with 32-bit byte offsets; the fp32 kernels index with 64 bits
  if (dt == EA_BF16 && (int64_t)max_seqlen_k * n_heads_q * head_dim * 2 > ((int64_t)1 << 31))
    return fail(EA_ERR_UNSUPPORTED, "sequence too long for 32-bit per-sequence addressing");
  if (!cu_seqlens_k) {
    cu_seqlens_k = cu_seqlens_q;
    cu_seqlens_k_host = cu_seqlens_q_host;
  }
  if ((cu_seqlens_q_host == nullptr) != (cu_seqlens_k_host == nullptr))
    return fail(EA_ERR_INVALID_ARG, "give both host copies of the packings or neither");
  if (cu_seqlens_q_host) {
    ea_status s = check_cu_host(cu_seqlens_q_host, batch, max_seqlen_q);
    if (s != EA_OK) return s;
    s = check_cu_host(cu_seqlens_k_host, batch, max_seqlen_k);
    if (s != EA_OK) return s;
    for (int32_t b = 0; b < batch; ++b)
      if (cu_seqlens_k_host[b + 1] - cu_seqlens_k_host[b] <
          cu_seqlens_q_host[b + 1] - cu_seqlens_q_host[b])
        return fail(EA_ERR_INVALID_ARG, "a chunk is longer than its key sequence");
    const size_t elem = dt == EA_BF16 ? 2 : 4;
    const size_t tq = (size_t)cu_seqlens_q_host[batch], tk = (size_t)cu_seqlens_k_host[batch];
    const size_t nq = tq * n_heads_q * head_dim, nkv = tk * n_heads_kv * head_dim;
    const void* ins[6] = {q, k, v, o, dout, lse};
    const size_t in_bytes[6] = {nq * elem, nkv * elem, nkv * elem, nq * elem, nq * elem,
                                tq * n_heads_q * 4};
    const void* outs[3] = {dq, dk, dv};
    const size_t out_bytes[3] = {nq * 4, nkv * 4, nkv * 4};
    for (int i = 0; i < 3; ++i) {
      for (int j = 0; j < 6; ++j)
        if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j]))
          return fail(EA_ERR_INVALID_ARG, "a gradient buffer overlaps an input");
      for (int j = i + 1; j < 3; ++j)
        if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j]))
          return fail(EA_ERR_INVALID_ARG, "gradient buffers overlap");
    }
  } else if (dq == dk || dq == dv || dk == dv) {
    return fail(EA_ERR_INVALID_ARG, "gradient buffers overlap");
  }
  window = clamp_window(window, max_seqlen_k);
  BwdLayout WL;
  if (!bwd_layout(dt, batch, max_seqlen_q, max_seqlen_k, n_heads_q, n_heads_kv, head_dim, &WL))
    return fail(EA_ERR_INVALID_ARG, "sizes overflow the workspace layout");
  if (ws_bytes < WL.total)
    return fail(EA_ERR_WORKSPACE, "workspace smaller than ea_attn_backward_workspace_size()");
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.route = route;
  a.delta = (float*)workspace;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.tq_cap = (int64_t)batch * max_seqlen_q;
  a.tk_cap = (int64_t)batch * max_seqlen_k;
  a.lse2 = dt == EA_BF16 ? (float*)((char*)workspace + WL.lse2) : nullptr;
  a.dk_part = WL.parts ? (float*)((char*)workspace + WL.dk_part) : nullptr;
  a.dv_part = WL.parts ? (float*)((char*)workspace + WL.dv_part) : nullptr;
  a.batch = batch;
  a.max_seqlen_q = max_seqlen_q;
  a.max_seqlen_k = max_seqlen_k;
  a.n_heads_q = n_heads_q;
  a.n_heads_kv = n_heads_kv;
  a.head_dim = head_dim;
  a.sink = sink;
  a.window = window;
  a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)head_dim);
  if (max_seqlen_k == 0) return EA_OK;  // nothing to do: every sequence is empty
  const hipError_t e = launch_attn_backward(a, dt == EA_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention backward launch");
  return EA_OK;
}

namespace {
struct RouteBwdLayout {
  int pool_chunks = 0, dr_chunks = 0;
  size_t pool_partial = 0, x = 0, u = 0, hs = 0, du = 0, dx = 0, dr_partial = 0, total = 0;
};
bool route_bwd_layout(int32_t batch, int32_t kv_dim, int32_t hidden, int32_t n_heads_q,
                      int32_t head_dim, RouteBwdLayout* L) {
  if (batch < 1 || kv_dim < 1 || hidden < 1 || n_heads_q < 1 || head_dim < 1) return false;
  if ((int64_t)batch * kv_dim > ((int64_t)1 << 31) || (int64_t)hidden * kv_dim > ((int64_t)1 << 31) ||
      (int64_t)n_heads_q * head_dim > ((int64_t)1 << 24))
    return false;
  L->pool_chunks = router_chunks(batch);
  L->dr_chunks = route_bwd_chunks(batch, n_heads_q * head_dim);
  size_t at = 0;
  auto take = [&](size_t floats) {
    const size_t here = at;
    at += align256(floats * 4);
    return here;
  };
  L->pool_partial = take((size_t)batch * L->pool_chunks * kv_dim);
  L->x = take((size_t)batch * kv_dim);
  L->u = take((size_t)batch * hidden);
  L->hs = take((size_t)batch * hidden);
  L->du = take((size_t)batch * hidden);
  L->dx = take((size_t)batch * kv_dim);
  L->dr_partial = take((size_t)batch * L->dr_chunks * n_heads_q);
  L->total = at;
  return true;
}
}  // namespace

size_t ea_route_backward_workspace_size(int32_t batch, int32_t kv_dim, int32_t hidden,
                                        int32_t n_heads_q, int32_t head_dim) {
  RouteBwdLayout L;
  return route_bwd_layout(batch, kv_dim, hidden, n_heads_q, head_dim, &L) ? L.total : 0;
}

ea_status ea_route_backward(const void* key_states, ea_dtype kdt, int32_t kv_dim,
                            const int32_t* cu_seqlens, int32_t batch, const float* w1,
                            const float* b1, int32_t hidden, const float* w2, const float* b2,
                            int32_t n_heads_q, const void* o_full, const void* o_sparse,
                            const void* dout, ea_dtype odt, int32_t head_dim, const float* noise,
                            float tau, float* dr_out, float* dz_out, float* dw1, float* db1,
                            float* dw2, float* db2, float* dkey_states, void* workspace,
                            size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!key_states || !cu_seqlens || !w1 || !b1 || !w2 || !b2 || !o_full || !o_sparse || !dout ||
      !dz_out || !dw1 || !db1 || !dw2 || !db2 || !workspace)
    return fail(EA_ERR_INVALID_ARG, "null pointer argument");
  if ((kdt != EA_BF16 && kdt != EA_F32) || (odt != EA_BF16 && odt != EA_F32))
    return fail(EA_ERR_INVALID_ARG, "unknown dtype");
  if (batch < 1 || batch > 65535 || kv_dim < 1 || hidden < 1 || hidden > 65535 ||
      n_heads_q < 1 || n_heads_q > 65535)
    return fail(EA_ERR_INVALID_ARG, "batch, kv_dim, hidden and n_heads_q out of range");
  if (head_dim != 64 && head_dim != 128)
    return fail(EA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!(tau > 0.f) || isinf(tau)) return fail(EA_ERR_INVALID_ARG, "tau must be positive and finite");
  if (dkey_states && (kv_dim % 4 != 0 || !aligned16(dkey_states)))
    return fail(EA_ERR_UNSUPPORTED, "dkey_states needs kv_dim % 4 == 0 and 16-byte alignment");
  if (!aligned16(key_states) || !aligned16(o_full) || !aligned16(o_sparse) || !aligned16(dout))
    return fail(EA_ERR_INVALID_ARG, "key_states and the outputs must be 16-byte aligned");
  if (((uintptr_t)workspace & 255) != 0)
    return fail(EA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  RouteBwdLayout L;
  if (!route_bwd_layout(batch, kv_dim, hidden, n_heads_q, head_dim, &L))
    return fail(EA_ERR_INVALID_ARG, "sizes overflow the workspace layout");
  if (ws_bytes < L.total)
    return fail(EA_ERR_WORKSPACE, "workspace smaller than ea_route_backward_workspace_size()");
  char* ws = (char*)workspace;
  RouteBwdArgs a{};
  a.key_states = key_states;
  a.cu = cu_seqlens;
  a.w1 = w1;
  a.b1 = b1;
  a.w2 = w2;
  a.b2 = b2;
  a.o_full = o_full;
  a.o_sparse = o_sparse;
  a.dout = dout;
  a.noise = noise;
  a.tau = tau;
  a.kdt = kdt == EA_BF16 ? 0 : 1;
  a.odt = odt == EA_BF16 ? 0 : 1;
  a.batch = batch;
  a.kv_dim = kv_dim;
  a.hidden = hidden;
  a.n_heads_q = n_heads_q;
  a.head_dim = head_dim;
  a.pool_chunks = L.pool_chunks;
  a.dr_chunks = L.dr_chunks;
  a.pool_partial = (float*)(ws + L.pool_partial);
  a.x = (float*)(ws + L.x);
  a.u = (float*)(ws + L.u);
  a.hs = (float*)(ws + L.hs);
  a.du = (float*)(ws + L.du);
  a.dx = (float*)(ws + L.dx);
  a.dr_partial = (float*)(ws + L.dr_partial);
  a.dr = dr_out;
  a.dz = dz_out;
  a.dw1 = dw1;
  a.db1 = db1;
  a.dw2 = dw2;
  a.db2 = db2;
  a.dkey_states = dkey_states;
  const hipError_t e = launch_route_backward(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "router backward launch");
  return EA_OK;
}

}  // extern "C"
