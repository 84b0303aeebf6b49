// ea_plan.hip -- front half of the persistent scheduler: the work list of the fused
// launch.  The Elastic Attention blog post (section 3, "Fused Kernel") hands the routing
// decision to one kernel as metadata so that full and sparse heads share a launch; here
// that metadata is a list of (sequence, head, q-tile, cost) items in longest-first order.
//
// Cost of an item = number of bn-key tiles the kernel visits for its rows [m0, m1) (query
// positions; in a chunked prefill over a KV prefix the chunk's rows start at position
// Lk - Lq, and a sequence with Lk < Lq gets no items):
//   full head:   tiles 0 .. (m1-1)/bn
//   sparse head: sink tiles 0 .. ceil(min(sink, m1)/bn)-1 united with window tiles
//                max(0, m0-window+1)/bn .. (m1-1)/bn
// Both costs depend on (sequence, q-tile, mode) only, so the planner sorts "cells" -- one
// per (sequence, q-tile, cost), holding the heads of that cost -- and expands them.
// Cell i = 2*slot + sub, slots numbered in (sequence, q-tile) order.  Sorting the keys
// (cost descending, then i) with a bitonic network in LDS gives exactly the order cost
// desc, (sequence, q-tile) asc; heads inside a cell are written in ascending order, so
// the list is cost desc, (sequence, q-tile, head) asc.  One workgroup of 1024 threads,
// integer only, deterministic.  The planner also zeroes the attention kernel's queue
// counters.
#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kNumWaves = kPlanThreads / 64;

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct HeadMask {
  uint64_t lo, hi;  // bit h (h < 64 in lo, 64 <= h < 128 in hi) = head h is sparse
};

// Cell i: {seq, q_tile, cost, mode mask (1 = full heads, 2 = sparse heads)}; cost 0 = empty.
// len_of[b] = chunk rows of sequence b, off_of[b] = position of its chunk row 0 (keys - rows).
__device__ __forceinline__ int4 make_cell(int i, const PlanArgs& a, const int* qt_prefix,
                                          const int* n_sparse_of, const int* len_of,
                                          const int* off_of) {
  const int f = i >> 1, sub = i & 1;
  int lo = 0, hi = a.batch - 1;  // last b with qt_prefix[b] <= f (never an empty sequence)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qt_prefix[mid] <= f) lo = mid; else hi = mid - 1;
  }
  const int b = lo, qt = f - qt_prefix[b];
  const int len = len_of[b];
  const int off = off_of[b];
  if (off < 0) return int4{b, qt, 0, 0};  // keys shorter than the chunk: no items
  const int m0 = off + qt * a.bm, m1 = off + min(qt * a.bm + a.bm, len);
  const int t_hi = (m1 - 1) / a.bn;
  const int n_sink = ceil_div(min(a.sink, m1), a.bn);
  const int t_lo = max(0, m0 - a.window + 1) / a.bn;
  const int c_full = t_hi + 1;
  const int c_sparse = n_sink >= t_lo ? t_hi + 1 : n_sink + (t_hi - t_lo + 1);
  const int ns = n_sparse_of[b], nf = a.n_heads_q - ns;
  int4 c = {b, qt, 0, 0};
  if (nf > 0 && ns > 0 && c_full == c_sparse) {
    if (sub == 0) { c.z = c_full; c.w = 3; }
  } else if (nf > 0 && ns > 0) {
    if (sub == 0) { c.z = c_full; c.w = 1; } else { c.z = c_sparse; c.w = 2; }
  } else if (sub == 0) {
    c.z = nf > 0 ? c_full : c_sparse;
    c.w = nf > 0 ? 1 : 2;
  }
  return c;
}

// Block-wide exclusive scan of one int per thread; *total receives the sum.
__device__ int block_exclusive_scan(int v, int* total, int* scratch /* >= kNumWaves+1 */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int n = __shfl_up(incl, d, 64);
    if (lane >= d) incl += n;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kNumWaves; ++w) {
      const int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[kNumWaves] = run;
  }
  __syncthreads();
  const int excl = scratch[wave] + incl - v;
  *total = scratch[kNumWaves];
  __syncthreads();
  return excl;
}

// An empty work list (every counter zero), for inputs the list cannot describe.
__device__ void empty_list(const PlanArgs& a) {
  if (threadIdx.x == 0) {
    for (int i = 0; i < 5; ++i) a.counters[i] = 0;
    if (a.n_items_out) *a.n_items_out = 0;
    if (a.piece_prefix) a.piece_prefix[0] = 0;
  }
}

// Phase 6 (split-KV): every item of cost c runs as ns = min(kSplitMaxPieces, ceil(c / T))
// pieces; T = max(kSplitMinTiles, ceil(total cost / (2 * workers))), doubled until the split
// items' pieces fit the kSplitSlots partial-result slots.  Writes piece_prefix (first piece of
// every item, and the total), slot_base (first slot of a split item, else -1), split_list and
// counters[3] (pieces), counters[4] (split items).  The list order is unchanged, so the pieces
// of one item are consecutive and long items still come first.
__device__ void split_phase(const PlanArgs& a, int n_items, int* scratch, const uint64_t* cells,
                            const int* cell_off, int n_valid) {
  __shared__ unsigned long long s_sum;
  __shared__ int s_slots;
  const int tid = threadIdx.x;
  // the cost of item i: that of the sorted cell holding it (the last p with cell_off[p] <= i)
  auto cost_of = [&](int i) {
    int lo = 0, hi = n_valid - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cell_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return (int)((cells[lo] >> 2) & 0x3fffff);
  };
  if (tid == 0) s_sum = 0;
  __syncthreads();
  unsigned long long part = 0;
  for (int i = tid; i < n_items; i += kPlanThreads) part += (unsigned)cost_of(i);
  atomicAdd(&s_sum, part);
  __syncthreads();
  const long long total = (long long)s_sum;
  long long budget = (total + 2LL * a.split_workers - 1) / (2LL * a.split_workers);
  if (budget < kSplitMinTiles) budget = kSplitMinTiles;
  auto pieces_of = [&](int cost) -> int {
    const long long ns = (cost + budget - 1) / budget;
    return (int)(ns < 1 ? 1 : (ns > kSplitMaxPieces ? kSplitMaxPieces : ns));
  };
  for (int round = 0; round < 40; ++round) {
    if (tid == 0) s_slots = 0;
    __syncthreads();
    int slots = 0;
    for (int i = tid; i < n_items; i += kPlanThreads) {
      const int ns = pieces_of(cost_of(i));
      if (ns > 1) slots += ns;
    }
    atomicAdd(&s_slots, slots);
    __syncthreads();
    const int used = s_slots;
    __syncthreads();
    if (used <= kSplitSlots) break;
    budget *= 2;
  }
  int carry_p = 0, carry_s = 0, carry_n = 0;
  for (int base = 0; base < n_items; base += kPlanThreads) {
    const int i = base + tid;
    const int ns = i < n_items ? pieces_of(cost_of(i)) : 0;
    const int sl = ns > 1 ? ns : 0;
    int tp, ts, tn;
    const int ep = block_exclusive_scan(ns, &tp, scratch);
    const int es = block_exclusive_scan(sl, &ts, scratch);
    const int en = block_exclusive_scan(sl > 0 ? 1 : 0, &tn, scratch);
    if (i < n_items) {
      a.piece_prefix[i] = carry_p + ep;
      a.slot_base[i] = sl > 0 ? carry_s + es : -1;
      if (sl > 0) a.split_list[carry_n + en] = i;
    }
    carry_p += tp;
    carry_s += ts;
    carry_n += tn;
  }
  if (tid == 0) {
    a.piece_prefix[n_items] = carry_p;
    a.counters[3] = carry_p;
    a.counters[4] = carry_n;
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ uint64_t keys[kPlanMaxCells];    // sort keys, then packed sorted cells
  __shared__ int cell_off[kPlanMaxCells];      // first item of every sorted cell
  __shared__ HeadMask masks[kPlanMaxBatch];    // sparse heads of every sequence
  __shared__ int qt_prefix[kPlanMaxBatch + 1]; // first slot of every sequence
  __shared__ int n_sparse_of[kPlanMaxBatch];
  __shared__ int len_of[kPlanMaxBatch];        // chunk rows of every sequence
  __shared__ int off_of[kPlanMaxBatch];        // position of its chunk row 0 (keys - rows)
  __shared__ int scratch[kNumWaves + 1];
  __shared__ int s_valid;
  const int tid = threadIdx.x;
  const int B = a.batch, Hq = a.n_heads_q;

  // Phase 1: sparse-head masks (one thread per routing byte), then per-sequence q-tile
  // counts and their exclusive prefix.
  if (tid == 0) s_valid = 0;
  for (int b = tid; b < B; b += kPlanThreads) masks[b] = HeadMask{0ull, 0ull};
  __syncthreads();
  for (int x = tid; x < B * Hq; x += kPlanThreads) {
    if (a.route[x] != 0) {
      const int b = x / Hq, h = x % Hq;
      if (h < 64) atomicOr((unsigned long long*)&masks[b].lo, 1ull << h);
      else atomicOr((unsigned long long*)&masks[b].hi, 1ull << (h - 64));
    }
  }
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int b = base + tid;
    int nq = 0;
    if (b < B) {
      const int len = a.cu[b + 1] - a.cu[b];
      len_of[b] = len;
      off_of[b] = a.cu_k ? (a.cu_k[b + 1] - a.cu_k[b]) - len : 0;
      nq = ceil_div(len, a.bm);
      n_sparse_of[b] = __popcll(masks[b].lo) + __popcll(masks[b].hi);
    }
    int tot;
    const int ex = block_exclusive_scan(nq, &tot, scratch);
    if (b < B) qt_prefix[b] = carry + ex;
    carry += tot;
  }
  if (tid == 0) qt_prefix[B] = carry;
  __syncthreads();
  // device lengths beyond what the host sized (more cells than the LDS holds): empty list
  if (2 * (int64_t)carry > kPlanMaxCells) {
    empty_list(a);
    return;
  }
  const int n_cells = 2 * carry;
  int n_pad = 2;
  while (n_pad < n_cells) n_pad <<= 1;

  // Phase 2: sort keys.  High word: 0x7fffffff - cost (descending cost); low word: i.
  for (int i = tid; i < n_pad; i += kPlanThreads) {
    uint64_t key = ~0ull;
    if (i < n_cells) {
      const int4 c = make_cell(i, a, qt_prefix, n_sparse_of, len_of, off_of);
      if (c.z > 0) {
        key = ((uint64_t)(0x7fffffff - c.z) << 32) | (uint32_t)i;
        atomicAdd(&s_valid, 1);
      }
    }
    keys[i] = key;
  }
  __syncthreads();

  // Phase 3: bitonic sort, ascending.  Up to one key per thread, each thread keeps its key
  // in registers and takes its partner's by a wavefront shuffle when the partner is in the
  // same wavefront (distance < 64), through LDS otherwise; element i keeps the smaller of
  // the pair when it is the lower index of an ascending pair or the higher of a descending
  // one, the larger otherwise (the compare-exchange, computed on both sides).
  if (n_pad <= kPlanThreads) {
    uint64_t v = tid < n_pad ? keys[tid] : ~0ull;
    for (int k = 2; k <= n_pad; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        uint64_t y;
        if (j < 64) {
          const unsigned lo = __shfl_xor((unsigned)v, j, 64);
          const unsigned hi = __shfl_xor((unsigned)(v >> 32), j, 64);
          y = ((uint64_t)hi << 32) | lo;
        } else {
          keys[tid] = v;
          __syncthreads();
          y = keys[tid ^ j];
          __syncthreads();
        }
        const bool keep_min = ((tid & k) == 0) == ((tid & j) == 0);
        v = keep_min ? (v < y ? v : y) : (v < y ? y : v);
      }
    }
    if (tid < n_pad) keys[tid] = v;
    __syncthreads();
  } else {  // several keys per thread: every step through LDS
    for (int k = 2; k <= n_pad; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n_pad; i += kPlanThreads) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint64_t x = keys[i], y = keys[ixj];
            const bool up = (i & k) == 0;
            if ((x > y) == up) {
              keys[i] = y;
              keys[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
  }

  // Phase 4: unpack the sorted cells (in place) and give every cell its first item.
  const int n_valid = s_valid;
  int items_total = 0;
  for (int base = 0; base < n_valid; base += kPlanThreads) {
    const int p = base + tid;
    int sz = 0;
    if (p < n_valid) {
      const int i = (int)(keys[p] & 0xffffffffu);
      const int4 c = make_cell(i, a, qt_prefix, n_sparse_of, len_of, off_of);
      const int ns = n_sparse_of[c.x];
      sz = ((c.w & 1) ? Hq - ns : 0) + ((c.w & 2) ? ns : 0);
      // packed cell: seq (20 bits) | q_tile (20 bits) | cost (22 bits) | mode (2 bits)
      keys[p] = ((uint64_t)c.x << 44) | ((uint64_t)c.y << 24) | ((uint64_t)c.z << 2) |
                (uint64_t)c.w;
    }
    int tot;
    const int ex = block_exclusive_scan(sz, &tot, scratch);
    if (p < n_valid) cell_off[p] = items_total + ex;
    items_total += tot;
  }
  __syncthreads();
  // more items than the list holds (device lengths beyond what the host sized): empty list
  if (items_total > a.item_cap) {
    empty_list(a);
    return;
  }

  // Phase 5: expansion, heads of a cell in ascending order.  Each cell's heads are cut into
  // 2^ls runs of `per` heads, as many as keep every thread busy, and one thread writes a run:
  // its first item goes to the cell's offset plus the number of the cell's heads below the
  // run (all of them for a cell of both modes, else the sparse or the full ones, by
  // popcount).
  {
    int ls = 0;
    while ((1 << ls) < Hq && n_valid * (2 << ls) <= kPlanThreads) ++ls;
    const int per = (Hq + (1 << ls) - 1) >> ls;
    for (int x = tid; x < (n_valid << ls); x += kPlanThreads) {
      const int p = x >> ls, hb = (x & ((1 << ls) - 1)) * per, he = min(Hq, hb + per);
      if (hb >= he) continue;
      const uint64_t pk = keys[p];
      const int b = (int)(pk >> 44), qt = (int)((pk >> 24) & 0xfffff);
      const int cost = (int)((pk >> 2) & 0x3fffff), mode = (int)(pk & 3);
      const HeadMask m = masks[b];
      const int sp_below = hb < 64 ? __popcll(m.lo & ((1ull << hb) - 1ull))
                                   : __popcll(m.lo) + __popcll(m.hi & ((1ull << (hb - 64)) - 1ull));
      int at = cell_off[p] + (mode == 3 ? hb : (mode == 2 ? sp_below : hb - sp_below));
      for (int h = hb; h < he; ++h) {
        const bool sp = ((h < 64 ? (m.lo >> h) : (m.hi >> (h - 64))) & 1ull) != 0;
        if (mode & (sp ? 2 : 1)) a.items[at++] = int4{b, h, qt, cost};
      }
    }
  }
  if (tid == 0) {
    a.counters[0] = items_total;
    a.counters[1] = 0;  // queue head
    a.counters[2] = 0;  // workgroups finished
    if (a.n_items_out) *a.n_items_out = items_total;
  }
  if (a.split_workers > 0) split_phase(a, items_total, scratch, keys, cell_off, n_valid);
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  plan_kernel<<<1, kPlanThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ea
