// ea_plan.hip -- front half of the persistent scheduler: the work list of the fused
// launch.  The Elastic Attention blog post (section 3, "Fused Kernel") hands the routing
// decision to one kernel as metadata so that full and sparse heads share a launch; here
// that metadata is a list of (sequence, head, q-tile, cost) items in longest-first order.
//
// Cost of an item = number of bn-key tiles the kernel visits for its rows [m0, m1):
//   full head:   tiles 0 .. (m1-1)/bn
//   sparse head: sink tiles 0 .. ceil(min(sink, m1)/bn)-1 united with window tiles
//                max(0, m0-window+1)/bn .. (m1-1)/bn
// Both costs depend on (sequence, q-tile, mode) only, so the planner sorts "cells" -- one
// per (sequence, q-tile, cost) holding the heads of that cost in ascending order -- and
// expands them.  Cells are generated in (sequence, q-tile) order and sorted by cost with a
// stable counting sort, which yields exactly the order cost desc, (sequence, q-tile, head)
// asc.  Everything runs in one workgroup of 1024 threads; integer only, deterministic.
#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct Costs {
  int full, sparse;
};

__device__ __forceinline__ Costs tile_costs(int len, int qt, int bm, int bn, int sink,
                                            int window) {
  const int m0 = qt * bm, m1 = min(m0 + bm, len);
  const int t_hi = (m1 - 1) / bn;
  const int n_sink = ceil_div(min(sink, m1), bn);
  const int t_lo = max(0, m0 - window + 1) / bn;
  Costs c;
  c.full = t_hi + 1;
  c.sparse = n_sink >= t_lo ? t_hi + 1 : n_sink + (t_hi - t_lo + 1);
  return c;
}

// Block-wide exclusive scan of one int per thread; returns the prefix and the total.
__device__ int block_exclusive_scan(int v, int* total, int* scratch /* >= 32 ints */) {
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
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      const int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[kPlanThreads / 64] = run;
  }
  __syncthreads();
  const int excl = scratch[wave] + incl - v;
  *total = scratch[kPlanThreads / 64];
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int bins[kPlanMaxBins];   // histogram, then running start offset per cost
  __shared__ int scratch[32];
  const int tid = threadIdx.x;
  const int B = a.batch, Hq = a.n_heads_q;

  // Phase 1: per-sequence q-tile counts (exclusive prefix) and sparse-head counts.
  int carry = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int b = base + tid;
    int nq = 0;
    if (b < B) {
      const int len = a.cu[b + 1] - a.cu[b];
      nq = ceil_div(len, a.bm);
      int ns = 0;
      for (int h = 0; h < Hq; ++h) ns += a.route[(int64_t)b * Hq + h] != 0;
      a.n_sparse[b] = ns;
    }
    int tot;
    const int ex = block_exclusive_scan(nq, &tot, scratch);
    if (b < B) a.qt_prefix[b] = carry + ex;
    carry += tot;
  }
  if (tid == 0) a.qt_prefix[B] = carry;
  const int slots = carry;  // (sequence, q-tile) pairs
  for (int i = tid; i < a.bins; i += kPlanThreads) bins[i] = 0;
  __threadfence_block();
  __syncthreads();

  // Phase 2: two cell slots per (sequence, q-tile); histogram of cell costs.
  // cell = {seq, q_tile, cost, mode mask (1 full heads, 2 sparse heads)}; cost 0 = empty.
  for (int f = tid; f < slots; f += kPlanThreads) {
    int lo = 0, hi = B - 1;  // last b with qt_prefix[b] <= f
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.qt_prefix[mid] <= f) lo = mid; else hi = mid - 1;
    }
    const int b = lo, qt = f - a.qt_prefix[b];
    const int len = a.cu[b + 1] - a.cu[b];
    const Costs c = tile_costs(len, qt, a.bm, a.bn, a.sink, a.window);
    const int ns = a.n_sparse[b], nf = Hq - ns;
    int4 c0 = {b, qt, 0, 0}, c1 = {b, qt, 0, 0};
    if (nf > 0) {
      c0.z = c.full;
      c0.w = 1 | ((ns > 0 && c.sparse == c.full) ? 2 : 0);
      if (ns > 0 && c.sparse != c.full) { c1.z = c.sparse; c1.w = 2; }
    } else {
      c0.z = c.sparse;
      c0.w = 2;
    }
    a.cells[2 * f] = c0;
    a.cells[2 * f + 1] = c1;
    if (c0.z > 0) atomicAdd(&bins[c0.z], 1);
    if (c1.z > 0) atomicAdd(&bins[c1.z], 1);
  }
  __syncthreads();

  // Phase 3: start offset of every cost, costs in descending order (exclusive scan of the
  // reversed histogram, one contiguous run of bins per thread).
  {
    const int per = ceil_div(a.bins, kPlanThreads);
    const int lo = tid * per, hi = min(a.bins, lo + per);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += bins[a.bins - 1 - i];
    int tot;
    int run = block_exclusive_scan(s, &tot, scratch);
    for (int i = lo; i < hi; ++i) {
      const int cidx = a.bins - 1 - i;
      const int cnt = bins[cidx];
      bins[cidx] = run;
      run += cnt;
    }
  }
  __syncthreads();

  // Phase 4: stable scatter of the cells by cost, one wavefront walking the cells in slot
  // order 64 at a time.  Lanes with equal cost are ranked through ballots over the cost
  // bits; the first lane of every group advances that cost's start offset.
  const int n_cells = 2 * slots;
  if (tid < 64) {
    const int lane = tid;
    int nbits = 1;
    while ((1 << nbits) < a.bins) ++nbits;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < n_cells; base += 64) {
      const int idx = base + lane;
      int4 cell = {0, 0, 0, 0};
      if (idx < n_cells) cell = a.cells[idx];
      const bool valid = cell.z > 0;
      uint64_t eq = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (cell.z >> bit) & 1;
        const uint64_t m = __ballot(set);
        eq &= set ? m : ~m;
      }
      if (valid) {
        const int rank = __popcll(eq & below);
        const int start = bins[cell.z];
        a.sorted[start + rank] = cell;
        // make every lane read `start` before the group leader moves it
        __builtin_amdgcn_wave_barrier();
        if (rank == 0) bins[cell.z] = start + __popcll(eq);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __threadfence();
  __syncthreads();

  // Phase 5: item offset of every sorted cell (heads per cell), then expansion.
  int n_valid = 0;  // number of non-empty cells
  {
    int cnt = 0;
    for (int i = tid; i < n_cells; i += kPlanThreads) cnt += a.cells[i].z > 0;
    int tot;
    block_exclusive_scan(cnt, &tot, scratch);
    n_valid = tot;
  }
  int item_carry = 0;
  for (int base = 0; base < n_valid; base += kPlanThreads) {
    const int i = base + tid;
    int sz = 0;
    if (i < n_valid) {
      const int4 cell = a.sorted[i];
      const int ns = a.n_sparse[cell.x];
      sz = (cell.w & 1 ? Hq - ns : 0) + (cell.w & 2 ? ns : 0);
    }
    int tot;
    const int ex = block_exclusive_scan(sz, &tot, scratch);
    if (i < n_valid) a.cell_off[i] = item_carry + ex;
    item_carry += tot;
  }
  __threadfence();
  __syncthreads();
  for (int i = tid; i < n_valid; i += kPlanThreads) {
    const int4 cell = a.sorted[i];
    int at = a.cell_off[i];
    for (int h = 0; h < Hq; ++h) {
      const int mode = a.route[(int64_t)cell.x * Hq + h] != 0 ? 2 : 1;
      if (cell.w & mode) a.items[at++] = int4{cell.x, h, cell.y, cell.z};
    }
  }
  if (tid == 0) {
    a.counters[0] = item_carry;
    a.counters[1] = 0;
    if (a.n_items_out) *a.n_items_out = item_carry;
  }
}

__global__ void reset_queue_kernel(int32_t* queue) { *queue = 0; }

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  plan_kernel<<<1, kPlanThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_reset_queue(int32_t* queue, hipStream_t stream) {
  reset_queue_kernel<<<1, 1, 0, stream>>>(queue);
  return hipGetLastError();
}

}  // namespace ea
