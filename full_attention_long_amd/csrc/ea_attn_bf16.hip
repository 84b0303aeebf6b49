// ea_attn_bf16.hip -- persistent routed hybrid-attention prefill, bf16 in/out, CDNA4 MFMA.
//
// What it computes (Elastic Attention blog post, section 2.1 "Attention Router": r = 0
// runs Full Attention, r = 1 runs Sparse Attention, outputs concatenated per head;
// section 1 and the gist.science explanation, section "问题所在", for the sparse pattern,
// read here as attention sink + causal sliding window; section 3 "Fused Kernel": one
// launch serves both kinds of head, the routing arriving as metadata):
//   for every work item (sequence b, query head h, 256-row q-tile):
//     O[rows, h, :] = softmax(scale * Q K^T + mask) V over the item's visible keys.
//
// Design (gfx950; one workgroup per CU = 8 wavefronts x 32 query rows; 64-key tiles):
//   * Ping-pong.  Wavefronts 0-3 (group A, rows 0-127 of the item) and 4-7 (group B,
//     rows 128-255) share every K/V tile but run half a step apart: while one group is
//     in its GEMM phase (P(t-1) V(t-1) then S(t) = K(t) Q^T, 32 MFMAs) the other is in its
//     softmax phase (VALU), and the roles swap at every workgroup barrier.  Each SIMD
//     holds one wavefront of each group, so its matrix core and its VALU work at the same
//     time instead of one wavefront alternating between them; the GEMM-phase wavefront
//     runs at the higher wave priority (s_setprio), so its MFMAs and operand reads issue
//     first.  Each group has its own loop over the slots.
//   * Persistent grid: each workgroup pops items from the longest-first work list with
//     one atomic per item, so long full-head items start first and short sparse items
//     fill the tail of the launch.  The last workgroup out re-zeroes the queue.
//   * Sparse items visit only their sink tiles and window tiles.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with Q held in registers as the B operand,
//     so each lane owns one query row of S: the row max needs one cross-half exchange
//     (v_permlane32_swap) and the row sum stays lane-partial until the epilogue.
//   * O^T = V^T P^T on the same MFMA: P comes straight from the S accumulators (bf16)
//     as the B operand; the V^T operand is read with ds_read_b64_tr_b16 from a
//     row-major V tile, and the contraction order of keys is permuted consistently on
//     both operands to match the accumulator layout.
//   * K and V tiles reach LDS with direct buffer-to-LDS loads (no staging registers),
//     issued two phases before use into double buffers; 16-byte chunks are XOR-swizzled
//     per row so the b128 K reads (16 rows) and the transposing V reads (4 rows x 64 bytes
//     per half-wavefront) hit distinct banks of the 64-bank LDS.
//   * Softmax uses exp2 with log2(e) folded into the scale; all state is fp32.  P is
//     taken relative to a per-row reference max and rounded to bf16.  The row sums add
//     the rounded values on the matrix core: one v_mfma_f32_16x16x32_bf16 per 16-key
//     slice of P against a constant 0/1 selector, issued in the GEMM phase next to P V
//     (the vector unit's dot2 runs on the matrix pipeline too, and waits behind the
//     partner wavefront's MFMAs; the VALU keeps only what co-issues with them).  The
//     reference only has to keep P <= 2^8, i.e. no score more than 8 / (scale log2 e)
//     above it; a lane max over the tile (v_max3) checks that, and the row max, the O
//     and l rescale run only on the (rare) tiles that fail it.
//   * Masks are applied only on tiles that hide a pair of the wavefront's rows, in the
//     cheapest form the tile needs: causal edge only, window edge only, or both.
//   * Raw buffer loads/stores bound every access: keys past the sequence end read as
//     zero and rows past the tile end are not stored.
#include <climits>
#include <type_traits>

#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int BM = kBf16BM;      // 256 query rows per item
constexpr int BN = kBf16BN;      // 64 keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSubN = BN / 32;      // 32-key MFMA sub-tiles per key tile

template <int D>
struct Shape {
  static constexpr int CHUNKS = D / 8;                  // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;     // one K or V tile
  static constexpr int LDS_BYTES = 4 * TILE_BYTES;      // K and V, double buffered
  static constexpr int ROWS_PER_LOAD = 64 / CHUNKS;     // rows one wave-wide 16-B load fills
  static constexpr int LOADS = BN / ROWS_PER_LOAD / 4;  // per loading wave per tile, K or V
  static constexpr int KSTEPS = D / 16;                 // MFMA k-steps over the head dim
  static constexpr int DT = D / 32;                     // 32-wide output column tiles
  // XOR swizzles of the 16-byte chunk index, per row.  K: chunk ^ (row % CHUNKS) keeps
  // the 16 rows read by one b128 access in distinct banks.  V: chunk ^ 4*(row % 4)
  // keeps the 4 rows x 64 bytes read by one half-wave of ds_read_b64_tr_b16 distinct.
  static __device__ __forceinline__ int swz_k(int r) { return r & (CHUNKS - 1); }
  static __device__ __forceinline__ int swz_v(int r) { return (4 * r) & (CHUNKS - 1) & ~3; }
};

// Tile-visit plan of one item.  Tiles [0, n1) (sink) then [s2, t_hi] (window or causal); a
// piece of a split item visits entries [base, base + count) of that sequence.
struct Visit {
  int n1, s2, t_hi, count, base;
  __device__ __forceinline__ int tile(int n) const {
    n += base;
    return n < n1 ? n : s2 + (n - n1);
  }
};

__device__ __forceinline__ Visit make_visit(bool sparse, int m0, int m1, int sink, int window) {
  Visit v;
  v.t_hi = (m1 - 1) / BN;
  if (sparse) {
    v.n1 = (min(sink, m1) + BN - 1) / BN;
    const int t_lo = max(0, m0 - window + 1) / BN;
    v.s2 = max(t_lo, v.n1);
  } else {
    v.n1 = 0;
    v.s2 = 0;
  }
  v.count = v.n1 + max(0, v.t_hi - v.s2 + 1);
  v.base = 0;
  return v;
}

// make_rsrc on a base address and size the compiler is told are wavefront-uniform, so the
// descriptor lives in scalar registers (a descriptor it takes for divergent is wrapped in a
// loop over lanes at every buffer access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_u(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return make_rsrc((const void*)(uintptr_t)(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane(bytes));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  using S = Shape<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[S::LDS_BYTES];
  __shared__ int s_item;
  // K tiles at [0, 2*TILE_BYTES), V tiles after them; buffer `buf` at buf * TILE_BYTES
  unsigned char* const kbase = lds;
  unsigned char* const vbase = lds + 2 * S::TILE_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);  // wave-uniform: group branches are scalar
  const int grp = wave >> 2;                  // ping-pong group: 0 = A, 1 = B
  const int row0 = 32 * wave;                 // first item row of this wavefront
  const int l32 = lane & 31, g = lane >> 5;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv;
  const int group = Hq / Hkv;
  const int n_items = min(*a.n_items, a.item_cap);
  const int total_tokens = a.cu[a.batch];
  const float c_log2 = a.scale * 1.4426950408889634f;  // scale * log2(e)
  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;

  // direct global -> LDS loads: load i of this wavefront fills rows lg*ROWS_PER_LOAD ..
  // (lg = wave*LOADS + i); lane fills physical chunk `pc` of row lg*ROWS_PER_LOAD + lrow
  // with the logical chunk the swizzle places there.  The lane part of the byte offset is
  // fixed for the kernel; the tile and row-group part is uniform (scalar offset).
  const int lrow = lane / S::CHUNKS, pc = lane % S::CHUNKS;
  // V^T operand (ds_read_b64_tr_b16): source row/column inside a 16-key x 32-column block
  const int tr_row = 4 * g + (lane & 15) / 4;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // Selector A operand of the row-sum MFMA (16x16x32): D[i][n] = sum over the four 8-key
  // blocks of B, weighted by A[i][block].  B is a P operand, whose lane n + 16 blk holds
  // query row n + 16 (blk % 2), keys of half blk / 2; output lane l holds D[4 (l / 16) + e]
  // [l % 16] and owns query row l % 32 = l % 16 + 16 ((l / 16) % 2).  So A[i][blk] = 1 iff
  // blk % 2 == (i / 4) % 2, and A's lane l (row l % 16, block l / 16) holds that for all 8
  // elements: every output of lane l is the sum over both halves of its own row.
  bf16x8 rsel;
  {
    const __bf16 one = (__bf16)((((lane >> 4) & 1) == ((lane >> 2) & 1)) ? 1.0f : 0.0f);
#pragma unroll
    for (int e = 0; e < 8; ++e) rsel[e] = one;
  }

  for (;;) {
    if (tid == 0) s_item = atomicAdd(&a.queue[0], 1);
    __syncthreads();
    // the item index is uniform: keeping it (and so the item, its tile plan and the
    // buffer offsets) in scalar registers keeps the direct-to-LDS loads' offsets scalar
    int it = uniform(s_item);
    int piece = 0, n_pieces = 1;
    if (a.piece_prefix) {
      // split-KV: the queue hands out pieces; piece `it` belongs to the last item whose first
      // piece is <= it
      const int v = it;
      if (v < 0 || v >= min(*a.n_pieces, a.piece_prefix[n_items])) break;
      int lo = 0, hi = n_items - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.piece_prefix[mid] <= v) lo = mid; else hi = mid - 1;
      }
      it = uniform(lo);
      piece = uniform(v - a.piece_prefix[it]);
      n_pieces = uniform(a.piece_prefix[it + 1] - a.piece_prefix[it]);
    } else if (it < 0 || it >= n_items) {  // a corrupt queue head ends the loop too
      break;
    }
    const int4 item = a.items[it];
    const int b = uniform(item.x), h = uniform(item.y), qt = uniform(item.z);
    // an item outside this call's sizes is skipped (the test is uniform across the
    // workgroup; the barrier keeps s_item stable until every thread has read it)
    // (and so is an item of a chunk longer than its key sequence)
    if (b < 0 || b >= a.batch || h < 0 || h >= Hq || qt < 0 || qt * BM >= a.cu[b + 1] - a.cu[b] ||
        (a.cu_k && a.cu_k[b + 1] - a.cu_k[b] < a.cu[b + 1] - a.cu[b])) {
      __syncthreads();
      continue;
    }
    const int seq0 = a.cu[b];
    const int len = a.cu[b + 1] - seq0;
    // keys: the sequence's own packing, or the KV-prefix packing of a chunked prefill, whose
    // query rows are the last `len` of its len_k positions (row r at position off + r)
    const int seq0k = a.cu_k ? uniform(a.cu_k[b]) : seq0;
    const int len_k = a.cu_k ? uniform(a.cu_k[b + 1]) - seq0k : len;
    const int off = len_k - len;
    // m0, m1, wr0, wr1 and qi below are positions in the sequence; the item's chunk rows
    // are [m0 - off, m1 - off)
    const int m0 = off + qt * BM, m1 = off + min(qt * BM + BM, len);
    const int kvh = h / group;
    const bool sparse = uniform(a.route[(int64_t)b * Hq + h]) != 0;
    Visit vis = make_visit(sparse, m0, m1, a.sink, a.window);
    vis.n1 = uniform(vis.n1);
    vis.s2 = uniform(vis.s2);
    vis.t_hi = uniform(vis.t_hi);
    if (n_pieces > 1) {  // this piece's share of the plan (every piece gets >= 1 tile)
      const int lo_n = piece * vis.count / n_pieces, hi_n = (piece + 1) * vis.count / n_pieces;
      vis.base = lo_n;
      vis.count = hi_n - lo_n;
    }
    vis.count = uniform(vis.count);
    vis.base = uniform(vis.base);
    const int wr0 = m0 + row0, wr1 = min(wr0 + 32, m1);  // this wavefront's rows

    // buffer windows: this item's Q/O rows of head h; this sequence's K/V of head kvh
    const int64_t qo_elem = ((int64_t)(seq0 + qt * BM) * Hq + h) * D;
    const uint32_t qo_bytes = (uint32_t)(m1 - m0 - 1) * q_row_bytes + D * 2;
    const auto qr = make_rsrc_u((const __bf16*)a.q + qo_elem, qo_bytes);
    const auto orr = make_rsrc_u((__bf16*)a.o + qo_elem, qo_bytes);
    const int64_t kv_elem = ((int64_t)seq0k * Hkv + kvh) * D;
    const uint32_t kv_bytes = (uint32_t)(len_k - 1) * kv_row_bytes + D * 2;
    const auto kr = make_rsrc_u((const __bf16*)a.k + kv_elem, kv_bytes);
    const auto vr = make_rsrc_u((const __bf16*)a.v + kv_elem, kv_bytes);

    // Issue the direct-to-LDS loads of one K or V tile into a buffer.  Only the four
    // wavefronts of group B issue tile loads (in the slots where they run the softmax
    // phase, which reads no LDS); each fills LOADS groups of ROWS_PER_LOAD rows.
    auto load_tile = [&](const __amdgpu_buffer_rsrc_t& rs, unsigned char* dst, int kt,
                         bool is_v) __attribute__((always_inline)) {
      // the wavefront and tile indices are uniform; readfirstlane keeps the row offset
      // scalar (the compiler cannot prove it and would otherwise loop over lanes)
      const int wv = uniform(wave & 3);
      kt = uniform(kt);
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i) {
        const int lg = wv * S::LOADS + i;
        const uint32_t row_base =
            (uint32_t)uniform((int)((uint32_t)(kt * BN + lg * S::ROWS_PER_LOAD) * kv_row_bytes));
        const int r = ((wave & 3) * S::LOADS + i) * S::ROWS_PER_LOAD + lrow;
        const int chunk = pc ^ (is_v ? S::swz_v(r) : S::swz_k(r));
        const uint32_t lane_off = (uint32_t)lrow * kv_row_bytes + (uint32_t)(chunk * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + lg * 1024), 16,
                                                 lane_off, row_base, 0, 0);
      }
    };

    // Q as the B operand: lane holds query row (row0 + l32), head-dim elements
    // 16*ks + 8*g .. +7 for every k-step ks.
    bf16x8 qreg[S::KSTEPS];
    {
      const uint32_t row_off = (uint32_t)(row0 + l32) * q_row_bytes;
#pragma unroll
      for (int ks = 0; ks < S::KSTEPS; ++ks)
        qreg[ks] = __builtin_bit_cast(bf16x8, buf_load16(qr, row_off + (16 * ks + 8 * g) * 2));
    }
    const int qi = wr0 + l32;  // this lane's query position in the sequence

    f32x16 oacc[S::DT];
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m_ref = -INFINITY;  // reference max (score units), equal on both lanes of a row
    float m_thr = -INFINITY;  // scores below m_ref + 8 / c_log2 give P < 2^8
    float m_c = 0.f;          // the reference in exp2 units (0 while there is none)
    // row sum of the bf16-rounded P: every lane holds its query row's sum four times
    f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
    f32x16 sacc[kSubN];   // S(t) from the GEMM phase, consumed by the softmax phase
    bf16x8 pb[kSubN][2];  // P(t) from the softmax phase, consumed by the next GEMM phase
#pragma unroll
    for (int j = 0; j < kSubN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[j][r] = 0.f;

    // GEMM phase X(t): O^T += V(t-1)^T P(t-1)^T, then S^T(t) = K(t) Q^T: 8 stages of KH
    // MFMAs, 4 KH operands read from LDS.  Operand i is read RING - 1 MFMAs before the MFMA
    // that uses it, into a ring of RING registers; sched_barrier after every MFMA keeps each
    // read where it is issued, so the LDS reads trickle in one per MFMA rather than in
    // bursts, and one wavefront keeps the matrix core busy on its own while its partner
    // wavefront runs the softmax.  (A ring of 4 ran about 1% faster than reading a whole
    // stage ahead in bursts, bit-identical; rings of 5 to 8 were no better.)
    // pv / qk: std::true_type or std::false_type (which of the two products to run)
    auto gemm_phase = [&](int t, auto pv, auto qk) __attribute__((always_inline)) {
      constexpr bool do_pv = decltype(pv)::value, do_qk = decltype(qk)::value;
      // the wavefront feeding the matrix core wins issue arbitration over its partner's
      // softmax (2.5-3.5% faster on the prefill workloads than equal priorities)
      __builtin_amdgcn_s_setprio(1);
      const unsigned char* vb = vbase + ((t - 1) & 1) * S::TILE_BYTES;
      const unsigned char* kb = kbase + (t & 1) * S::TILE_BYTES;
      constexpr int KH = S::KSTEPS / 2;
      static_assert(S::DT == KH, "stages hold DT V operands or KSTEPS/2 K operands");
      constexpr int RING = 4;
      // operand i = KH c + q of stage c: for c < 4 the V^T operand of column tile q and
      // 16-key slice (j, kh) = (c / 2, c % 2) (P keys 32j + 16kh + 8(e/4) + 4g + e%4), read
      // transposed from the row-major V tile; for c >= 4 the K operand of sub-tile
      // j = (c - 4) / 2, k-step KH ((c - 4) % 2) + q
      auto read1 = [&](int i, bf16x8& o) __attribute__((always_inline)) {
        const int c = i / KH, q = i % KH;
        if (c < 4) {
          const int j = c / 2, kh = c % 2;
          const int row = 32 * j + 16 * kh + tr_row;
          const int col = 32 * q + tr_col;  // element column; rows row and row + 8
          const unsigned char* p0 =
              vb + row * S::ROW_BYTES + (((col / 8) ^ S::swz_v(row)) * 16) + (col % 8) * 2;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * S::ROW_BYTES));
          o = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          const int j = (c - 4) / 2, k0 = KH * ((c - 4) % 2);
          const int row = 32 * j + l32;
          o = *(const bf16x8*)(kb + row * S::ROW_BYTES +
                               (((2 * (k0 + q) + g) ^ S::swz_k(row)) * 16));
        }
      };
      // sacc[j][r] = score(key kt*BN + 32j + 8(r/4) + 4g + r%4, query qi); the row sums of
      // each 16-key slice of P run on the matrix core after its last P V MFMA
      auto run1 = [&](int i, const bf16x8& o) __attribute__((always_inline)) {
        const int c = i / KH, q = i % KH;
        if (c < 4) {
          const int j = c / 2, kh = c % 2;
          oacc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, pb[j][kh], oacc[q], 0, 0, 0);
          if (q == KH - 1)
            lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rsel, pb[j][kh], lacc, 0, 0, 0);
        } else {
          const int j = (c - 4) / 2, k0 = KH * ((c - 4) % 2);
          if (k0 == 0 && q == 0)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[j][r] = 0.f;
          sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, qreg[k0 + q], sacc[j], 0, 0, 0);
        }
      };
      constexpr int i0 = (do_pv ? 0 : 4) * KH, i1 = (do_qk ? 8 : 4) * KH;
      bf16x8 ring[RING];
#pragma unroll
      for (int m = 0; m < RING - 1; ++m)
        if (i0 + m < i1) read1(i0 + m, ring[m]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = i0; i < i1; ++i) {
        if (i + RING - 1 < i1) read1(i + RING - 1, ring[(i - i0 + RING - 1) % RING]);
        run1(i, ring[(i - i0) % RING]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Softmax phase Y(t).  P(t) = exp2(S*c - m_ref*c) is taken relative to the row's
    // reference max m_ref and rounded to bf16, the operand of P V and of the row sum.  The
    // reference has to keep every P <= 2^8, i.e. every score below m_thr; only when some
    // lane's tile max is not below it (or there is no reference yet) does the wavefront
    // take the exact path: row max, new reference for every row, O and l rescaled.
    auto compute_p = [&](float mc) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < kSubN; ++j)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][r], c_log2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][r + 1], c_log2, -mc));
          const bf16x2 w = {(__bf16)p0, (__bf16)p1};
          pb[j][r / 8][r % 8] = w[0];
          pb[j][r / 8][r % 8 + 1] = w[1];
        }
    };
    auto softmax_phase = [&](int t) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(0);
      const int kt = vis.tile(t);
      const int k0 = kt * BN;
      // hidden pairs in this tile for this wavefront's rows: past the diagonal (or past
      // the sequence end), or below the window start of a sparse row outside the sink
      const bool m_causal = k0 + BN - 1 > wr0;
      const bool m_win = sparse && k0 + BN > a.sink && k0 <= wr1 - 1 - a.window;
      if (m_causal && !m_win) {
        const int lim = qi - k0;  // key k0 + off is visible iff off <= lim
#pragma unroll
        for (int j = 0; j < kSubN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * j + 8 * (r / 4) + 4 * g + (r % 4);
            sacc[j][r] = off <= lim ? sacc[j][r] : -INFINITY;
          }
      } else if (m_win && !m_causal && k0 >= a.sink) {
        const int wlo = qi - a.window + 1 - k0;  // visible iff off >= wlo
#pragma unroll
        for (int j = 0; j < kSubN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * j + 8 * (r / 4) + 4 * g + (r % 4);
            sacc[j][r] = off >= wlo ? sacc[j][r] : -INFINITY;
          }
      } else if (m_causal || m_win) {
        // general: off <= lim and, for a sparse head, (off >= wlo or off < slim)
        const int lim = qi - k0;
        const int wlo = sparse ? qi - a.window + 1 - k0 : INT_MIN;
        const int slim = sparse ? a.sink - k0 : INT_MIN;
#pragma unroll
        for (int j = 0; j < kSubN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * j + 8 * (r / 4) + 4 * g + (r % 4);
            const bool visible = (off <= lim) & ((off >= wlo) | (off < slim));
            sacc[j][r] = visible ? sacc[j][r] : -INFINITY;
          }
      }
      // lane max of the tile: four chains of 3-input maxima
      float mx[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = q / 2, r = 8 * (q % 2);
        float m = fmaxf(fmaxf(sacc[j][r], sacc[j][r + 1]), sacc[j][r + 2]);
        m = fmaxf(fmaxf(m, sacc[j][r + 3]), sacc[j][r + 4]);
        m = fmaxf(fmaxf(m, sacc[j][r + 5]), sacc[j][r + 6]);
        mx[q] = fmaxf(m, sacc[j][r + 7]);
      }
      float mt = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
      if (__builtin_amdgcn_ballot_w64(!(mt < m_thr)) != 0) {
        // row max across the two lanes of the row
        mt = fmaxf(mt, xor32(mt));
        const float m_new = fmaxf(m_ref, mt);
        // alpha = 0 when there was no reference yet (O and l are still zero)
        const float alpha =
            m_new == m_ref ? 1.0f : __builtin_amdgcn_exp2f((m_ref - m_new) * c_log2);
        lacc *= alpha;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        m_ref = m_new;
        m_thr = m_ref + 8.0f / c_log2;
        m_c = (m_ref == -INFINITY ? 0.f : m_ref) * c_log2;
      }
      compute_p(m_c);
    };

    // Slot schedule.  Tiles t = 0..N-1.  Group A runs X(t) in slot 2t and Y(t) in slot
    // 2t+1; group B runs Y(t-1) in slot 2t and X(t) in slot 2t+1; X(N) is the last P V.
    // K(t) is read in slots 2t, 2t+1 and V(t) in slots 2t+2, 2t+3; group B loads both at
    // the start of slot 2t-2 (K) / 2t (V), while it runs a softmax phase, into the buffer
    // freed by the barrier before.  Group B's next GEMM phase, one slot later, is the first
    // LDS read after its loads (the compiler waits for them there: the DMA writes may alias
    // any LDS read), and every odd slot ends with a full wait, so a load never stalls the
    // GEMM phase of the slot that issued it.  Each group runs its own loop over the slots
    // (the wavefront index is uniform, so the split is a scalar branch): no slot picks one
    // of two phases at run time, which keeps both loop bodies straight-line code that the
    // register allocator handles without spills.
    const int N = vis.count;  // >= 1 for every valid item
    const std::true_type yes;
    const std::false_type no;
    // group B issues K(u+1) and V(u) at the start of slot 2u
    auto issue_loads = [&](int u) __attribute__((always_inline)) {
      if (u + 1 < N) load_tile(kr, kbase + ((u + 1) & 1) * S::TILE_BYTES, vis.tile(u + 1), false);
      load_tile(vr, vbase + (u & 1) * S::TILE_BYTES, vis.tile(u), true);
    };
    auto end_even = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): LDS reads of this slot are done
      __builtin_amdgcn_s_barrier();
    };
    auto end_odd = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0);  // this slot's LDS reads and the loads of slot s-1
      __syncthreads();
    };
    if (grp == 1) load_tile(kr, kbase, vis.tile(0), false);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Each group runs its own slot sequence (2N + 2 slots, the same barriers): no slot
    // chooses between the two phases, so each loop body is straight-line code.
    if (grp == 0) {
      // group A: X(u) in slot 2u, Y(u) in slot 2u+1
      gemm_phase(0, no, yes);
      end_even();
      softmax_phase(0);
      end_odd();
      for (int u = 1; u < N; ++u) {
        gemm_phase(u, yes, yes);
        end_even();
        softmax_phase(u);
        end_odd();
      }
      gemm_phase(N, yes, no);
      end_even();
      end_odd();
    } else {
      // group B: Y(u-1) and the loads of K(u+1), V(u) in slot 2u, X(u) in slot 2u+1
      issue_loads(0);
      end_even();
      gemm_phase(0, no, yes);
      end_odd();
      for (int u = 1; u < N; ++u) {
        issue_loads(u);
        softmax_phase(u - 1);
        end_even();
        gemm_phase(u, yes, yes);
        end_odd();
      }
      softmax_phase(N - 1);
      end_even();
      gemm_phase(N, yes, no);
      end_odd();
    }

    // ---- epilogue of a piece of a split item: unnormalised O, the row's reference max and
    // sum, in fp32, to the piece's slot (merged by the combine kernel)
    if (n_pieces > 1) {
      const float l_tot = lacc[0];
      const int64_t slot = a.slot_base[it] + piece;
      const int row = row0 + l32;
      float* op = a.o_part + (slot * BM + row) * D;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x4 w = {oacc[dt][4 * rq + 0], oacc[dt][4 * rq + 1], oacc[dt][4 * rq + 2],
                           oacc[dt][4 * rq + 3]};
          *(f32x4*)(op + 32 * dt + 8 * rq + 4 * g) = w;
        }
      if (g == 0) {
        a.ml_part[(slot * BM + row) * 2 + 0] = m_ref;
        a.ml_part[(slot * BM + row) * 2 + 1] = l_tot;
      }
      __syncthreads();  // s_item and the LDS tiles are reused by the next item
      continue;
    }
    // ---- epilogue: O = O / l, round to bf16, store this lane's query row
    const float l_tot = lacc[0];
    const float inv = 1.0f / l_tot;
    const uint32_t row_off = (uint32_t)(row0 + l32) * q_row_bytes;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * dt + 8 * rq + 4 * g;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[dt][4 * rq + 0] * inv, oacc[dt][4 * rq + 1] * inv);
        w[1] = pack_bf16x2(oacc[dt][4 * rq + 2] * inv, oacc[dt][4 * rq + 3] * inv);
        buf_store8(orr, row_off + d0 * 2, w);
      }
    if (a.lse && g == 0 && qi < m1) {
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      a.lse[(int64_t)h * total_tokens + seq0 + (qi - off)] = m_use * a.scale + logf(l_tot);
    }
    __syncthreads();  // s_item and the LDS tiles are reused by the next item
  }
  // The last workgroup out leaves the queue counters at zero for the next launch.
  if (tid == 0 && atomicAdd(&a.queue[1], 1) == (int)gridDim.x - 1) {
    atomicExch(&a.queue[0], 0);
    atomicExch(&a.queue[1], 0);
  }
}

// Merge of a split item's pieces: for each of its rows, M = max of the pieces' reference
// maxima, w_p = 2^((m_p - M) * scale * log2 e), O = sum_p O_p w_p / sum_p l_p w_p (fp32, one
// bf16 rounding), LSE = M * scale + ln sum_p l_p w_p.  One workgroup per (split item, block
// of 256 / (D / 4) rows); a thread takes 4 head dimensions of one row and issues the loads
// of every piece before the first use (one memory round trip for the maxima and sums, one
// for the partial outputs), then adds the pieces in order.
template <int D>
constexpr int combine_rows() { return 256 / (D / 4); }
template <int D>
__global__ __launch_bounds__(256) void split_combine_kernel(AttnArgs a, const int32_t* split_list,
                                                            const int32_t* n_split) {
  const int k = blockIdx.x, rblk = blockIdx.y;
  if (k >= min(*n_split, kSplitSlots)) return;
  const int it = split_list[k];
  const int4 item = a.items[it];
  const int b = item.x, h = item.y, qt = item.z;
  const int Hq = a.n_heads_q;
  const int seq0 = a.cu[b];
  const int len = a.cu[b + 1] - seq0;
  const int r0 = qt * BM, nrows = min(BM, len - r0);
  constexpr int C4 = D / 4;
  const int c = threadIdx.x % C4;
  const int r = rblk * combine_rows<D>() + threadIdx.x / C4;
  if (r >= nrows) return;
  const int ns = min(a.piece_prefix[it + 1] - a.piece_prefix[it], kSplitMaxPieces);
  const int64_t slot0 = a.slot_base[it];
  const int total_tokens = a.cu[a.batch];
  const float c_log2 = a.scale * 1.4426950408889634f;
  float mp[kSplitMaxPieces], lp[kSplitMaxPieces];
  f32x4 op[kSplitMaxPieces];
#pragma unroll
  for (int p = 0; p < kSplitMaxPieces; ++p)
    if (p < ns) {
      mp[p] = a.ml_part[((slot0 + p) * BM + r) * 2];
      lp[p] = a.ml_part[((slot0 + p) * BM + r) * 2 + 1];
      op[p] = *(const f32x4*)(a.o_part + ((slot0 + p) * BM + r) * D + 4 * c);
    }
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kSplitMaxPieces; ++p)
    if (p < ns) M = fmaxf(M, mp[p]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < kSplitMaxPieces; ++p)
    if (p < ns) {
      const float m = mp[p];
      const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - Mu) * c_log2);
      l += lp[p] * w;
      acc += w * op[p];
    }
  const float inv = 1.0f / l;
  __bf16* o = (__bf16*)a.o + ((int64_t)(seq0 + r0 + r) * Hq + h) * D + 4 * c;
  u32x2 wv;
  wv[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  wv[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(u32x2*)o = wv;
  if (a.lse && c == 0) a.lse[(int64_t)h * total_tokens + seq0 + r0 + r] = Mu * a.scale + logf(l);
}

}  // namespace

int attn_bf16_blocks_per_cu() { return 1; }

hipError_t launch_split_combine(const AttnArgs& a, const int32_t* split_list,
                                const int32_t* n_split, hipStream_t stream) {
  // at most kSplitSlots / 2 split items (each has >= 2 pieces), BM / combine_rows row blocks
  if (a.head_dim == 128)
    split_combine_kernel<128><<<dim3(kSplitSlots / 2, BM / combine_rows<128>()), 256, 0, stream>>>(
        a, split_list, n_split);
  else
    split_combine_kernel<64><<<dim3(kSplitSlots / 2, BM / combine_rows<64>()), 256, 0, stream>>>(
        a, split_list, n_split);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, int grid, hipStream_t stream) {
  if (a.head_dim == 128)
    attn_bf16_kernel<128><<<grid, kThreads, 0, stream>>>(a);
  else
    attn_bf16_kernel<64><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ea
