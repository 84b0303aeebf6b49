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
//     time instead of one wavefront alternating between them.
//   * Persistent grid: each workgroup pops items from the longest-first work list with
//     one atomic per item, so long full-head items start first and short sparse items
//     fill the tail of the launch.  The last workgroup out re-zeroes the queue.
//   * Sparse items visit only their sink tiles and window tiles; the element mask is
//     branch-free and applied only on tiles that are not fully visible for a wavefront.
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
//     taken relative to the new running max (its largest entry is exactly 1); the
//     O *= alpha pass runs only when some row of the wavefront finds a new maximum.
//   * Raw buffer loads/stores bound every access: keys past the sequence end read as
//     zero and rows past the tile end are not stored.
#include <climits>

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
  static constexpr int LOADS = BN / ROWS_PER_LOAD / kWaves;  // per wave per tile, K or V
  static constexpr int KSTEPS = D / 16;                 // MFMA k-steps over the head dim
  static constexpr int DT = D / 32;                     // 32-wide output column tiles
  // XOR swizzles of the 16-byte chunk index, per row.  K: chunk ^ (row % CHUNKS) keeps
  // the 16 rows read by one b128 access in distinct banks.  V: chunk ^ 4*(row % 4)
  // keeps the 4 rows x 64 bytes read by one half-wave of ds_read_b64_tr_b16 distinct.
  static __device__ __forceinline__ int swz_k(int r) { return r & (CHUNKS - 1); }
  static __device__ __forceinline__ int swz_v(int r) { return (4 * r) & (CHUNKS - 1) & ~3; }
};

// Tile-visit plan of one item.  Tiles [0, n1) (sink) then [s2, t_hi] (window or causal).
struct Visit {
  int n1, s2, t_hi, count;
  __device__ __forceinline__ int tile(int n) const { return n < n1 ? n : s2 + (n - n1); }
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
  return v;
}

// True if some (row, key) pair of the tile is hidden for rows [r0, r1).
__device__ __forceinline__ bool tile_needs_mask(int kt, bool sparse, int r0, int r1, int sink,
                                                int window) {
  const int k0 = kt * BN, k1 = k0 + BN;
  if (k1 - 1 > r0) return true;                       // causal edge (or keys past the end)
  if (!sparse) return false;
  return !(k1 <= sink || k0 > r1 - 1 - window);       // neither all-sink nor all-window
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
  const int wave = tid >> 6;
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

  for (;;) {
    if (tid == 0) s_item = atomicAdd(&a.queue[0], 1);
    __syncthreads();
    const int it = s_item;
    if (it >= n_items) break;
    const int4 item = a.items[it];
    const int b = item.x, h = item.y, qt = item.z;
    // an item outside this call's sizes is skipped (the test is uniform across the
    // workgroup; the barrier keeps s_item stable until every thread has read it)
    if (b < 0 || b >= a.batch || h < 0 || h >= Hq || qt < 0 || qt * BM >= a.cu[b + 1] - a.cu[b]) {
      __syncthreads();
      continue;
    }
    const int seq0 = a.cu[b];
    const int len = a.cu[b + 1] - seq0;
    const int m0 = qt * BM, m1 = min(m0 + BM, len);
    const int kvh = h / group;
    const bool sparse = a.route[(int64_t)b * Hq + h] != 0;
    const Visit vis = make_visit(sparse, m0, m1, a.sink, a.window);
    const int wr0 = m0 + row0, wr1 = min(wr0 + 32, m1);  // this wavefront's rows

    // buffer windows: this item's Q/O rows of head h; this sequence's K/V of head kvh
    const int64_t qo_elem = ((int64_t)(seq0 + m0) * Hq + h) * D;
    const uint32_t qo_bytes = (uint32_t)(m1 - m0 - 1) * q_row_bytes + D * 2;
    const auto qr = make_rsrc((const __bf16*)a.q + qo_elem, qo_bytes);
    const auto orr = make_rsrc((__bf16*)a.o + qo_elem, qo_bytes);
    const int64_t kv_elem = ((int64_t)seq0 * Hkv + kvh) * D;
    const uint32_t kv_bytes = (uint32_t)(len - 1) * kv_row_bytes + D * 2;
    const auto kr = make_rsrc((const __bf16*)a.k + kv_elem, kv_bytes);
    const auto vr = make_rsrc((const __bf16*)a.v + kv_elem, kv_bytes);

    // Issue the direct-to-LDS loads of one K or V tile into a buffer: each of the 8
    // wavefronts fills LOADS groups of ROWS_PER_LOAD rows.
    auto load_tile = [&](const __amdgpu_buffer_rsrc_t& rs, unsigned char* dst, int kt,
                         bool is_v) {
      // the wavefront index is uniform; readfirstlane lets the scalar offset stay scalar
      const int wv = uniform(wave);
#pragma unroll
      for (int i = 0; i < S::LOADS; ++i) {
        const int lg = wv * S::LOADS + i;
        const uint32_t row_base = (uint32_t)(kt * BN + lg * S::ROWS_PER_LOAD) * kv_row_bytes;
        const int r = (wave * S::LOADS + i) * S::ROWS_PER_LOAD + lrow;
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
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 sacc[kSubN];   // S(t) from the GEMM phase, consumed by the softmax phase
    bf16x8 pb[kSubN][2];  // P(t) from the softmax phase, consumed by the next GEMM phase
#pragma unroll
    for (int j = 0; j < kSubN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[j][r] = 0.f;

    // GEMM phase X(t): O^T += V(t-1)^T P(t-1)^T, then S^T(t) = K(t) Q^T, as 8 stages of 4
    // MFMAs.  The LDS operands of stage i+1 are read during stage i (sched_barrier keeps
    // the compiler from sinking the reads next to their MFMAs), so one wavefront keeps
    // the matrix core busy on its own while its partner wavefront runs the softmax.
    auto gemm_phase = [&](int t, int N) {
      const bool do_pv = t >= 1, do_qk = t < N;
      const unsigned char* vb = vbase + ((t - 1) & 1) * S::TILE_BYTES;
      const unsigned char* kb = kbase + (t & 1) * S::TILE_BYTES;
      constexpr int KH = S::KSTEPS / 2;
      static_assert(S::DT == KH, "stages hold DT V operands or KSTEPS/2 K operands");
      // stage c < 4: V^T operands of 16-key slice (j, kh) = (c / 2, c % 2), all column
      // tiles (P keys 32j + 16kh + 8(e/4) + 4g + e%4); stage c >= 4: K operands of
      // sub-tile j = (c - 4) / 2, k-steps KH*((c - 4) % 2) + [0, KH).
      auto read_ops = [&](int c, bf16x8 (&op)[KH]) {
        if (c < 4) {
          const int j = c / 2, kh = c % 2;
          const int row = 32 * j + 16 * kh + tr_row;
#pragma unroll
          for (int dt = 0; dt < S::DT; ++dt) {
            const int col = 32 * dt + tr_col;  // element column; rows row and row + 8
            const unsigned char* p0 =
                vb + row * S::ROW_BYTES + (((col / 8) ^ S::swz_v(row)) * 16) + (col % 8) * 2;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
            const s16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * S::ROW_BYTES));
            op[dt] = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        } else {
          const int j = (c - 4) / 2, k0 = KH * ((c - 4) % 2);
          const int row = 32 * j + l32;
#pragma unroll
          for (int q = 0; q < KH; ++q)
            op[q] = *(const bf16x8*)(kb + row * S::ROW_BYTES +
                                     (((2 * (k0 + q) + g) ^ S::swz_k(row)) * 16));
        }
      };
      // sacc[j][r] = score(key kt*BN + 32j + 8(r/4) + 4g + r%4, query qi)
      auto run_ops = [&](int c, const bf16x8 (&op)[KH]) {
        if (c < 4) {
          const int j = c / 2, kh = c % 2;
#pragma unroll
          for (int dt = 0; dt < S::DT; ++dt)
            oacc[dt] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[dt], pb[j][kh], oacc[dt], 0, 0, 0);
        } else {
          const int j = (c - 4) / 2, k0 = KH * ((c - 4) % 2);
          if (k0 == 0)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[j][r] = 0.f;
#pragma unroll
          for (int q = 0; q < KH; ++q)
            sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[q], qreg[k0 + q], sacc[j], 0, 0, 0);
        }
      };
      const int c0 = do_pv ? 0 : 4, c1 = do_qk ? 8 : 4;
      bf16x8 opa[KH], opb[KH];
      read_ops(c0, opa);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < 8; c += 2) {
        if (c < c0 || c >= c1) continue;
        if (c + 1 < c1) read_ops(c + 1, opb);
        run_ops(c, opa);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 1 >= c1) break;
        if (c + 2 < c1) read_ops(c + 2, opa);
        run_ops(c + 1, opb);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Softmax phase Y(t): mask, running max, P(t) = exp2(S*c - m*c) as bf16, row sums,
    // rescale of O when the max moved.
    auto softmax_phase = [&](int t) {
      const int kt = vis.tile(t);
      if (tile_needs_mask(kt, sparse, wr0, wr1, a.sink, a.window)) {
        // key kt*BN + off is visible iff off <= qi - kbase and, for a sparse head,
        // (off >= qi - window + 1 - kbase or off < sink - kbase)
        const int kbase_key = kt * BN;
        const int lim = qi - kbase_key;
        const int wlo = sparse ? qi - a.window + 1 - kbase_key : INT_MIN;
        const int slim = sparse ? a.sink - kbase_key : INT_MIN;
#pragma unroll
        for (int j = 0; j < kSubN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * j + 8 * (r / 4) + 4 * g + (r % 4);
            const bool visible = (off <= lim) & ((off >= wlo) | (off < slim));
            sacc[j][r] = visible ? sacc[j][r] : -INFINITY;
          }
      }
      // row max and row sum as 8-way trees (short dependency chains)
      float mx[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) mx[i] = fmaxf(sacc[i / 4][4 * (i % 4)], sacc[i / 4][4 * (i % 4) + 1]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        mx[i] = fmaxf(mx[i], fmaxf(sacc[i / 4][4 * (i % 4) + 2], sacc[i / 4][4 * (i % 4) + 3]));
      float mt = fmaxf(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])),
                       fmaxf(fmaxf(mx[4], mx[5]), fmaxf(mx[6], mx[7])));
      mt = fmaxf(mt, xor32(mt));
      const float m_new = fmaxf(m_run, mt);
      const float mc = (m_new == -INFINITY ? 0.f : m_new) * c_log2;
      float ps[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ps[i] = 0.f;
#pragma unroll
      for (int j = 0; j < kSubN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][r], c_log2, -mc));
          ps[(16 * j + r) % 8] += p;
          pb[j][r / 8][r % 8] = (__bf16)p;
        }
      const float psum = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
      // rescale O and l when some row of the wavefront has a new max (alpha = 1 elsewhere)
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
        const float alpha =
            m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f((m_run - m_new) * c_log2);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }
      l_run += psum;
      m_run = m_new;
    };

    // Slot schedule.  Tiles t = 0..N-1.  Group A runs X(t) in slot 2t and Y(t) in slot
    // 2t+1; group B runs Y(t-1) in slot 2t and X(t) in slot 2t+1; X(N) is the last P V.
    // K(t) is read in slots 2t, 2t+1 and V(t) in slots 2t+2, 2t+3; both are loaded at the
    // start of slot 2t-2 (K) / 2t (V) into the buffer freed two slots earlier, and every
    // odd slot ends with a full wait, so each load has two slots to land.
    const int N = vis.count;
    load_tile(kr, kbase, vis.tile(0), false);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int s = 0; s < 2 * N + 2; ++s) {
      const int u = s >> 1;
      if ((s & 1) == 0) {
        if (u + 1 < N) load_tile(kr, kbase + ((u + 1) & 1) * S::TILE_BYTES, vis.tile(u + 1), false);
        if (u < N) load_tile(vr, vbase + (u & 1) * S::TILE_BYTES, vis.tile(u), true);
      }
      if ((s & 1) == grp) {
        gemm_phase(u, N);
      } else {
        const int ty = grp == 0 ? u : u - 1;
        if (ty >= 0 && ty < N) softmax_phase(ty);
      }
      if (s & 1) {
        __builtin_amdgcn_s_waitcnt(0);  // this slot's LDS reads and the loads of slot s-1
        __syncthreads();
      } else {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): LDS reads of this slot are done
        __builtin_amdgcn_s_barrier();
      }
    }

    // ---- epilogue: O = O / l, round to bf16, store this lane's query row
    const float l_tot = l_run + xor32(l_run);
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
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      a.lse[(int64_t)h * total_tokens + seq0 + qi] = m_use * a.scale + logf(l_tot);
    }
    __syncthreads();  // s_item and the LDS tiles are reused by the next item
  }
  // The last workgroup out leaves the queue counters at zero for the next launch.
  if (tid == 0 && atomicAdd(&a.queue[1], 1) == (int)gridDim.x - 1) {
    atomicExch(&a.queue[0], 0);
    atomicExch(&a.queue[1], 0);
  }
}

}  // namespace

int attn_bf16_blocks_per_cu() { return 1; }

hipError_t launch_attn_bf16(const AttnArgs& a, int grid, hipStream_t stream) {
  if (a.head_dim == 128)
    attn_bf16_kernel<128><<<grid, kThreads, 0, stream>>>(a);
  else
    attn_bf16_kernel<64><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ea
