// ea_attn_bf16.hip -- persistent routed hybrid-attention prefill, bf16 in/out, CDNA4 MFMA.
//
// What it computes (Elastic Attention blog post, section 2.1 "Attention Router": r = 0
// runs Full Attention, r = 1 runs Sparse Attention, outputs concatenated per head;
// section 1 and the gist.science explanation, section "问题所在", for the sparse pattern,
// read here as attention sink + causal sliding window; section 3 "Fused Kernel": one
// launch serves both kinds of head, the routing arriving as metadata):
//   for every work item (sequence b, query head h, 128-row q-tile):
//     O[rows, h, :] = softmax(scale * Q K^T + mask) V over the item's visible keys.
//
// Design (gfx950, one workgroup = 4 wavefronts = 128 query rows, 64-key tiles):
//   * Persistent grid: each workgroup pops items from the longest-first work list with
//     one atomic per item, so long full-head items start first and short sparse items
//     fill the tail of the launch.
//   * Sparse items visit only their sink tiles and window tiles; the element mask is
//     applied only on tiles that are not fully visible.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with Q held in registers as the B operand,
//     so each lane owns one query row of S: the row max needs one cross-half exchange
//     (v_permlane32_swap) and the row sum stays lane-partial until the epilogue.
//   * O^T = V^T P^T on the same MFMA: P comes straight from the S accumulators (bf16)
//     as the B operand; the V^T operand is read with ds_read_b64_tr_b16 from a
//     row-major V tile, and the contraction order of keys is permuted consistently on
//     both operands to match the accumulator layout.
//   * K and V tiles are double buffered in LDS (global loads for tile n+1 are in flight
//     while tile n is computed) with padded rows: K rows stride 272 B and V rows 320 B
//     (D = 128), which keep the b128 K reads and the transposing V reads free of bank
//     conflicts on the 64-bank LDS.
//   * Softmax uses exp2 with log2(e) folded into the scale; all state is fp32.  Lazy
//     rescaling: the running max used in the exponent only moves when a row's max grows
//     by more than 2^8 in exp2 units (or on the first visible tile), so most tiles skip
//     the O *= alpha pass; P stays below 256, well inside bf16 and fp32 range.
//   * Raw buffer loads/stores bound every access: keys past the sequence end read as
//     zero and rows past the tile end are not stored.
#include <climits>

#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int BM = kBf16BM;      // 128 query rows per item
constexpr int BN = kBf16BN;      // 64 keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSubN = BN / 32;   // 32-key MFMA sub-tiles per key tile

template <int D>
struct Shape {
  static constexpr int KS = D + 8;     // K row stride in LDS (elements)
  static constexpr int VS = D + 32;    // V row stride in LDS (elements)
  static constexpr int KTILE = BN * KS;
  static constexpr int VTILE = BN * VS;
  static constexpr int LDS_BYTES = 2 * (KTILE + VTILE) * 2;
  static constexpr int CHUNKS = D / 8;             // 16-byte chunks per row
  static constexpr int ROWS_PER_PASS = kThreads / CHUNKS;
  static constexpr int PASSES = BN / ROWS_PER_PASS;
  static constexpr int KSTEPS = D / 16;            // MFMA k-steps over the head dim
  static constexpr int DT = D / 32;                // 32-wide output column tiles
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

// True if some (row, key) pair of the tile is hidden for rows [m0, m1).
__device__ __forceinline__ bool tile_needs_mask(int kt, bool sparse, int m0, int m1, int sink,
                                                int window) {
  const int k0 = kt * BN, k1 = k0 + BN;
  if (k1 - 1 > m0) return true;                       // causal edge (or keys past the end)
  if (!sparse) return false;
  return !(k1 <= sink || k0 > m1 - 1 - window);       // neither all-sink nor all-window
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  using S = Shape<D>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[S::LDS_BYTES / 2];
  __shared__ int s_item;
  // K tiles at [0, 2*KTILE), V tiles after them; buffer `buf` of each at buf * tile size
  __bf16* const kbase = lds;
  __bf16* const vbase = lds + 2 * S::KTILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv;
  const int group = Hq / Hkv;
  const int n_items = *a.n_items;
  const int total_tokens = a.cu[a.batch];
  const float c_log2 = a.scale * 1.4426950408889634f;  // scale * log2(e)
  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;

  // global -> LDS copy assignment: row `crow` (+ pass * ROWS_PER_PASS), 16-byte chunk `cch`
  const int crow = tid / S::CHUNKS, cch = tid % S::CHUNKS;

  for (;;) {
    if (tid == 0) s_item = atomicAdd(&a.queue[0], 1);
    __syncthreads();
    const int it = s_item;
    if (it >= n_items) break;
    const int4 item = a.items[it];
    const int b = item.x, h = item.y, qt = item.z;
    const int seq0 = a.cu[b];
    const int len = a.cu[b + 1] - seq0;
    const int m0 = qt * BM, m1 = min(m0 + BM, len);
    const int kvh = h / group;
    const bool sparse = a.route[(int64_t)b * Hq + h] != 0;
    const Visit vis = make_visit(sparse, m0, m1, a.sink, a.window);

    // buffer windows: this item's Q/O rows of head h; this sequence's K/V of head kvh
    const int64_t qo_elem = ((int64_t)(seq0 + m0) * Hq + h) * D;
    const uint32_t qo_bytes = (uint32_t)(m1 - m0 - 1) * q_row_bytes + D * 2;
    const auto qr = make_rsrc((const __bf16*)a.q + qo_elem, qo_bytes);
    const auto orr = make_rsrc((__bf16*)a.o + qo_elem, qo_bytes);
    const int64_t kv_elem = ((int64_t)seq0 * Hkv + kvh) * D;
    const uint32_t kv_bytes = (uint32_t)(len - 1) * kv_row_bytes + D * 2;
    const auto kr = make_rsrc((const __bf16*)a.k + kv_elem, kv_bytes);
    const auto vr = make_rsrc((const __bf16*)a.v + kv_elem, kv_bytes);

    // Q as the B operand: lane holds query row (32*wave + l32), head-dim elements
    // 16*ks + 8*g .. +7 for every k-step ks.
    bf16x8 qreg[S::KSTEPS];
    {
      const uint32_t row_off = (uint32_t)(32 * wave + l32) * q_row_bytes;
#pragma unroll
      for (int ks = 0; ks < S::KSTEPS; ++ks)
        qreg[ks] = __builtin_bit_cast(bf16x8, buf_load16(qr, row_off + (16 * ks + 8 * g) * 2));
    }

    f32x16 oacc[S::DT];
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const int qi = m0 + 32 * wave + l32;  // this lane's query position in the sequence

    u32x4 kst[S::PASSES], vst[S::PASSES];
    auto fetch = [&](int kt) {
#pragma unroll
      for (int p = 0; p < S::PASSES; ++p) {
        const uint32_t key = (uint32_t)(kt * BN + p * S::ROWS_PER_PASS + crow);
        const uint32_t off = key * kv_row_bytes + cch * 16;
        kst[p] = buf_load16(kr, off);
        vst[p] = buf_load16(vr, off);
      }
    };
    auto stash = [&](int buf) {
#pragma unroll
      for (int p = 0; p < S::PASSES; ++p) {
        const int row = p * S::ROWS_PER_PASS + crow;
        *(u32x4*)(kbase + buf * S::KTILE + row * S::KS + cch * 8) = kst[p];
        *(u32x4*)(vbase + buf * S::VTILE + row * S::VS + cch * 8) = vst[p];
      }
    };

    fetch(vis.tile(0));
    stash(0);
    __syncthreads();

    for (int n = 0; n < vis.count; ++n) {
      const int buf = n & 1;
      const int kt = vis.tile(n);
      const bool more = n + 1 < vis.count;
      if (more) fetch(vis.tile(n + 1));

      // ---- S^T = K Q^T : sacc[j][r] = score(key kt*BN + 32j + 8(r/4) + 4g + r%4, query qi)
      f32x16 sacc[kSubN];
      const __bf16* kb = kbase + buf * S::KTILE;
#pragma unroll
      for (int j = 0; j < kSubN; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[j][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < S::KSTEPS; ++ks) {
          const bf16x8 ka = *(const bf16x8*)(kb + (32 * j + l32) * S::KS + 16 * ks + 8 * g);
          sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], sacc[j], 0, 0, 0);
        }
      }

      if (tile_needs_mask(kt, sparse, m0, m1, a.sink, a.window)) {
        // key kj = kt*BN + off is visible to query qi iff off <= qi - kbase and, for a
        // sparse head, (off >= qi - window + 1 - kbase or off < sink - kbase); branch-free
        const int kbase = kt * BN;
        const int lim = qi - kbase;
        const int wlo = sparse ? qi - a.window + 1 - kbase : INT_MIN;
        const int slim = sparse ? a.sink - kbase : INT_MIN;
#pragma unroll
        for (int j = 0; j < kSubN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * j + 8 * (r / 4) + 4 * g + (r % 4);
            const bool visible = (off <= lim) & ((off >= wlo) | (off < slim));
            sacc[j][r] = visible ? sacc[j][r] : -INFINITY;
          }
      }

      // ---- online softmax (one query per lane; partner lane ^32 holds the other keys)
      float mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < kSubN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[j][r]);
      mt = fmaxf(mt, xor32(mt));
      // rescale only when some row of the wavefront has a new max (alpha = 1 elsewhere);
      // P is always relative to the true running max, so its largest entry is exactly 1
      if (__builtin_amdgcn_ballot_w64(mt > m_run) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha =
            m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f((m_run - m_new) * c_log2);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        m_run = m_new;
      }
      const float mc = (m_run == -INFINITY ? 0.f : m_run) * c_log2;
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < kSubN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][r], c_log2, -mc));
          sacc[j][r] = p;
          psum += p;
        }
      l_run += psum;

      // ---- O^T += V^T P^T over 16-key slices (j, kh): P keys 32j+16kh+8(e/4)+4g+e%4
      const __bf16* vb = vbase + buf * S::VTILE;
      const int tr_row = 4 * g + (lane & 15) / 4;               // + 32j + 16kh (+8)
      const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32dt
#pragma unroll
      for (int j = 0; j < kSubN; ++j)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[j][8 * kh + e];
          const int row = 32 * j + 16 * kh + tr_row;
#pragma unroll
          for (int dt = 0; dt < S::DT; ++dt) {
            const __bf16* p0 = vb + row * S::VS + 32 * dt + tr_col;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(p0));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(p0 + 8 * S::VS));
            const bf16x8 va = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[dt], 0, 0, 0);
          }
        }

      if (more) stash(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: O = O / l, round to bf16, store this lane's query row
    const float l_tot = l_run + xor32(l_run);
    const float inv = 1.0f / l_tot;
    const uint32_t row_off = (uint32_t)(32 * wave + l32) * q_row_bytes;
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

int attn_bf16_blocks_per_cu() { return 2; }

hipError_t launch_attn_bf16(const AttnArgs& a, int grid, hipStream_t stream) {
  if (a.head_dim == 128)
    attn_bf16_kernel<128><<<grid, kThreads, 0, stream>>>(a);
  else
    attn_bf16_kernel<64><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ea
