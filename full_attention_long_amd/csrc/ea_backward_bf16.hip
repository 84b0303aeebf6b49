// ea_backward_bf16.hip -- backward of the routed hybrid attention on the CDNA4 matrix cores
// (bf16 inputs, fp32 accumulation and gradients).
//
// What it computes (Elastic Attention blog post, section 2.1: routed Full / Sparse Attention
// heads trained through the router's "training trick"; sparse pattern: attention sink + causal
// sliding window), per sequence, query head h and visible pair (row i, key j), with
// P_ij = exp(scale <q_i, k_j> - lse_i) and D_i = <dO_i, O_i> (computed beforehand):
//   dS_ij = P_ij (<dO_i, v_j> - D_i),
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j.
//
// Two kernels (no atomics: every gradient element is written once, in a fixed order):
//   * bwd_dkv_mfma: one workgroup per (128-key tile, query head, sequence), 8 wavefronts (4 key
//     blocks of 32 keys x 2 row parities, two wavefronts per SIMD).  K and V of the tile sit in
//     LDS as the B operand of v_mfma_f32_32x32x16_bf16; for every 64-row stage of the rows that
//     can see the tile (all later rows for a full head or a tile with sink keys, else the next
//     window - 1 positions), Q, dO, lse and D arrive in LDS by direct loads (double buffered)
//     and each wavefront runs the 32-row sub-tile of its parity:
//       S = Q K^T and dP = dO V^T   (lane: one key, 16 rows),
//       P, dS on the vector ALU, rounded to bf16 as B operands,
//       dV^T += dO^T P and dK^T += Q^T dS   (dO^T, Q^T read transposed from the row-major
//       stage with ds_read_b64_tr_b16; rows permuted consistently on both operands).
//     The two parities add their partial sums through LDS in a fixed order.  One query head
//     per workgroup bounds the longest workgroup (a sink tile, or a tile of a full head) at one
//     head's rows; with several query heads per KV head each writes fp32 partials that
//     bwd_dkv_reduce adds in head order (deterministic).
//   * bwd_dq_mfma: one workgroup per (128-row q-tile, head, sequence), 4 wavefronts of 32
//     rows, Q and dO of the wavefront's rows in registers; per 64-key tile of the forward's
//     visit plan (sink tiles, then window or causal tiles), K and V staged in LDS:
//       S^T = K Q^T and dP^T = V dO^T   (lane: one row, 16 keys),
//       dQ^T += K^T dS^T   (K^T read transposed from the row-major tile).
// Workgroup order: longest first (the tiles with the most rows), and the head index rotated by
// the tile index, so that consecutive workgroups -- which the dispatcher deals round-robin to
// the eight XCDs -- do not pin every tile of one head to one XCD.
// LDS rows are XOR-swizzled per 16-byte chunk so that both the plain 16-byte reads (16
// consecutive rows, one chunk) and the transposing 8-byte reads (4 aligned rows x 64 bytes)
// hit distinct banks.  Rows and keys past a sequence read as zero; a row past the sequence
// gets P = 0 (lse = +inf in dq, the masked path in dk/dv), and masks are applied only on
// sub-tiles that hide some pair.
#include <math.h>

#include <type_traits>

#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStage = 64;            // rows (dk/dv kernel) or keys (dq kernel) per LDS stage
constexpr int kKeyTile = 32 * kWaves; // keys per dk/dv workgroup
constexpr int kRowTile = 32 * kWaves; // rows per dq workgroup
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct BS {
  static constexpr int CHUNKS = D / 8;
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = kStage * ROW_BYTES;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int LOADS = kStage * CHUNKS / kThreads;  // 16-byte chunks per thread per tile
  // physical chunk = logical chunk ^ swz(row)
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (CHUNKS == 16)
      return 4 * (r & 3) + ((r >> 2) & 3);
    else
      return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
  // byte offset of element (row r, column col) in a stage tile (col % 4 == 0)
  static __device__ __forceinline__ int off(int r, int col) {
    return r * ROW_BYTES + (((col >> 3) ^ swz(r)) << 4) + (col & 7) * 2;
  }
};

__device__ __forceinline__ bool pair_visible(int i, int j, bool sparse, int sink, int window) {
  return j <= i && (!sparse || j < sink || j > i - window);
}

// A operand of a transposed product: element (row R + 8(e/4) + 4g + e%4, column 32*dt + l32)
// of a row-major stage tile in slot e (the two ds_read_b64_tr_b16 cover rows R.. and R+8..).
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const unsigned char* base, int R, int dt, int tr_row,
                                          int tr_col) {
  using S = BS<D>;
  const int row = R + tr_row, col = 32 * dt + tr_col;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + S::off(row, col)));
  const s16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + S::off(row + 8, col)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand of a plain product: row R + l32, columns 16*ks + 8g .. + 7
template <int D>
__device__ __forceinline__ bf16x8 read_plain(const unsigned char* base, int R, int ks, int l32,
                                             int g) {
  return *(const bf16x8*)(base + BS<D>::off(R + l32, 16 * ks + 8 * g));
}

// ------------------------------------------------------------------------------ dk / dv

// Products of one 32-row sub-tile in the dk/dv kernel (sched_barrier keeps each group's LDS
// reads where they are issued):
//   A groups (KSTEPS): S += Q K^T and dP += dO V^T over one k-step, the four operands (Q, dO
//   rows; K, V of the key block) read one group ahead;
//   C groups (NC = DT): dV^T += dO^T P and dK^T += Q^T dS for one 16-row slice kh and two
//   32-column tiles, operands single-buffered (the partner wavefront covers the latency).
template <int D>
struct DkvOps {
  using S = BS<D>;
  static constexpr int NC = S::DT;
  static constexpr int HALF = S::DT / 2;  // column-tile pairs per 16-row slice
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS of the dk/dv kernel: the K and V tiles of the workgroup's kKeyTile keys, then two
// buffers of a Q stage and a dO stage of kRowsDkv rows (bf16, swizzled as BS<D>) with their
// lse2 and D.  After the last stage the whole area holds the partial dK, dV exchange.
constexpr int kRowsDkv = 64;
constexpr int kWavesDkv = 8;                 // 4 key blocks x 2 row parities
constexpr int kThreadsDkv = 64 * kWavesDkv;
template <int D>
struct DkvLds {
  static constexpr int KV_TILE = kKeyTile * D * 2;
  static constexpr int TILE = kRowsDkv * D * 2;
  static constexpr int RPL = 1024 / (D * 2);            // rows one wave-wide 16-byte load fills
  static constexpr int KV_WAVE_LOADS = KV_TILE / 1024 / kWavesDkv;
  static constexpr int WAVE_LOADS = TILE / 1024 / kWavesDkv;
  static constexpr int VEC = kRowsDkv * 4;              // lse2 or D of a stage
  static constexpr int BUF = 2 * TILE + 2 * VEC;
  static constexpr int BYTES = 2 * KV_TILE + 2 * BUF;
  static constexpr int k_at() { return 0; }
  static constexpr int v_at() { return KV_TILE; }
  static constexpr int q_at(int buf) { return 2 * KV_TILE + buf * BUF; }
  static constexpr int g_at(int buf) { return 2 * KV_TILE + buf * BUF + TILE; }
  static constexpr int l_at(int buf) { return 2 * KV_TILE + buf * BUF + 2 * TILE; }
  static constexpr int d_at(int buf) { return 2 * KV_TILE + buf * BUF + 2 * TILE + VEC; }
  // partial exchange: 4 key blocks x (dK, dV) x DT x 16 registers x 64 lanes x 4 bytes
  static constexpr int XCHG = 4 * 2 * (D / 32) * 16 * 64 * 4;
  static_assert(XCHG <= BYTES, "the exchange reuses the tile area");
};

template <int D>
__global__ __launch_bounds__(kThreadsDkv, 1) void bwd_dkv_mfma(BwdArgs a) {
  using S = BS<D>;
  using O = DkvOps<D>;
  using M = DkvLds<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[M::BYTES];
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, G = Hq / Hkv;
  // longest first: every (query head, sequence) pair of key tile 0, then of tile 1, ...; the
  // pair index rotated by the tile index (XCD spread)
  const int pairs = Hq * a.batch;
  const int kt = blockIdx.x / pairs;
  const int pair = (blockIdx.x % pairs + kt) % pairs;
  const int h = pair % Hq, b = pair / Hq;
  const int kvh = h / G, hh = h % G;
  const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
  const int Tq = a.cu_q[a.batch];
  if (q0 < 0 || k0 < 0 || Lq > a.max_seqlen_q || Lk > a.max_seqlen_k || Lk < Lq ||
      Tq > a.tq_cap || a.cu_k[a.batch] > a.tk_cap)
    return;
  if (kt * kKeyTile >= Lk) return;
  const int off = Lk - Lq;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wavefront index is uniform; readfirstlane lets the compiler know, so every test
  // built on it (skip, mask) is a scalar branch rather than a per-lane exec mask
  const int wave = uniform(tid >> 6);
  const int kb = wave & 3;   // key block: keys kw0 .. kw0 + 31
  const int rp = wave >> 2;  // row parity: the sub-tile rp of every 64-row stage
  const int l32 = lane & 31, g = lane >> 5;
  const int tr_row = 4 * g + (lane & 15) / 4;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int j0 = kt * kKeyTile, j1 = min(j0 + kKeyTile, Lk);
  const int kw0 = j0 + 32 * kb;
  const int key = kw0 + l32;
  const float c_log2 = a.scale * kLog2e;
  const bool sparse = a.route[(int64_t)b * Hq + h] != 0;
  const int lrow = lane / S::CHUNKS, pc = lane % S::CHUNKS;

  // K and V tiles of the workgroup's keys, direct to LDS (keys past the sequence read as zero)
  {
    const uint32_t row_bytes = (uint32_t)Hkv * D * 2;
    const uint32_t bytes = (uint32_t)(Lk - 1) * row_bytes + D * 2;
    const int64_t base = ((int64_t)k0 * Hkv + kvh) * D;
    const auto kr = make_rsrc((const __bf16*)a.k + base, bytes);
    const auto vr = make_rsrc((const __bf16*)a.v + base, bytes);
#pragma unroll
    for (int i = 0; i < M::KV_WAVE_LOADS; ++i) {
      const int lg = wave * M::KV_WAVE_LOADS + i;
      const int row = lg * M::RPL + lrow;
      const uint32_t lane_off = (uint32_t)lrow * row_bytes + (uint32_t)((pc ^ S::swz(row)) * 16);
      const uint32_t row_base = (uint32_t)uniform((int)((uint32_t)(j0 + lg * M::RPL) * row_bytes));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(lds + M::k_at() + lg * 1024), 16,
                                               lane_off, row_base, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(lds + M::v_at() + lg * 1024), 16,
                                               lane_off, row_base, 0, 0);
    }
  }
  f32x16 dk[S::DT], dv[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[dt][r] = dv[dt][r] = 0.f;

  // rows that can see the tile: positions [max(j0, off), pe) in stages of kRowsDkv
  const int pb0 = max(j0, off);
  const int pe = (!sparse || j0 < a.sink) ? Lk : min(Lk, j1 - 1 + a.window);
  const int n_stages = pe > pb0 ? (pe - pb0 + kRowsDkv - 1) / kRowsDkv : 0;

  // Direct loads of a stage: the Q and dO rows [p, p + kRowsDkv) of head h (chunk rows
  // p - off; rows past the sequence read as zero) and their lse2 (wave 0) and D (wave 1).
  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  const int64_t qbase = ((int64_t)q0 * Hq + h) * D;
  const uint32_t qbytes = (uint32_t)(Lq - 1) * q_row_bytes + D * 2;
  const auto qr = make_rsrc((const __bf16*)a.q + qbase, qbytes);
  const auto gr = make_rsrc((const __bf16*)a.dout + qbase, qbytes);
  const auto lr = make_rsrc(a.lse2 + (int64_t)h * Tq + q0, (uint32_t)Lq * 4);
  const auto dr = make_rsrc(a.delta + (int64_t)h * Tq + q0, (uint32_t)Lq * 4);
  auto issue = [&](int p, int buf) {
    const int r0 = uniform(p - off);
#pragma unroll
    for (int i = 0; i < M::WAVE_LOADS; ++i) {
      const int lg = wave * M::WAVE_LOADS + i;
      const int row = lg * M::RPL + lrow;
      const uint32_t lane_off = (uint32_t)lrow * q_row_bytes + (uint32_t)((pc ^ S::swz(row)) * 16);
      const uint32_t row_base = (uint32_t)uniform((int)((uint32_t)(r0 + lg * M::RPL) * q_row_bytes));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void*)(lds + M::q_at(buf) + lg * 1024),
                                               16, lane_off, row_base, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(gr, (lds_void*)(lds + M::g_at(buf) + lg * 1024),
                                               16, lane_off, row_base, 0, 0);
    }
    if (wave < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wave == 0 ? lr : dr,
          (lds_void*)(lds + (wave == 0 ? M::l_at(buf) : M::d_at(buf))), 4, (uint32_t)lane * 4,
          (uint32_t)uniform(r0 * 4), 0, 0);
  };

  if (n_stages > 0) issue(pb0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const unsigned char* kvk = lds + M::k_at();
  const unsigned char* kvv = lds + M::v_at();
  for (int n = 0; n < n_stages; ++n) {
    const int p_c = pb0 + n * kRowsDkv;
    const bool more = n + 1 < n_stages;
    // buffer (n + 1) & 1 was last read in stage n - 1, which every wavefront has finished
    if (more) issue(p_c + kRowsDkv, (n + 1) & 1);
    const int buf = n & 1;
    const unsigned char* qb = lds + M::q_at(buf);
    const unsigned char* gb = lds + M::g_at(buf);
    const float* sl = (const float*)(lds + M::l_at(buf));
    const float* sd = (const float*)(lds + M::d_at(buf));
    const int j = rp;               // this wavefront's sub-tile of the stage
    const int i0 = p_c + 32 * j;    // its first row position
    // no visible pair between rows [i0, i0 + 32) and keys [kw0, kw0 + 32): skip
    const bool none = kw0 >= Lk || i0 >= Lk || i0 + 31 < kw0 ||
                      (sparse && kw0 >= a.sink && i0 - a.window + 1 > kw0 + 31);
    if (!none) {
      // every pair visible (and every row inside the sequence)
      const bool full_vis = i0 >= kw0 + 31 && i0 + 31 < Lk &&
                            (!sparse || kw0 + 31 < a.sink || kw0 > i0 + 31 - a.window);
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
      bf16x8 pb[2], db[2];
      // A: S += Q K^T and dP += dO V^T, one MFMA per k-step and product; each MFMA's two
      // operands are read RA - 1 MFMAs ahead into a ring (one pair per MFMA, not in bursts)
      {
        constexpr int NA2 = 2 * S::KSTEPS, RA = 3;
        // MFMA m: S (Q rows, K^T: lane holds key l32's dims) for even m, dP (dO, V) for odd,
        // k-step m / 2
        auto rdA = [&](int m, bf16x8 (&o)[2]) __attribute__((always_inline)) {
          const int ks = m / 2;
          o[0] = read_plain<D>(m % 2 == 0 ? qb : gb, 32 * j, ks, l32, g);
          o[1] = read_plain<D>(m % 2 == 0 ? kvk : kvv, 32 * kb, ks, l32, g);
        };
        bf16x8 ra[RA][2];
#pragma unroll
        for (int m = 0; m < RA - 1; ++m) rdA(m, ra[m]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NA2; ++m) {
          if (m + RA - 1 < NA2) rdA(m + RA - 1, ra[(m + RA - 1) % RA]);
          if (m % 2 == 0)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[m % RA][0], ra[m % RA][1], sacc, 0, 0, 0);
          else
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[m % RA][0], ra[m % RA][1], pacc, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // P and dS: sacc[r] = S[row i0 + 8(r/4) + 4g + r%4][key]; `masked` selects the code
      // path once per sub-tile (uniform), the masked one hiding invisible pairs and rows past
      // the sequence
      auto phase_b = [&](auto masked_t) {
        constexpr bool masked = decltype(masked_t)::value;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int lr4 = 32 * j + 8 * q4 + 4 * g;  // local row of r = 4 q4
          const f32x4 l4 = *(const f32x4*)&sl[lr4];
          const f32x4 d4 = *(const f32x4*)&sd[lr4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c_log2, -l4[e]));
            if constexpr (masked) {
              const int row = p_c + lr4 + e;
              const bool vis = (row < Lk) & (key <= row) &
                               (!sparse | (key < a.sink) | (key > row - a.window));
              p = vis ? p : 0.f;
            }
            pb[r / 8][r % 8] = (__bf16)p;
            db[r / 8][r % 8] = (__bf16)(p * (pacc[r] - d4[e]));
          }
        }
      };
      if (full_vis)
        phase_b(std::false_type{});
      else
        phase_b(std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      // C: dV^T += dO^T P and dK^T += Q^T dS for 16-row slice kh and column tile dt; MFMA m is
      // (kh, dt) = (c / HALF, 2 (c % HALF) + w / 2) with c = m / 4, w = m % 4, dV for even w;
      // its transposed operand is read RC - 1 MFMAs ahead into a ring
      {
        constexpr int NC4 = 4 * O::NC, RC = 6;
        auto rdC = [&](int m, bf16x8& o) __attribute__((always_inline)) {
          const int c = m / 4, w = m % 4;
          const int kh = c / O::HALF, dt0 = 2 * (c % O::HALF);
          o = read_tr<D>(w % 2 == 0 ? gb : qb, 32 * j + 16 * kh, dt0 + w / 2, tr_row, tr_col);
        };
        bf16x8 rc[RC];
#pragma unroll
        for (int m = 0; m < RC - 1; ++m) rdC(m, rc[m]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NC4; ++m) {
          if (m + RC - 1 < NC4) rdC(m + RC - 1, rc[(m + RC - 1) % RC]);
          const int c = m / 4, w = m % 4;
          const int kh = c / O::HALF, dt = 2 * (c % O::HALF) + w / 2;
          if (w % 2 == 0)
            dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rc[m % RC], pb[kh], dv[dt], 0, 0, 0);
          else
            dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rc[m % RC], db[kh], dk[dt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // the next stage's loads (this wavefront's share) have landed; after the barrier every
    // wavefront's have, and nobody reads this stage's buffer any more
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // The two row parities of a key block add their partial sums through LDS (parity 1 writes,
  // parity 0 adds, in that fixed order): lane-major float4 slots per register quad.
  __syncthreads();  // (no stage ran: the K/V loads may still be landing in the area)
  float* xb = (float*)lds + kb * (2 * S::DT * 16 * 64);
  if (rp == 1) {
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = dk[dt][4 * q4 + e];
          v4[e] = dv[dt][4 * q4 + e];
        }
        *(f32x4*)(xb + ((0 * S::DT + dt) * 4 + q4) * 256 + lane * 4) = k4;
        *(f32x4*)(xb + ((1 * S::DT + dt) * 4 + q4) * 256 + lane * 4) = v4;
      }
  }
  __syncthreads();
  // dk[dt][r] = dK^T[dim 32dt + 8(r/4) + 4g + r%4][key]; one query head's share: the
  // gradient itself when the KV head has one query head, else its partial
  if (rp == 0 && key < Lk) {
    const int64_t at = ((int64_t)(k0 + key) * Hkv + kvh) * D;
    const int64_t slice = G > 1 ? (int64_t)hh * a.tk_cap * Hkv * D : 0;
    float* dkp = (G > 1 ? a.dk_part + slice : a.dk) + at;
    float* dvp = (G > 1 ? a.dv_part + slice : a.dv) + at;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * g;
        const f32x4 k1 = *(const f32x4*)(xb + ((0 * S::DT + dt) * 4 + q4) * 256 + lane * 4);
        const f32x4 v1 = *(const f32x4*)(xb + ((1 * S::DT + dt) * 4 + q4) * 256 + lane * 4);
        f32x4 kv4, vv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv4[e] = (dk[dt][4 * q4 + e] + k1[e]) * a.scale;
          vv4[e] = dv[dt][4 * q4 + e] + v1[e];
        }
        *(f32x4*)(dkp + d) = kv4;
        *(f32x4*)(dvp + d) = vv4;
      }
  }
}

// ------------------------------------------------------------------------------ dq

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_mfma(BwdArgs a) {
  using S = BS<D>;
  constexpr int NA = S::KSTEPS / 2;  // S^T / dP^T groups of two k-steps
  constexpr int RPL = 1024 / (D * 2);  // rows one wave-wide 16-byte direct load fills
  constexpr int WAVE_LOADS = S::TILE_BYTES / 1024 / kWaves;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * S::TILE_BYTES];
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, G = Hq / Hkv;
  // longest first: the last q-tiles (most keys) of every (head, sequence) pair first
  const int pairs = Hq * a.batch;
  const int step = blockIdx.x / pairs;
  const int qt = (int)(gridDim.x / pairs) - 1 - step;
  const int pair = (blockIdx.x % pairs + step) % pairs;  // rotated: XCD spread
  const int h = pair % Hq, b = pair / Hq;
  const int kvh = h / G;
  const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
  const int Tq = a.cu_q[a.batch];
  if (q0 < 0 || k0 < 0 || Lq > a.max_seqlen_q || Lk > a.max_seqlen_k || Lk < Lq ||
      Tq > a.tq_cap)
    return;
  if (qt * kRowTile >= Lq) return;
  const int off = Lk - Lq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);  // uniform: skips and masks are scalar branches
  const int l32 = lane & 31, g = lane >> 5;
  const int tr_row = 4 * g + (lane & 15) / 4;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const bool sparse = a.route[(int64_t)b * Hq + h] != 0;
  const float c_log2 = a.scale * kLog2e;
  const int cr0 = qt * kRowTile;                // first chunk row of the workgroup
  const int p0 = off + cr0, p1 = off + min(cr0 + kRowTile, Lq);  // its positions
  const int wr0 = p0 + 32 * wave;               // this wavefront's first row position
  const int cr = cr0 + 32 * wave + l32;         // this lane's chunk row
  const int pos = off + cr;

  // Q and dO of the lane's row as B operands
  bf16x8 qreg[S::KSTEPS], greg[S::KSTEPS];
  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  {
    const int64_t base = ((int64_t)q0 * Hq + h) * D;
    const uint32_t bytes = (uint32_t)(Lq - 1) * q_row_bytes + D * 2;
    const auto qr = make_rsrc((const __bf16*)a.q + base, bytes);
    const auto gr = make_rsrc((const __bf16*)a.dout + base, bytes);
    const uint32_t ro = (uint32_t)cr * q_row_bytes;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) {
      qreg[ks] = __builtin_bit_cast(bf16x8, buf_load16(qr, ro + (16 * ks + 8 * g) * 2));
      greg[ks] = __builtin_bit_cast(bf16x8, buf_load16(gr, ro + (16 * ks + 8 * g) * 2));
    }
  }
  const bool row_ok = cr < Lq;
  const int64_t at = (int64_t)h * Tq + q0 + min(cr, Lq - 1);
  const float lse2 = row_ok ? a.lse2[at] : INFINITY;  // rows past the sequence: P = 0
  const float dlt = row_ok ? a.delta[at] : 0.f;
  f32x16 dq[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  // visit plan over kStage-key tiles for positions [p0, p1): sink tiles [0, n1), then
  // [s2, t_hi] (window or causal)
  const int t_hi = (p1 - 1) / kStage;
  int n1 = 0, s2 = 0;
  if (sparse) {
    n1 = (min(a.sink, p1) + kStage - 1) / kStage;
    s2 = max(max(0, p0 - a.window + 1) / kStage, n1);
  }
  const int count = n1 + max(0, t_hi - s2 + 1);
  auto tile_of = [&](int n) { return n < n1 ? n : s2 + (n - n1); };

  // direct global -> LDS loads of a K and a V tile (keys past the sequence read as zero;
  // lane placement as in the dk/dv kernel)
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;
  const int64_t kv_base = ((int64_t)k0 * Hkv + kvh) * D;
  const uint32_t kv_bytes = (uint32_t)(Lk - 1) * kv_row_bytes + D * 2;
  const auto kr = make_rsrc((const __bf16*)a.k + kv_base, kv_bytes);
  const auto vr = make_rsrc((const __bf16*)a.v + kv_base, kv_bytes);
  const int lrow = lane / S::CHUNKS, pc = lane % S::CHUNKS;
  auto issue = [&](int t, int buf) {
    const int key0 = uniform(t * kStage);
#pragma unroll
    for (int i = 0; i < WAVE_LOADS; ++i) {
      const int lg = wave * WAVE_LOADS + i;
      const int row = lg * RPL + lrow;
      const uint32_t lane_off =
          (uint32_t)lrow * kv_row_bytes + (uint32_t)((pc ^ S::swz(row)) * 16);
      const uint32_t row_base =
          (uint32_t)uniform((int)((uint32_t)(key0 + lg * RPL) * kv_row_bytes));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          kr, (lds_void*)(lds + (2 * buf) * S::TILE_BYTES + lg * 1024), 16, lane_off, row_base,
          0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vr, (lds_void*)(lds + (2 * buf + 1) * S::TILE_BYTES + lg * 1024), 16, lane_off,
          row_base, 0, 0);
    }
  };

  if (count > 0) issue(tile_of(0), 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int n = 0; n < count; ++n) {
    const bool more = n + 1 < count;
    if (more) issue(tile_of(n + 1), (n + 1) & 1);
    const int buf = n & 1;
    const unsigned char* kb = lds + (2 * buf) * S::TILE_BYTES;
    const unsigned char* vb = lds + (2 * buf + 1) * S::TILE_BYTES;
    const int t = tile_of(n);
#pragma unroll
    for (int jk = 0; jk < kStage / 32; ++jk) {
      const int c0 = t * kStage + 32 * jk;  // first key of the sub-tile
      // rows [wr0, wr0 + 32) against keys [c0, c0 + 32)
      const bool none = wr0 >= Lk || wr0 + 31 < c0 ||
                        (sparse && c0 >= a.sink && wr0 - a.window + 1 > c0 + 31);
      if (none) continue;
      const bool full_vis = wr0 >= c0 + 31 &&
                            (!sparse || c0 + 31 < a.sink || c0 > wr0 + 31 - a.window);
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
      auto readA = [&](int c, bf16x8 (&op)[4]) {
        op[0] = read_plain<D>(kb, 32 * jk, 2 * c, l32, g);
        op[1] = read_plain<D>(kb, 32 * jk, 2 * c + 1, l32, g);
        op[2] = read_plain<D>(vb, 32 * jk, 2 * c, l32, g);
        op[3] = read_plain<D>(vb, 32 * jk, 2 * c + 1, l32, g);
      };
      auto runA = [&](int c, const bf16x8 (&op)[4]) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[0], qreg[2 * c], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[2], greg[2 * c], pacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[1], qreg[2 * c + 1], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[3], greg[2 * c + 1], pacc, 0, 0, 0);
      };
      // C groups: 16-key slice kh, column tiles dt0, dt0 + 1 (DT / 2 pairs per slice)
      auto readC = [&](int c, bf16x8 (&op)[4]) {
        const int kh = c / (S::DT / 2), dt0 = 2 * (c % (S::DT / 2));
        op[0] = read_tr<D>(kb, 32 * jk + 16 * kh, dt0, tr_row, tr_col);
        op[1] = read_tr<D>(kb, 32 * jk + 16 * kh, dt0 + 1, tr_row, tr_col);
      };
      bf16x8 db[2];
      auto runC = [&](int c, const bf16x8 (&op)[4]) {
        const int kh = c / (S::DT / 2), dt0 = 2 * (c % (S::DT / 2));
        dq[dt0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[0], db[kh], dq[dt0], 0, 0, 0);
        dq[dt0 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[1], db[kh], dq[dt0 + 1], 0, 0, 0);
      };
      bf16x8 op[2][4];
      readA(0, op[0]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < NA; ++c) {
        if (c + 1 < NA)
          readA(c + 1, op[(c + 1) & 1]);
        else
          readC(0, op[(c + 1) & 1]);
        runA(c, op[c & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // dS: sacc[r] = S^T[key c0 + 8(r/4) + 4g + r%4][row pos]; the masked path is chosen
      // once per sub-tile (uniform)
      auto phase_b = [&](auto masked_t) {
        constexpr bool masked = decltype(masked_t)::value;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c_log2, -lse2));
          if constexpr (masked) {
            const int kk = c0 + 8 * (r / 4) + 4 * g + r % 4;
            const bool vis = (kk <= pos) & (!sparse | (kk < a.sink) | (kk > pos - a.window));
            p = vis ? p : 0.f;
          }
          db[r / 8][r % 8] = (__bf16)(p * (pacc[r] - dlt));
        }
      };
      if (full_vis)
        phase_b(std::false_type{});
      else
        phase_b(std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      constexpr int NC = S::DT;  // two MFMAs per group
      constexpr int c_first = NA & 1;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + 1 < NC) readC(c + 1, op[(c + 1 + c_first) & 1]);
        runC(c, op[(c + c_first) & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // dq[dt][r] = dQ^T[dim 32dt + 8(r/4) + 4g + r%4][row cr]
  if (row_ok) {
    float* dqp = a.dq + ((int64_t)(q0 + cr) * Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = dq[dt][4 * q4 + e] * a.scale;
        *(f32x4*)(dqp + 32 * dt + 8 * q4 + 4 * g) = v4;
      }
  }
}

// dk, dv = sum over the G query heads of a KV head of their partials, in head order; grid
// (chunks, batch): the keys of sequence blockIdx.y, skipped as a whole when its packing breaks
// the bounds the dk/dv kernel checks (then it wrote no partials, and dk, dv stay unwritten).
__global__ __launch_bounds__(256) void bwd_dkv_reduce(BwdArgs a) {
  const int b = blockIdx.y;
  const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
  if (q0 < 0 || k0 < 0 || Lq > a.max_seqlen_q || Lk > a.max_seqlen_k || Lk < Lq ||
      a.cu_q[a.batch] > a.tq_cap || a.cu_k[a.batch] > a.tk_cap || Lk <= 0)
    return;
  const int G = a.n_heads_q / a.n_heads_kv;
  const int64_t row4 = (int64_t)a.n_heads_kv * a.head_dim / 4;  // float4 per key row
  const int64_t i0 = (int64_t)k0 * row4, n4 = (int64_t)Lk * row4;
  const int64_t slice4 = a.tk_cap * row4;
  const f32x4* kp = (const f32x4*)a.dk_part;
  const f32x4* vp = (const f32x4*)a.dv_part;
  for (int64_t i = i0 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < i0 + n4;
       i += (int64_t)gridDim.x * 256) {
    f32x4 sk = kp[i], sv = vp[i];
    for (int hh = 1; hh < G; ++hh) {
      sk += kp[hh * slice4 + i];
      sv += vp[hh * slice4 + i];
    }
    ((f32x4*)a.dk)[i] = sk;
    ((f32x4*)a.dv)[i] = sv;
  }
}

template <int D>
hipError_t launch_mfma(const BwdArgs& a, hipStream_t stream) {
  if (a.max_seqlen_q > 0) {
    const int tiles = (a.max_seqlen_q + kRowTile - 1) / kRowTile;
    bwd_dq_mfma<D><<<tiles * a.n_heads_q * a.batch, kThreads, 0, stream>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int ktiles = (a.max_seqlen_k + kKeyTile - 1) / kKeyTile;
  bwd_dkv_mfma<D><<<ktiles * a.n_heads_q * a.batch, kThreadsDkv, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_heads_q == a.n_heads_kv) return e;
  const int chunks = (2048 + a.batch - 1) / a.batch;  // about 2048 workgroups in all
  bwd_dkv_reduce<<<dim3(chunks, a.batch), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_backward_bf16_mfma(const BwdArgs& a, hipStream_t stream) {
  return a.head_dim == 128 ? launch_mfma<128>(a, stream) : launch_mfma<64>(a, stream);
}

}  // namespace ea
