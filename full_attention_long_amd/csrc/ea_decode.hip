// ea_decode.hip -- one decode step of the routed hybrid attention, split over the KV cache.
//
// What it computes (Elastic Attention blog post, section 2.1 "Attention Router": r = 0
// runs Full Attention, r = 1 runs Sparse Attention; section 1 and the gist.science
// explanation, section "问题所在", for the sparse pattern, read as attention sink + causal
// sliding window): sequence b holds L = seqlens[b] tokens in its cache, the newest being the
// query's own, and every query head h attends from position i = L - 1 under its mode,
//   O[b, h, :] = softmax(scale * q K^T + mask) V   over the visible keys of row i.
//
// Design (gfx950; the step is bound by HBM reads of the cache):
//   * decode_split_kernel: one workgroup (4 wavefronts) per (split, KV head, sequence) reads
//     up to kSplit cached keys once and serves every query head of the GQA group.  A group
//     whose heads are all sparse reads only its visible keys (sink and window, enumerated as
//     one index range); a group with a full head reads the whole cache and its sparse heads
//     mask the rest.  Rows are read with 16-byte loads, one row spread over D*elt/16 lanes.
//   * Scores: each lane holds its slice of q for every head of the group (pre-scaled by
//     scale * log2 e); partial dots reduce across the row's lanes with xor shuffles; the
//     workgroup keeps the split's scores in LDS, takes per-head max and exp2, and forms the
//     unnormalised P V with fp32 FMAs, reduced across wavefronts in LDS.
//   * decode_combine_kernel: per (sequence, head), merges the splits' (O, m, l) into O and
//     the log-sum-exp.
//   * A sequence whose length is outside [1, min(cap, max_seqlen)] gets NaN outputs; every
//     cache read is bounded by a buffer descriptor over that sequence's KV head.
#include <math.h>

#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int kThreads = 256;  // 4 wavefronts

template <typename T>
__device__ __forceinline__ void widen16(const u32x4 w, float* f);  // 16 bytes -> floats

template <>
__device__ __forceinline__ void widen16<__bf16>(const u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void widen16<float>(const u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}

// Visible-key bookkeeping of one (sequence, KV-head group) for the query at i = L - 1:
// n_vis keys, enumerated as v -> key(v).  A group with a full head enumerates [0, L); an
// all-sparse group enumerates the sink keys below the window, then the window [L - n_win, L).
struct KeyRange {
  int n_vis, n_sink_only, win_start;
  bool all;
  __device__ __forceinline__ int key(int v) const {
    return all ? v : (v < n_sink_only ? v : win_start + (v - n_sink_only));
  }
};

__device__ __forceinline__ KeyRange key_range(int L, bool any_full, int sink, int window) {
  KeyRange r;
  r.all = any_full;
  const int n_win = min(window, L);
  r.n_sink_only = any_full ? 0 : min(sink, max(0, L - window));
  r.win_start = L - n_win;
  r.n_vis = any_full ? L : r.n_sink_only + n_win;
  return r;
}

// Where the cached rows of one (sequence, KV head) live, and which row holds key j.
//   dense cache [batch, cap, Hkv, D]: key j at row j of the sequence, rows Hkv * D apart;
//   pooled cache [pool_rows, D]: the (b, kvh) region, rows D apart; a KV head with a full
//   query head keeps key j at row j, an all-sparse one the sink keys at rows j < sink and
//   the window in a ring of `window` rows: key j >= sink at row sink + (j - sink) % window.
//   The window keys of the query are consecutive, so the ring rows of those >= jb follow
//   from one remainder ra = (jb - sink) % window with a single wrap.
struct CacheView {
  int64_t elem0;        // element offset of row 0 in the K and V arrays
  uint32_t row_bytes;   // bytes between consecutive rows
  uint32_t span;        // bytes of the region (reads past it return zeros)
  int sink, window, jb, ra;
  bool ring, ok;
  __device__ __forceinline__ uint32_t row(int j) const {
    if (!ring || j < sink) return (uint32_t)j;
    const int t = ra + (j - jb);
    return (uint32_t)(sink + (t >= window ? t - window : t));
  }
};

// Pooled region of (b, kvh) and whether it can serve a query at L - 1: its rows lie in the
// pool, stay within 32-bit byte offsets, and hold every key the query can see (all L for a
// group with a full head, sink + window rows for a ring).
template <int D, int ELT>
__device__ __forceinline__ CacheView cache_view(const DecodeArgs& a, int b, int kvh, int L,
                                                bool any_full, const KeyRange& kr) {
  CacheView c;
  c.sink = a.sink;
  c.window = a.window;
  c.ring = false;
  c.jb = 0;
  c.ra = 0;
  if (!a.pooled) {
    c.elem0 = ((int64_t)b * a.cap * a.n_heads_kv + kvh) * D;
    c.row_bytes = (uint32_t)a.n_heads_kv * D * ELT;
    c.span = (uint32_t)(a.cap - 1) * c.row_bytes + D * ELT;
    c.ok = true;
    return c;
  }
  const int64_t base = a.region_base[(int64_t)b * a.n_heads_kv + kvh];
  const int32_t rows = a.region_rows[(int64_t)b * a.n_heads_kv + kvh];
  const int64_t need = any_full ? (int64_t)L : (int64_t)a.sink + a.window;
  c.ok = base >= 0 && rows >= 1 && base + rows <= a.pool_rows &&
         (int64_t)rows * D * ELT < ((int64_t)1 << 31) && rows >= need;
  c.elem0 = c.ok ? base * D : 0;
  c.row_bytes = D * ELT;
  c.span = c.ok ? (uint32_t)rows * D * ELT : 0;
  if (!any_full) {
    c.ring = true;
    c.jb = max(kr.win_start, a.sink);
    c.ra = (c.jb - a.sink) % a.window;
  }
  return c;
}

// GM: compile-time bound on the group size G (query heads per KV head).
template <typename T, int D, int GM>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int ELT = sizeof(T);
  constexpr int LPR = D * ELT / 16;      // lanes per cached row (16 bytes each)
  constexpr int RPP = 64 / LPR;          // rows per wavefront pass
  constexpr int DPL = 16 / ELT;          // dims per lane
  constexpr int KS = kDecodeSplit;       // keys per split
  __shared__ float s_p[GM][KS];          // scores, then P
  __shared__ float s_o[4][GM][D];        // per-wavefront partial P V
  __shared__ float s_m[GM], s_l[GM];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = a.seqlens[b];
  if (L < 1 || L > a.cap || L > a.max_seqlen) return;  // the combine kernel writes NaN
  // Route bytes and q slices of the group's heads, all loads issued before any is used
  // (head g >= G repeats head G - 1, so a bound check never serialises them).
  const int sub = lane % LPR, rsub = lane / LPR;  // slice index, row within the pass
  // One route byte per lane (lane l holds head min(l, G - 1)); a ballot gives every head's bit.
  const uint8_t* rt = a.route + (int64_t)b * Hq + kvh * G;
  const uint64_t sp_bits = __builtin_amdgcn_ballot_w64(rt[min(lane, G - 1)] != 0);
  const bool any_full = ~sp_bits != 0;
  u32x4 qraw[GM];
  bool sparse[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    const int gg = min(g, G - 1);
    sparse[g] = (sp_bits >> g) & 1;
    qraw[g] = *(const u32x4*)((const T*)a.q + ((int64_t)b * Hq + kvh * G + gg) * D + sub * DPL);
  }
  const KeyRange kr = key_range(L, any_full, a.sink, a.window);
  const CacheView cv = cache_view<D, ELT>(a, b, kvh, L, any_full, kr);
  const int v0 = split * KS;
  if (!cv.ok || v0 >= kr.n_vis) return;  // a region that cannot serve the query: NaN outputs
  const int nv = min(KS, kr.n_vis - v0);
  const int i = L - 1;

  const uint32_t row_bytes = cv.row_bytes, span = cv.span;
  const auto krs = make_rsrc((const T*)a.kc + cv.elem0, span);
  const auto vrs = make_rsrc((const T*)a.vc + cv.elem0, span);

  // q slices scaled by scale * log2(e), so that scores come out in log2 units
  const float c_log2 = a.scale * 1.4426950408889634f;
  float qv[GM][DPL];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    float f[DPL];
    widen16<T>(qraw[g], f);
#pragma unroll
    for (int e = 0; e < DPL; ++e) qv[g][e] = f[e] * c_log2;
  }

  // Each lane serves rows vi = wave*RPP + 4*RPP*p + rsub, p < NP, in chunks of CH rows whose
  // loads are all issued before any is used (HBM latency is hidden by loads in flight, not
  // by occupancy).  A row past the split's last visible key reads at offset `span`, outside
  // the buffer, and gets zeros.
  constexpr int NP = KS / (4 * RPP);
  constexpr int CH = NP < 16 ? NP : 16;
  auto row_off = [&](int p) __attribute__((always_inline)) {
    const int vi = wave * RPP + 4 * RPP * p + rsub;
    return vi < nv ? cv.row(kr.key(v0 + vi)) * row_bytes + sub * 16 : span;
  };

  // ---- scores of the split's keys
  u32x4 w[CH];
  for (int p0 = 0; p0 < NP; p0 += CH) {
#pragma unroll
    for (int c = 0; c < CH; ++c) w[c] = buf_load16(krs, row_off(p0 + c));
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int vi = wave * RPP + 4 * RPP * (p0 + c) + rsub;
      float kf[DPL];
      widen16<T>(w[c], kf);
      float dot[GM];
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc = __builtin_fmaf(qv[g][e], kf[e], acc);
        dot[g] = acc;
      }
      // sum over the LPR lanes of the row
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1)
#pragma unroll
        for (int g = 0; g < GM; ++g) dot[g] += __shfl_xor(dot[g], off);
      if (sub == 0) {
        const int j = vi < nv ? kr.key(v0 + vi) : 0;
#pragma unroll
        for (int g = 0; g < GM; ++g) {
          if (g < G) {
            // key j is visible to a sparse head iff j < sink or j > i - window
            const bool vis = vi < nv && (!sparse[g] || j < a.sink || j > i - a.window);
            s_p[g][vi] = vis ? dot[g] : -INFINITY;
          }
        }
      }
    }
  }
  // V rows of the first chunk are in flight while the softmax runs
#pragma unroll
  for (int c = 0; c < CH; ++c) w[c] = buf_load16(vrs, row_off(c));
  __syncthreads();

  // ---- per-head max, P = exp2(s - m), row sum: wavefront w takes heads w, w+4, ...
  for (int g = wave; g < G; g += 4) {
    float m = -INFINITY;
    for (int x = lane; x < KS; x += 64) m = fmaxf(m, s_p[g][x]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float mu = m == -INFINITY ? 0.f : m;
    float l = 0.f;
    for (int x = lane; x < KS; x += 64) {
      const float p = __builtin_amdgcn_exp2f(s_p[g][x] - mu);
      s_p[g][x] = p;
      l += p;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) {
      s_m[g] = m;
      s_l[g] = l;
    }
  }
  __syncthreads();

  // ---- P V over the same rows (rows past the split read zeros and have P = 0)
  float acc[GM][DPL];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[g][e] = 0.f;
  for (int p0 = 0; p0 < NP; p0 += CH) {
    if (p0 > 0) {
#pragma unroll
      for (int c = 0; c < CH; ++c) w[c] = buf_load16(vrs, row_off(p0 + c));
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int vi = wave * RPP + 4 * RPP * (p0 + c) + rsub;
      float vf[DPL];
      widen16<T>(w[c], vf);
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        const float p = g < G ? s_p[g][vi] : 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[g][e] = __builtin_fmaf(p, vf[e], acc[g][e]);
      }
    }
  }
  // reduce over the RPP rows of a pass (lanes with the same slice), then over wavefronts
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[g][e] += __shfl_xor(acc[g][e], off);
  if (rsub == 0) {
#pragma unroll
    for (int g = 0; g < GM; ++g)
      if (g < G)
#pragma unroll
        for (int e = 0; e < DPL; ++e) s_o[wave][g][sub * DPL + e] = acc[g][e];
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += kThreads) {
    const int g = x / D, d = x % D;
    const float o = (s_o[0][g][d] + s_o[1][g][d]) + (s_o[2][g][d] + s_o[3][g][d]);
    const int64_t bh = (int64_t)b * Hq + kvh * G + g;
    a.o_part[(bh * a.max_splits + split) * D + d] = o;
  }
  if (tid < G) {
    const int64_t bh = (int64_t)b * Hq + kvh * G + tid;
    a.ml_part[(bh * a.max_splits + split) * 2 + 0] = s_m[tid];
    a.ml_part[(bh * a.max_splits + split) * 2 + 1] = s_l[tid];
  }
}

// bf16 caches: the same split, with the scores on the matrix cores.  Wavefront w takes the
// split's keys [64 w, 64 w + 64) as 4 blocks of 16.  Scores of a block are one
// v_mfma_f32_16x16x32_bf16 per 32 dimensions: A = 16 keys x 32 dims, B = 32 dims x 16 query
// heads (heads past G repeat head G - 1 and are ignored).  The dot product does not depend on
// which dimensions fill which k slot, so lane l's A fragment is simply the 16-byte load of key
// row (l % 16), dimension chunk 4 t + l / 16, and the q fragment uses the same chunk: every
// operand comes straight from a load.  P V stays on the vector ALU over row-contiguous V loads
// (lane l: row l / (D / 8), 8 dims), with the split's P read from LDS as one vector per row.
template <int D, int GM>
__global__ __launch_bounds__(kThreads) void decode_split_bf16_kernel(DecodeArgs a) {
  constexpr int KS = kDecodeSplit;
  constexpr int KW = KS / 4;          // keys per wavefront
  constexpr int NB = KW / 16;         // 16-key blocks per wavefront
  constexpr int NT = D / 32;          // MFMA k steps (32 dims each)
  constexpr int LPR = D / 8;          // lanes per V row (16 bytes = 8 dims each)
  constexpr int RPP = 64 / LPR;       // V rows per wavefront load
  constexpr int NV = KW / RPP;        // V loads per lane
  static_assert(GM == 1 || GM == 2 || GM == 4 || GM == 8, "group bound");
  typedef float pvec __attribute__((ext_vector_type(GM)));
  __shared__ pvec s_p[KS];            // P of every key, one vector of GM heads per key
  __shared__ float s_mw[4][GM], s_lw[4][GM];
  __shared__ float s_o[4][GM][D];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the length, the route bytes and the q fragments do not depend on one another: all three
  // loads are in flight together
  const int L = a.seqlens[b];
  const uint8_t route_byte = a.route[(int64_t)b * Hq + kvh * G + min(lane, G - 1)];
  const int n = lane & 15, kq = lane >> 4;
  const __bf16* qh = (const __bf16*)a.q + ((int64_t)b * Hq + kvh * G + min(n, G - 1)) * D;
  u32x4 qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) qf[t] = *(const u32x4*)(qh + (4 * t + kq) * 8);
  // (a length outside the contract exits here too, with no cache read; the combine kernel
  // writes NaN for it)
  const bool bad_len = L < 1 || L > a.cap || L > a.max_seqlen;
  const uint64_t sp_bits = __builtin_amdgcn_ballot_w64(route_byte != 0);
  const bool any_full = ~sp_bits != 0;
  const KeyRange kr = key_range(L, any_full, a.sink, a.window);
  const CacheView cv = cache_view<D, 2>(a, b, kvh, L, any_full, kr);
  const int v0 = split * KS;
  if (bad_len || !cv.ok || v0 >= kr.n_vis) return;
  const int nv = min(KS, kr.n_vis - v0);
  const int iq = L - 1;

  const uint32_t row_bytes = cv.row_bytes, span = cv.span;
  const auto krs = make_rsrc((const __bf16*)a.kc + cv.elem0, span);
  const auto vrs = make_rsrc((const __bf16*)a.vc + cv.elem0, span);
  // byte offset of local key vi's row; past the split's last key: `span`, outside the buffer
  // (loads there return zeros; span + 256 < 2^32 since span < 2^31)
  auto row_off = [&](int vi) __attribute__((always_inline)) {
    return vi < nv ? cv.row(kr.key(v0 + vi)) * row_bytes : span;
  };

  // every K and V load of the split is issued here, K blocks first
  u32x4 kf[NB][NT];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const uint32_t off = row_off(wave * KW + 16 * blk + n);
#pragma unroll
    for (int t = 0; t < NT; ++t) kf[blk][t] = buf_load16(krs, off + (4 * t + kq) * 16);
  }
  const int vr = lane / LPR, vc = lane % LPR;
  u32x4 vf[NV];
#pragma unroll
  for (int p = 0; p < NV; ++p) vf[p] = buf_load16(vrs, row_off(wave * KW + p * RPP + vr) + vc * 16);

  // scores: lane l holds keys wave*KW + 16 blk + 4 (l / 16) + i of head l % 16
  const float c_log2 = a.scale * 1.4426950408889634f;
  const bool sp = (sp_bits >> min(n, G - 1)) & 1;
  float sc[NB][4];
  float mloc = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[blk][t]),
                                                    __builtin_bit_cast(bf16x8, qf[t]), acc, 0,
                                                    0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vi = wave * KW + 16 * blk + 4 * kq + i;
      const int j = vi < nv ? kr.key(v0 + vi) : 0;
      // key j is visible to a sparse head iff j < sink or j > i - window
      const bool vis = vi < nv && (!sp || j < a.sink || j > iq - a.window);
      sc[blk][i] = vis ? acc[i] * c_log2 : -INFINITY;
      mloc = fmaxf(mloc, sc[blk][i]);
    }
  }
  // per-head max over the split: lanes n, n+16, n+32, n+48, then the 4 wavefronts
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  if (lane < GM) s_mw[wave][lane] = mloc;
  __syncthreads();
  const int gn = min(n, GM - 1);
  const float M = fmaxf(fmaxf(s_mw[0][gn], s_mw[1][gn]), fmaxf(s_mw[2][gn], s_mw[3][gn]));
  const float Mu = M == -INFINITY ? 0.f : M;
  float lloc = 0.f;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(sc[blk][i] - Mu);
      lloc += p;
      if (n < GM) s_p[wave * KW + 16 * blk + 4 * kq + i][n] = p;
    }
  lloc += __shfl_xor(lloc, 16);
  lloc += __shfl_xor(lloc, 32);
  if (lane < GM) s_lw[wave][lane] = lloc;
  __syncthreads();

  // P V on the vector ALU (rows past the split read zeros and have P = 0)
  float acc[GM][8];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
#pragma unroll
  for (int p = 0; p < NV; ++p) {
    const pvec pw = s_p[wave * KW + p * RPP + vr];
    float v[8];
    widen16<__bf16>(vf[p], v);
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = __builtin_fmaf(pw[g], v[e], acc[g][e]);
  }
  // sum over the RPP rows of a load (lanes with the same chunk), then over wavefronts
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] += __shfl_xor(acc[g][e], off);
  if (vr == 0) {
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][g][vc * 8 + e] = acc[g][e];
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += kThreads) {
    const int g = x / D, d = x % D;
    const float o = (s_o[0][g][d] + s_o[1][g][d]) + (s_o[2][g][d] + s_o[3][g][d]);
    const int64_t bh = (int64_t)b * Hq + kvh * G + g;
    a.o_part[(bh * a.max_splits + split) * D + d] = o;
  }
  if (tid < G) {
    const int64_t bh = (int64_t)b * Hq + kvh * G + tid;
    const float Mg = fmaxf(fmaxf(s_mw[0][tid], s_mw[1][tid]), fmaxf(s_mw[2][tid], s_mw[3][tid]));
    a.ml_part[(bh * a.max_splits + split) * 2 + 0] = Mg;
    a.ml_part[(bh * a.max_splits + split) * 2 + 1] =
        (s_lw[0][tid] + s_lw[1][tid]) + (s_lw[2][tid] + s_lw[3][tid]);
  }
}

// Per (sequence, head): O = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), M = max_s m_s.
// 256 threads: a pass covers SR = 256 / (D / 4) split rows, one float4 of O_s per thread, and
// the SR row partials are summed in LDS at the end.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeArgs a) {
  constexpr int C4 = D / 4;             // float4 columns of a row
  constexpr int SR = kThreads / C4;     // split rows per pass
  __shared__ float s_red[kThreads / 64];
  __shared__ f32x4 s_acc[SR][C4];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int Hq = a.n_heads_q, G = Hq / a.n_heads_kv;
  const int L = a.seqlens[b];
  const int64_t bh = (int64_t)b * Hq + h;
  T* o = (T*)a.o + bh * D;
  if (L < 1 || L > a.cap || L > a.max_seqlen) {  // outside the contract: NaN, no reads
    for (int d = tid; d < D; d += kThreads) o[d] = (T)NAN;
    if (a.lse && tid == 0) a.lse[bh] = NAN;
    return;
  }
  const uint8_t* rt = a.route + (int64_t)b * Hq + (h / G) * G;
  const bool any_full = __builtin_amdgcn_ballot_w64(rt[min(tid & 63, G - 1)] == 0) != 0;
  const KeyRange kr = key_range(L, any_full, a.sink, a.window);
  if (!cache_view<D, sizeof(T)>(a, b, h / G, L, any_full, kr).ok) {  // no usable region: NaN
    for (int d = tid; d < D; d += kThreads) o[d] = (T)NAN;
    if (a.lse && tid == 0) a.lse[bh] = NAN;
    return;
  }
  const int ns = (kr.n_vis + kDecodeSplit - 1) / kDecodeSplit;
  const float* ml = a.ml_part + bh * a.max_splits * 2;
  const f32x4* op = (const f32x4*)(a.o_part + bh * a.max_splits * D);

  // M = max over splits
  float M = -INFINITY;
  for (int s = tid; s < ns; s += kThreads) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  // split weights 2^(m_s - M) (0 for a split with no visible key) and their l-weighted sum
  float lt = 0.f;
  for (int s = tid; s < ns; s += kThreads) {
    const float m = ml[2 * s];
    if (m != -INFINITY) lt += ml[2 * s + 1] * __builtin_amdgcn_exp2f(m - M);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lt += __shfl_xor(lt, off);
  if ((tid & 63) == 0) s_red[tid >> 6] = lt;
  __syncthreads();
  lt = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);

  // weighted sum of the splits' O rows
  const int c = tid % C4, r = tid / C4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = r; s < ns; s += SR) {
    const float m = ml[2 * s];
    const float wgt = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
    const f32x4 x = op[(int64_t)s * C4 + c];
    acc += wgt * x;
  }
  s_acc[r][c] = acc;
  __syncthreads();
  if (tid < C4) {
    f32x4 t = s_acc[0][tid];
#pragma unroll
    for (int rr = 1; rr < SR; ++rr) t += s_acc[rr][tid];
    const float inv = 1.0f / lt;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[4 * tid + e] = (T)(t[e] * inv);
  }
  // scores were in log2 units: lse = (M + log2 l) * ln 2
  if (a.lse && tid == 0) a.lse[bh] = (M + log2f(lt)) * 0.6931471805599453f;
}

// ---- pooled cache writers

// Region of (b, kvh) and the row of position j in it, or -1 where the position is not kept
// (a ring keeps the sink and the last `window` positions before `upto`) or the region is
// unusable (outside the pool, or too small for the row).
__device__ __forceinline__ int64_t pool_row(const PoolWriteArgs& a, int b, int kvh, int j,
                                            int upto, int row_bytes) {
  const int G = a.n_heads_q / a.n_heads_kv;
  const uint8_t* rt = a.route + (int64_t)b * a.n_heads_q + kvh * G;
  bool any_full = false;
  for (int g = 0; g < G; ++g) any_full |= rt[g] == 0;
  const int64_t base = a.region_base[(int64_t)b * a.n_heads_kv + kvh];
  const int32_t rows = a.region_rows[(int64_t)b * a.n_heads_kv + kvh];
  if (base < 0 || rows < 1 || base + rows > a.pool_rows ||
      (int64_t)rows * row_bytes >= ((int64_t)1 << 31) || j < 0)
    return -1;
  int64_t r;
  if (any_full) {
    r = j;
  } else {
    if (!(j < a.sink || j >= upto - a.window)) return -1;
    r = j < a.sink ? j : a.sink + (j - a.sink) % a.window;
  }
  return r < rows ? base + r : -1;
}

// Prefill K/V of packed sequences into the pool: workgroup (block of 64 positions, kvh, b),
// one 16-byte chunk of a K or V row per thread.
__global__ __launch_bounds__(256) void pool_fill_kernel(PoolWriteArgs a, int row_bytes) {
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int seq0 = a.cu[b], L = a.cu[b + 1] - seq0;
  const int chunks = row_bytes / 16, rpp = 256 / chunks;
  const int c = threadIdx.x % chunks;
  const int j1 = min(L, (int)(blockIdx.x + 1) * 64);
  for (int j = blockIdx.x * 64 + threadIdx.x / chunks; j < j1; j += rpp) {
    const int64_t r = pool_row(a, b, kvh, j, L, row_bytes);
    if (r < 0) continue;
    const int64_t src = ((int64_t)(seq0 + j) * a.n_heads_kv + kvh) * row_bytes + c * 16;
    const int64_t dst = r * row_bytes + c * 16;
    *(u32x4*)((char*)a.k_pool + dst) = *(const u32x4*)((const char*)a.k + src);
    *(u32x4*)((char*)a.v_pool + dst) = *(const u32x4*)((const char*)a.v + src);
  }
}

// One new K/V row per (sequence, KV head), at position positions[b] (the ring keeps it as the
// newest of its window); workgroup (kvh, b), one 16-byte chunk per thread (K then V).
__global__ __launch_bounds__(64) void pool_append_kernel(PoolWriteArgs a, int row_bytes) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int j = a.positions[b];
  const int64_t r = pool_row(a, b, kvh, j, j + 1, row_bytes);
  const int chunks = row_bytes / 16;
  const int t = threadIdx.x;
  if (r < 0 || t >= 2 * chunks) return;
  const bool is_v = t >= chunks;
  const int c = is_v ? t - chunks : t;
  const int64_t src = ((int64_t)b * a.n_heads_kv + kvh) * row_bytes + c * 16;
  const int64_t dst = r * row_bytes + c * 16;
  *(u32x4*)((char*)(is_v ? a.v_pool : a.k_pool) + dst) =
      *(const u32x4*)((const char*)(is_v ? a.v : a.k) + src);
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, int G, hipStream_t stream) {
  const dim3 grid(a.max_splits, a.n_heads_kv, a.batch);
  if constexpr (sizeof(T) == 2) {
    if (G <= 1)
      decode_split_bf16_kernel<D, 1><<<grid, kThreads, 0, stream>>>(a);
    else if (G <= 2)
      decode_split_bf16_kernel<D, 2><<<grid, kThreads, 0, stream>>>(a);
    else if (G <= 4)
      decode_split_bf16_kernel<D, 4><<<grid, kThreads, 0, stream>>>(a);
    else
      decode_split_bf16_kernel<D, 8><<<grid, kThreads, 0, stream>>>(a);
  } else if (G <= 1)
    decode_split_kernel<T, D, 1><<<grid, kThreads, 0, stream>>>(a);
  else if (G <= 2)
    decode_split_kernel<T, D, 2><<<grid, kThreads, 0, stream>>>(a);
  else if (G <= 4)
    decode_split_kernel<T, D, 4><<<grid, kThreads, 0, stream>>>(a);
  else
    decode_split_kernel<T, D, 8><<<grid, kThreads, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<T, D><<<dim3(a.n_heads_q, a.batch), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool_fill(const PoolWriteArgs& a, int elem_bytes, hipStream_t stream) {
  const int row_bytes = a.head_dim * elem_bytes;
  const dim3 grid((a.max_seqlen + 63) / 64, a.n_heads_kv, a.batch);
  pool_fill_kernel<<<grid, 256, 0, stream>>>(a, row_bytes);
  return hipGetLastError();
}

hipError_t launch_pool_append(const PoolWriteArgs& a, int elem_bytes, hipStream_t stream) {
  const int row_bytes = a.head_dim * elem_bytes;
  pool_append_kernel<<<dim3(a.n_heads_kv, a.batch), 64, 0, stream>>>(a, row_bytes);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  const int G = a.n_heads_q / a.n_heads_kv;
  if (bf16)
    return a.head_dim == 128 ? launch_decode_t<__bf16, 128>(a, G, stream)
                             : launch_decode_t<__bf16, 64>(a, G, stream);
  return a.head_dim == 128 ? launch_decode_t<float, 128>(a, G, stream)
                           : launch_decode_t<float, 64>(a, G, stream);
}

}  // namespace ea
