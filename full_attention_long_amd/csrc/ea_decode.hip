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

__device__ __forceinline__ bool group_has_full(const uint8_t* route, int b, int Hq, int kvh,
                                               int G) {
  bool any = false;
  for (int g = 0; g < G; ++g) any |= route[(int64_t)b * Hq + kvh * G + g] == 0;
  return any;
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
  const bool any_full = group_has_full(a.route, b, Hq, kvh, G);
  const KeyRange kr = key_range(L, any_full, a.sink, a.window);
  const int v0 = split * KS;
  if (v0 >= kr.n_vis) return;
  const int nv = min(KS, kr.n_vis - v0);
  const int i = L - 1;

  // this sequence's rows of KV head kvh: row j at byte j * Hkv * D * ELT
  const uint32_t row_bytes = (uint32_t)Hkv * D * ELT;
  const int64_t base = ((int64_t)b * a.cap * Hkv + kvh) * D;
  const uint32_t span = (uint32_t)(a.cap - 1) * row_bytes + D * ELT;
  const auto krs = make_rsrc((const T*)a.kc + base, span);
  const auto vrs = make_rsrc((const T*)a.vc + base, span);

  // q slice of every head of the group, scaled by scale * log2(e)
  const int sub = lane % LPR, rsub = lane / LPR;  // slice index, row within the pass
  const float c_log2 = a.scale * 1.4426950408889634f;
  float qv[GM][DPL];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    if (g < G) {
      const T* qp = (const T*)a.q + ((int64_t)b * Hq + kvh * G + g) * D + sub * DPL;
      float f[DPL];
      widen16<T>(*(const u32x4*)qp, f);
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[g][e] = f[e] * c_log2;
    }
  }
  bool sparse[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g)
    sparse[g] = g < G && a.route[(int64_t)b * Hq + kvh * G + g] != 0;

  // ---- scores of the split's keys: wavefront w takes local rows w*RPP + 4*RPP*p, ...
  for (int r0 = wave * RPP; r0 < KS; r0 += 4 * RPP) {
    const int vi = r0 + rsub;  // local index of this lane's row
    const bool live = vi < nv;
    const int j = live ? kr.key(v0 + vi) : 0;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (live) w = buf_load16(krs, (uint32_t)j * row_bytes + sub * 16);
    float kf[DPL];
    widen16<T>(w, kf);
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
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        if (g < G) {
          // key j is visible to a sparse head iff j < sink or j > i - window
          const bool vis = live && (!sparse[g] || j < a.sink || j > i - a.window);
          s_p[g][vi] = vis ? dot[g] : -INFINITY;
        }
      }
    }
  }
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

  // ---- P V: wavefront w takes the same rows as in the score pass
  float acc[GM][DPL];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[g][e] = 0.f;
  for (int r0 = wave * RPP; r0 < KS; r0 += 4 * RPP) {
    const int vi = r0 + rsub;
    if (vi < nv) {
      const int j = kr.key(v0 + vi);
      float vf[DPL];
      widen16<T>(buf_load16(vrs, (uint32_t)j * row_bytes + sub * 16), vf);
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

// Per (sequence, head): O = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), M = max_s m_s.
template <typename T>
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int Hq = a.n_heads_q, G = Hq / a.n_heads_kv, D = a.head_dim;
  const int L = a.seqlens[b];
  const int64_t bh = (int64_t)b * Hq + h;
  T* o = (T*)a.o + bh * D;
  if (L < 1 || L > a.cap || L > a.max_seqlen) {  // outside the contract: NaN, no reads
    for (int d = threadIdx.x; d < D; d += blockDim.x) o[d] = (T)NAN;
    if (a.lse && threadIdx.x == 0) a.lse[bh] = NAN;
    return;
  }
  const bool any_full = group_has_full(a.route, b, Hq, h / G, G);
  const KeyRange kr = key_range(L, any_full, a.sink, a.window);
  const int ns = (kr.n_vis + kDecodeSplit - 1) / kDecodeSplit;
  const float* ml = a.ml_part + bh * a.max_splits * 2;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
  float lt = 0.f;
  for (int s = 0; s < ns; ++s)
    if (ml[2 * s] != -INFINITY) lt += ml[2 * s + 1] * __builtin_amdgcn_exp2f(ml[2 * s] - M);
  const float inv = 1.0f / lt;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < ns; ++s)
      if (ml[2 * s] != -INFINITY)
        acc += a.o_part[(bh * a.max_splits + s) * D + d] * __builtin_amdgcn_exp2f(ml[2 * s] - M);
    o[d] = (T)(acc * inv);
  }
  // scores were in log2 units: lse = (M + log2 l) * ln 2
  if (a.lse && threadIdx.x == 0) a.lse[bh] = (M + log2f(lt)) * 0.6931471805599453f;
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, int G, hipStream_t stream) {
  const dim3 grid(a.max_splits, a.n_heads_kv, a.batch);
  if (G <= 1)
    decode_split_kernel<T, D, 1><<<grid, kThreads, 0, stream>>>(a);
  else if (G <= 2)
    decode_split_kernel<T, D, 2><<<grid, kThreads, 0, stream>>>(a);
  else if (G <= 4)
    decode_split_kernel<T, D, 4><<<grid, kThreads, 0, stream>>>(a);
  else
    decode_split_kernel<T, D, 8><<<grid, kThreads, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<T><<<dim3(a.n_heads_q, a.batch), 128, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  const int G = a.n_heads_q / a.n_heads_kv;
  if (bf16)
    return a.head_dim == 128 ? launch_decode_t<__bf16, 128>(a, G, stream)
                             : launch_decode_t<__bf16, 64>(a, G, stream);
  return a.head_dim == 128 ? launch_decode_t<float, 128>(a, G, stream)
                           : launch_decode_t<float, 64>(a, G, stream);
}

}  // namespace ea
