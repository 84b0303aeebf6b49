// ea_backward.hip -- backward of the routed hybrid attention (training of the method).
//
// What it computes (Elastic Attention blog post, section 2.1: r = 0 runs Full Attention,
// r = 1 Sparse Attention, and the "training trick" of the same section: the model is trained
// through its routed attention, so gradients flow through both kinds of head; the sparse
// pattern as in the forward: attention sink + causal sliding window): for every sequence b,
// query head h and query row i (position i = Lk - Lq + r of chunk row r), with P the softmax
// of the forward,
//   D_i  = <dO_i, O_i>,  dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - D_i)  (visible j),
//   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i,   dV_j = sum_i P_ij dO_i,
// dK and dV summed over the query heads of a KV head.  P is recomputed from the forward's
// log-sum-exp: P_ij = exp(scale <q_i, k_j> - lse_i).
//
// Design (fp32 inputs; bf16 inputs take the matrix-core kernels of ea_backward_bf16.hip after
// the D kernel here; fp32 arithmetic on the vector ALU, deterministic, no atomics):
//   * bwd_delta_kernel: D for every (row, head), both dtypes (and lse * log2(e) for bf16).
//   * bwd_dq_kernel: one workgroup per (64-row q-tile, head, sequence), 4 threads per row
//     (D/4 dimensions each); the item's key tiles (the forward's visit plan) staged through LDS
//     as fp32; per key: two 4-lane dot products (score, dP), then dQ += dS k.
//   * bwd_dkv_kernel: one workgroup per (64-key tile, KV head, sequence), 4 threads per key,
//     k and v of the key in registers; for every query head of the group, the query rows that
//     can see the tile (all later rows for a full head or a tile holding sink keys, else the
//     next `window` positions) staged through LDS with their lse and D; dV += P dO, dK += dS q.
#include <math.h>

#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int kBwdRows = 64;     // q rows per dQ workgroup, keys per dK/dV workgroup
constexpr int kBwdTile = 32;     // keys (dQ) or rows (dK/dV) staged per step
constexpr int kBwdThreads = 256; // 64 x 4

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) {
  return (float)p[i];
}

__device__ __forceinline__ bool visible(int i, int j, bool sparse, int sink, int window) {
  return j <= i && (!sparse || j < sink || j > i - window);
}

// D[h * Tq + t] = <dO[t, h, :], O[t, h, :]> (and lse2 = lse * log2(e) for the matrix-core
// kernels): each lane reads one 16-byte chunk of a (t, h) row, the D*elt/16 lanes of a row add
// their partial sums in lane order (butterfly), a grid-stride loop over the rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  constexpr int EPC = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int LPR = D / EPC;          // lanes per row (8..32)
  constexpr int RPB = 256 / LPR;        // rows per workgroup pass
  const int Tq = a.cu_q[a.batch];
  if (Tq < 0 || Tq > a.tq_cap) return;  // packing beyond the host's sizing: nothing written
  const int64_t n = (int64_t)Tq * a.n_heads_q;
  const int sub = threadIdx.x % LPR;
  for (int64_t w = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR; w - threadIdx.x / LPR < n;
       w += (int64_t)gridDim.x * RPB) {
    float acc = 0.f;
    if (w < n) {
      const int64_t at = w * D + sub * EPC;  // rows [t][h] are contiguous: w = t * Hq + h
      if constexpr (sizeof(T) == 2) {
        const u32x4 ro = *(const u32x4*)((const T*)a.o + at);
        const u32x4 rg = *(const u32x4*)((const T*)a.dout + at);
        const T* o = (const T*)&ro;
        const T* gg = (const T*)&rg;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc = __builtin_fmaf((float)o[e], (float)gg[e], acc);
      } else {
        const f32x4 o = *(const f32x4*)((const T*)a.o + at);
        const f32x4 gg = *(const f32x4*)((const T*)a.dout + at);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc = __builtin_fmaf(o[e], gg[e], acc);
      }
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (w < n && sub == 0) {
      const int64_t t = w / a.n_heads_q;
      const int h = (int)(w % a.n_heads_q);
      a.delta[(int64_t)h * Tq + t] = acc;
      // the matrix-core kernels stage lse in base-2 units
      if (a.lse2) a.lse2[(int64_t)h * Tq + t] = a.lse[(int64_t)h * Tq + t] * 1.4426950408889634f;
    }
  }
}

// visit plan of the forward for positions [p0, p1): key tiles of kBwdTile keys
struct KVPlan {
  int n1, s2, t_hi, count;
  __device__ __forceinline__ int tile(int n) const { return n < n1 ? n : s2 + (n - n1); }
};
__device__ __forceinline__ KVPlan kv_plan(bool sparse, int p0, int p1, int sink, int window) {
  KVPlan v;
  v.t_hi = (p1 - 1) / kBwdTile;
  if (sparse) {
    v.n1 = (min(sink, p1) + kBwdTile - 1) / kBwdTile;
    v.s2 = max(max(0, p0 - window + 1) / kBwdTile, v.n1);
  } else {
    v.n1 = 0;
    v.s2 = 0;
  }
  v.count = v.n1 + max(0, v.t_hi - v.s2 + 1);
  return v;
}

template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(BwdArgs a) {
  constexpr int DP = D / 4;
  constexpr int RS = D + 4;  // padded LDS row (floats)
  __shared__ float ks[kBwdTile * RS], vs[kBwdTile * RS];
  // the last q-tiles see the most keys: dispatch them first
  const int qt = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, G = Hq / Hkv, kvh = h / G;
  const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
  const int Tq = a.cu_q[a.batch];
  // a chunk longer than its keys, or a packing beyond the host's sizing: nothing written
  if (q0 < 0 || k0 < 0 || Lq > a.max_seqlen_q || Lk > a.max_seqlen_k || Lk < Lq ||
      Tq > a.tq_cap)
    return;
  if (qt * kBwdRows >= Lq) return;
  const int off = Lk - Lq;
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int r = qt * kBwdRows + row;               // chunk row
  const bool live = r < Lq;
  const int pos = off + r;                         // its position
  const int p0 = off + qt * kBwdRows, p1 = off + min(qt * kBwdRows + kBwdRows, Lq);
  const bool sparse = a.route[(int64_t)b * Hq + h] != 0;
  const KVPlan plan = kv_plan(sparse, p0, p1, a.sink, a.window);
  float q[DP], g[DP], dq[DP];
  const int64_t qi = ((int64_t)(q0 + (live ? r : 0)) * Hq + h) * D + part * DP;
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    q[e] = live ? ld((const T*)a.q, qi + e) : 0.f;
    g[e] = live ? ld((const T*)a.dout, qi + e) : 0.f;
    dq[e] = 0.f;
  }
  const float lse = live ? a.lse[(int64_t)h * Tq + q0 + r] : 0.f;
  const float Di = live ? a.delta[(int64_t)h * Tq + q0 + r] : 0.f;
  for (int n = 0; n < plan.count; ++n) {
    const int kt = plan.tile(n);
    __syncthreads();
    for (int idx = threadIdx.x; idx < kBwdTile * D; idx += kBwdThreads) {
      const int kr = idx / D, c = idx % D;
      const int key = kt * kBwdTile + kr;
      float kv = 0.f, vv = 0.f;
      if (key < Lk) {
        const int64_t at = ((int64_t)(k0 + key) * Hkv + kvh) * D + c;
        kv = ld((const T*)a.k, at);
        vv = ld((const T*)a.v, at);
      }
      ks[kr * RS + c] = kv;
      vs[kr * RS + c] = vv;
    }
    __syncthreads();
    for (int jj = 0; jj < kBwdTile; ++jj) {
      const int j = kt * kBwdTile + jj;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) {
        s = __builtin_fmaf(q[e], ks[jj * RS + part * DP + e], s);
        dp = __builtin_fmaf(g[e], vs[jj * RS + part * DP + e], dp);
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      dp += __shfl_xor(dp, 1, 64);
      dp += __shfl_xor(dp, 2, 64);
      const bool vis = live && j < Lk && visible(pos, j, sparse, a.sink, a.window);
      const float p = vis ? expf(s * a.scale - lse) : 0.f;
      const float ds = p * (dp - Di) * a.scale;
#pragma unroll
      for (int e = 0; e < DP; ++e) dq[e] = __builtin_fmaf(ds, ks[jj * RS + part * DP + e], dq[e]);
    }
  }
  if (live) {
    float* out = a.dq + ((int64_t)(q0 + r) * Hq + h) * D + part * DP;
#pragma unroll
    for (int e = 0; e < DP; ++e) out[e] = dq[e];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkv_kernel(BwdArgs a) {
  constexpr int DP = D / 4;
  constexpr int RS = D + 4;
  __shared__ float qs[kBwdTile * RS], gs[kBwdTile * RS];
  __shared__ float s_lse[kBwdTile], s_d[kBwdTile];
  const int kt = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, G = Hq / Hkv;
  const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
  const int Tq = a.cu_q[a.batch];
  if (q0 < 0 || k0 < 0 || Lq > a.max_seqlen_q || Lk > a.max_seqlen_k || Lk < Lq ||
      Tq > a.tq_cap)
    return;
  if (kt * kBwdRows >= Lk) return;
  const int off = Lk - Lq;
  const int kr = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int j = kt * kBwdRows + kr;   // this thread's key position
  const bool live = j < Lk;
  const int j0 = kt * kBwdRows, j1 = min(j0 + kBwdRows, Lk);
  float kk[DP], vv[DP], dk[DP], dv[DP];
  const int64_t ki = ((int64_t)(k0 + (live ? j : 0)) * Hkv + kvh) * D + part * DP;
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    kk[e] = live ? ld((const T*)a.k, ki + e) : 0.f;
    vv[e] = live ? ld((const T*)a.v, ki + e) : 0.f;
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  for (int hh = 0; hh < G; ++hh) {
    const int h = kvh * G + hh;
    const bool sparse = a.route[(int64_t)b * Hq + h] != 0;
    // positions that can see a key of [j0, j1): from j0 on; for a sparse head without sink
    // keys in the tile, only up to j1 - 1 + window - 1
    const int pe = (!sparse || j0 < a.sink) ? Lk : min(Lk, j1 - 1 + a.window);
    const int pb = max(j0, off);                     // rows exist from position off on
    for (int p = pb; p < pe; p += kBwdTile) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < kBwdTile * D; idx += kBwdThreads) {
        const int rr = idx / D, c = idx % D;
        const int pos = p + rr;
        float qv = 0.f, gv = 0.f;
        if (pos < pe) {
          const int64_t at = ((int64_t)(q0 + pos - off) * Hq + h) * D + c;
          qv = ld((const T*)a.q, at);
          gv = ld((const T*)a.dout, at);
        }
        qs[rr * RS + c] = qv;
        gs[rr * RS + c] = gv;
      }
      if (threadIdx.x < kBwdTile) {
        const int pos = p + threadIdx.x;
        const bool ok = pos < pe;
        s_lse[threadIdx.x] = ok ? a.lse[(int64_t)h * Tq + q0 + pos - off] : 0.f;
        s_d[threadIdx.x] = ok ? a.delta[(int64_t)h * Tq + q0 + pos - off] : 0.f;
      }
      __syncthreads();
      for (int rr = 0; rr < kBwdTile; ++rr) {
        const int pos = p + rr;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < DP; ++e) {
          s = __builtin_fmaf(kk[e], qs[rr * RS + part * DP + e], s);
          dp = __builtin_fmaf(vv[e], gs[rr * RS + part * DP + e], dp);
        }
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        dp += __shfl_xor(dp, 1, 64);
        dp += __shfl_xor(dp, 2, 64);
        const bool vis = live && pos < pe && visible(pos, j, sparse, a.sink, a.window);
        const float pr = vis ? expf(s * a.scale - s_lse[rr]) : 0.f;
        const float ds = pr * (dp - s_d[rr]) * a.scale;
#pragma unroll
        for (int e = 0; e < DP; ++e) {
          dv[e] = __builtin_fmaf(pr, gs[rr * RS + part * DP + e], dv[e]);
          dk[e] = __builtin_fmaf(ds, qs[rr * RS + part * DP + e], dk[e]);
        }
      }
    }
  }
  if (live) {
    const int64_t at = ((int64_t)(k0 + j) * Hkv + kvh) * D + part * DP;
#pragma unroll
    for (int e = 0; e < DP; ++e) {
      a.dk[at + e] = dk[e];
      a.dv[at + e] = dv[e];
    }
  }
}

template <typename T, int D>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  hipError_t e;
  if (a.max_seqlen_q > 0) {
    bwd_delta_kernel<T, D><<<2048, 256, 0, stream>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2) {
    // bf16: the matrix-core kernels
    return launch_attn_backward_bf16_mfma(a, stream);
  } else {
    // fp32: the vector-ALU kernels
    if (a.max_seqlen_q > 0) {  // no query rows: no dq, but dk = dv = 0 below
      bwd_dq_kernel<T, D><<<dim3((a.max_seqlen_q + kBwdRows - 1) / kBwdRows, a.n_heads_q,
                                 a.batch),
                            kBwdThreads, 0, stream>>>(a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    bwd_dkv_kernel<T, D><<<dim3((a.max_seqlen_k + kBwdRows - 1) / kBwdRows, a.n_heads_kv,
                                a.batch),
                           kBwdThreads, 0, stream>>>(a);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_attn_backward(const BwdArgs& a, bool bf16, hipStream_t stream) {
  if (bf16)
    return a.head_dim == 128 ? launch_bwd_t<__bf16, 128>(a, stream)
                             : launch_bwd_t<__bf16, 64>(a, stream);
  return a.head_dim == 128 ? launch_bwd_t<float, 128>(a, stream) : launch_bwd_t<float, 64>(a, stream);
}

}  // namespace ea
