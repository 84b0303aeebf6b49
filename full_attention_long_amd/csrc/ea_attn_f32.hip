// ea_attn_f32.hip -- persistent routed hybrid-attention prefill in fp32 (the accuracy
// path).  Same work list, visit plan and mask as the bf16 MFMA kernel (Elastic Attention
// blog post, sections 2.1 and 3: per-head routing to full or sparse attention inside one
// launch; sparse = attention sink + causal sliding window), computed with fp32 FMAs.
//
// One workgroup = 256 threads = 64 query rows x 4 threads; each thread owns a quarter of
// the head dimension of its row's q and o.  Key/value tiles of 32 keys are staged in LDS;
// a score is the sum of the four quarter dot products (two xor shuffles), softmax uses
// expf on fp32 state, and nothing is rounded below fp32.
#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int BM = kF32BM;  // 64 rows
constexpr int BN = kF32BN;  // 32 keys
constexpr int kThreads = 256;
constexpr int kParts = 4;   // threads per query row

struct Visit {
  int n1, s2, t_hi, count;
  __device__ __forceinline__ int tile(int n) const { return n < n1 ? n : s2 + (n - n1); }
};

__device__ __forceinline__ Visit make_visit(bool sparse, int m0, int m1, int sink, int window) {
  Visit v;
  v.t_hi = (m1 - 1) / BN;
  if (sparse) {
    v.n1 = (min(sink, m1) + BN - 1) / BN;
    v.s2 = max(max(0, m0 - window + 1) / BN, v.n1);
  } else {
    v.n1 = 0;
    v.s2 = 0;
  }
  v.count = v.n1 + max(0, v.t_hi - v.s2 + 1);
  return v;
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnArgs a) {
  constexpr int DP = D / kParts;    // head-dim elements per thread
  constexpr int RS = D + 4;         // LDS row stride (floats)
  __shared__ __attribute__((aligned(16))) float ks[BN * RS];
  __shared__ __attribute__((aligned(16))) float vs[BN * RS];
  __shared__ int s_item;

  const int tid = threadIdx.x;
  const int row = tid / kParts, part = tid % kParts;
  const int Hq = a.n_heads_q, Hkv = a.n_heads_kv, group = Hq / Hkv;
  const int n_items = min(*a.n_items, a.item_cap);
  const int total_tokens = a.cu[a.batch];

  for (;;) {
    if (tid == 0) s_item = atomicAdd(&a.queue[0], 1);
    __syncthreads();
    const int it = s_item;
    if (it < 0 || it >= n_items) break;  // a corrupt queue head ends the loop too
    const int4 item = a.items[it];
    const int b = item.x, h = item.y, qt = item.z;
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
    // keys: the sequence's own packing, or the KV-prefix packing of a chunked prefill whose
    // chunk row r sits at position off + r
    const int seq0k = a.cu_k ? a.cu_k[b] : seq0;
    const int len_k = a.cu_k ? a.cu_k[b + 1] - seq0k : len;
    const int off = len_k - len;
    const int m0 = off + qt * BM, m1 = off + min(qt * BM + BM, len);  // positions
    const int kvh = h / group;
    const bool sparse = a.route[(int64_t)b * Hq + h] != 0;
    const Visit vis = make_visit(sparse, m0, m1, a.sink, a.window);
    const int qi = m0 + row;       // position of this thread's query
    const int qrow = qi - off;     // its chunk row
    const bool live = qi < m1;

    float q[DP], o[DP];
    const float* qp = (const float*)a.q + ((int64_t)(seq0 + qrow) * Hq + h) * D + part * DP;
#pragma unroll
    for (int e = 0; e < DP; ++e) {
      q[e] = live ? qp[e] : 0.f;
      o[e] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;

    for (int n = 0; n < vis.count; ++n) {
      const int kt = vis.tile(n);
      // stage the key/value tile; keys past the sequence end read as zero
      for (int idx = tid; idx < BN * (D / 4); idx += kThreads) {
        const int kr = idx / (D / 4), c4 = idx % (D / 4);
        const int key = kt * BN + kr;
        f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
        if (key < len_k) {
          const int64_t at = ((int64_t)(seq0k + key) * Hkv + kvh) * D + c4 * 4;
          kv = *(const f32x4*)((const float*)a.k + at);
          vv = *(const f32x4*)((const float*)a.v + at);
        }
        *(f32x4*)(ks + kr * RS + c4 * 4) = kv;
        *(f32x4*)(vs + kr * RS + c4 * 4) = vv;
      }
      __syncthreads();

      float s[BN];
      float mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < DP; ++e) dot = __builtin_fmaf(q[e], ks[j * RS + part * DP + e], dot);
        dot += __shfl_xor(dot, 1, 64);
        dot += __shfl_xor(dot, 2, 64);
        const int kj = kt * BN + j;
        const bool visible = kj <= qi && (!sparse || kj < a.sink || kj > qi - a.window);
        s[j] = visible ? dot * a.scale : -INFINITY;
        mt = fmaxf(mt, s[j]);
      }
      const float m_new = fmaxf(m_run, mt);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = expf(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) o[e] *= alpha;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        const float p = expf(s[j] - m_use);
        psum += p;
#pragma unroll
        for (int e = 0; e < DP; ++e) o[e] = __builtin_fmaf(p, vs[j * RS + part * DP + e], o[e]);
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      __syncthreads();
    }

    if (live) {
      float* op = (float*)a.o + ((int64_t)(seq0 + qrow) * Hq + h) * D + part * DP;
      const float inv = 1.0f / l_run;
#pragma unroll
      for (int e = 0; e < DP; ++e) op[e] = o[e] * inv;
      if (a.lse && part == 0) {
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        a.lse[(int64_t)h * total_tokens + seq0 + qrow] = m_use + logf(l_run);
      }
    }
    __syncthreads();
  }
  // The last workgroup out leaves the queue counters at zero for the next launch.
  if (tid == 0 && atomicAdd(&a.queue[1], 1) == (int)gridDim.x - 1) {
    atomicExch(&a.queue[0], 0);
    atomicExch(&a.queue[1], 0);
  }
}

}  // namespace

int attn_f32_blocks_per_cu() { return 2; }

hipError_t launch_attn_f32(const AttnArgs& a, int grid, hipStream_t stream) {
  if (a.head_dim == 128)
    attn_f32_kernel<128><<<grid, kThreads, 0, stream>>>(a);
  else
    attn_f32_kernel<64><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ea
