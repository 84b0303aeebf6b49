// ea_router.hip -- the Attention Router (Elastic Attention blog post, section 2.1: the
// router reads the current key hidden states, an MLP emits one routing signal per head,
// r = 0 full attention, r = 1 sparse attention; about 0.27M parameters per layer for an
// 8B model, section 2.2).
//
// Step 1 (route_pool): each sequence is cut into `chunks` row ranges; one workgroup sums
// the key states of one range column by column in fp32, in a fixed order, and writes the
// partial sums.  This is a streaming read of the key states (HBM bound).
// Step 2 (route_mlp): one workgroup per sequence adds the partials in chunk order, divides
// by the length (an empty sequence pools to zero), runs W1/SiLU/W2 with wavefront dot
// products and thresholds z > 0.  No float atomics anywhere, so the bits are reproducible.
#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int kPoolThreads = 256;
constexpr int kMlpThreads = 256;

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

template <typename T, int VW>
__device__ __forceinline__ void add_row(const T* p, float* acc) {
  if constexpr (VW * sizeof(T) == 16) {
    u32x4 raw = *(const u32x4*)p;
    const T* vals = (const T*)&raw;
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[e] += to_f32(vals[e]);
  } else {
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[e] += to_f32(p[e]);
  }
}

// One workgroup sums rows [r0, r1) of sequence `blockIdx.y` (chunk `blockIdx.x`), VW
// consecutive columns per thread.  When a row has fewer column groups than threads,
// several threads take interleaved rows of the same group and their sums are added in
// row-offset order through LDS.
template <typename T, int VW>
__global__ __launch_bounds__(kPoolThreads) void route_pool(const T* __restrict__ ks, int kv_dim,
                                                           const int32_t* __restrict__ cu,
                                                           int chunks,
                                                           float* __restrict__ partial) {
  __shared__ float red[kPoolThreads * VW];
  const int chunk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t s0 = cu[b];
  const int64_t len = (int64_t)cu[b + 1] - s0;
  const int64_t r0 = len * chunk / chunks, r1 = len * (chunk + 1) / chunks;
  const int groups = kv_dim / VW;  // column groups per row
  float* out = partial + ((int64_t)b * chunks + chunk) * kv_dim;
  float acc[VW];
  if (groups <= kPoolThreads) {
    const int rows_per_step = kPoolThreads / groups;
    const int grp = tid % groups, roff = tid / groups;
    const bool on = roff < rows_per_step;
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[e] = 0.f;
    if (on)
      for (int64_t r = r0 + roff; r < r1; r += rows_per_step)
        add_row<T, VW>(ks + (s0 + r) * kv_dim + (int64_t)grp * VW, acc);
#pragma unroll
    for (int e = 0; e < VW; ++e) red[tid * VW + e] = on ? acc[e] : 0.f;
    __syncthreads();
    if (tid < groups) {
#pragma unroll
      for (int e = 0; e < VW; ++e) acc[e] = 0.f;
      for (int ro = 0; ro < rows_per_step; ++ro)
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[e] += red[(ro * groups + tid) * VW + e];
#pragma unroll
      for (int e = 0; e < VW; ++e) out[(int64_t)tid * VW + e] = acc[e];
    }
  } else {
    for (int grp = tid; grp < groups; grp += kPoolThreads) {
#pragma unroll
      for (int e = 0; e < VW; ++e) acc[e] = 0.f;
      for (int64_t r = r0; r < r1; ++r)
        add_row<T, VW>(ks + (s0 + r) * kv_dim + (int64_t)grp * VW, acc);
#pragma unroll
      for (int e = 0; e < VW; ++e) out[(int64_t)grp * VW + e] = acc[e];
    }
  }
}

__device__ __forceinline__ float wave_sum(float x) {
  // butterfly over the 64 lanes; every lane ends with the same, order-fixed sum
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__global__ __launch_bounds__(kMlpThreads) void route_mlp(
    const float* __restrict__ partial, int chunks, const int32_t* __restrict__ cu, int kv_dim,
    const float* __restrict__ w1, const float* __restrict__ b1, int hidden,
    const float* __restrict__ w2, const float* __restrict__ b2, int n_heads,
    float* __restrict__ logits, uint8_t* __restrict__ route) {
  extern __shared__ float sm[];
  float* x = sm;               // [kv_dim]
  float* hv = sm + kv_dim;     // [hidden]
  const int b = blockIdx.x;
  const int len = cu[b + 1] - cu[b];
  const float inv_len = len > 0 ? 1.0f / (float)len : 0.0f;
  for (int c = threadIdx.x; c < kv_dim; c += kMlpThreads) {
    float s = 0.f;
    for (int ch = 0; ch < chunks; ++ch) s += partial[((int64_t)b * chunks + ch) * kv_dim + c];
    x[c] = len > 0 ? s * inv_len : 0.f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kMlpThreads / 64;
  for (int j = wave; j < hidden; j += nw) {
    float s = 0.f;
    for (int c = lane; c < kv_dim; c += 64) s += w1[(int64_t)j * kv_dim + c] * x[c];
    const float u = wave_sum(s) + b1[j];
    if (lane == 0) hv[j] = u / (1.0f + expf(-u));   // SiLU
  }
  __syncthreads();
  for (int h = wave; h < n_heads; h += nw) {
    float s = 0.f;
    for (int j = lane; j < hidden; j += 64) s += w2[(int64_t)h * hidden + j] * hv[j];
    const float z = wave_sum(s) + b2[h];
    if (lane == 0) {
      if (logits) logits[(int64_t)b * n_heads + h] = z;
      route[(int64_t)b * n_heads + h] = z > 0.f ? 1 : 0;
    }
  }
}

}  // namespace

int router_chunks(int32_t batch) {
  int c = 512 / (batch > 0 ? batch : 1);
  return c < 8 ? 8 : (c > 256 ? 256 : c);
}

hipError_t launch_route(const void* ks, int kdt, int kv_dim, const int32_t* cu, int batch,
                        const float* w1, const float* b1, int hidden, const float* w2,
                        const float* b2, int n_heads_q, float* logits, uint8_t* route,
                        float* partial, int chunks, hipStream_t stream) {
  dim3 grid(chunks, batch);
  if (kdt == 0) {
    if (kv_dim % 8 == 0)
      route_pool<__bf16, 8><<<grid, kPoolThreads, 0, stream>>>((const __bf16*)ks, kv_dim, cu,
                                                               chunks, partial);
    else
      route_pool<__bf16, 1><<<grid, kPoolThreads, 0, stream>>>((const __bf16*)ks, kv_dim, cu,
                                                               chunks, partial);
  } else {
    if (kv_dim % 4 == 0)
      route_pool<float, 4><<<grid, kPoolThreads, 0, stream>>>((const float*)ks, kv_dim, cu,
                                                              chunks, partial);
    else
      route_pool<float, 1><<<grid, kPoolThreads, 0, stream>>>((const float*)ks, kv_dim, cu,
                                                              chunks, partial);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(float) * ((size_t)kv_dim + (size_t)hidden);
  route_mlp<<<batch, kMlpThreads, lds, stream>>>(partial, chunks, cu, kv_dim, w1, b1, hidden, w2,
                                                 b2, n_heads_q, logits, route);
  return hipGetLastError();
}

}  // namespace ea
