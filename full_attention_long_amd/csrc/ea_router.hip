// ea_router.hip -- the Attention Router (Elastic Attention blog post, section 2.1: the
// router reads the current key hidden states, an MLP emits one routing signal per head,
// r = 0 full attention, r = 1 sparse attention; about 0.27M parameters per layer for an
// 8B model, section 2.2).
//
// Four short launches, all deterministic (fixed summation orders, no float atomics):
//   route_pool    grid (row chunks, column chunks, batch): every workgroup sums the key
//                 states of its rows for 16 column groups in fp32 and writes one partial
//                 row; a streaming read of the key states with 8 loads in flight per
//                 thread (HBM bound).
//   route_mean    adds the partial rows of each column in chunk order and divides by the
//                 length (an empty sequence pools to zero).
//   route_hidden  h = SiLU(W1 x + b1), eight hidden units per workgroup, wavefront dot
//                 products over the key features.
//   route_out     z = W2 h + b2, r = (z > 0).
#include "ea_device.h"
#include "ea_internal.h"

namespace ea {

namespace {

constexpr int kPoolThreads = 256;

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

template <typename T, int VW>
__device__ __forceinline__ void load_row(const T* p, u32x4* raw, T* vals) {
  if constexpr (VW * sizeof(T) == 16) {
    *raw = *(const u32x4*)p;
  } else {
#pragma unroll
    for (int e = 0; e < VW; ++e) vals[e] = p[e];
  }
}

constexpr int kGroupsPerBlock = 16;                          // column groups per workgroup
constexpr int kRowLanes = kPoolThreads / kGroupsPerBlock;    // rows summed side by side
constexpr int kUnroll = 8;                                   // loads in flight per thread

// Sums rows [r0, r1) of sequence blockIdx.z for the VW-wide column groups
// blockIdx.y*16 .. +15.  Thread (row lane tr, group tg) adds rows r0+tr, r0+tr+16, ...;
// the 16 row-lane sums of a group are then added in row-lane order.
template <typename T, int VW>
__global__ __launch_bounds__(kPoolThreads) void route_pool(const T* __restrict__ ks, int kv_dim,
                                                           const int32_t* __restrict__ cu,
                                                           int row_chunks,
                                                           float* __restrict__ partial) {
  __shared__ float red[kRowLanes][kGroupsPerBlock * VW + 1];
  const int rc = blockIdx.x, b = blockIdx.z, tid = threadIdx.x;
  const int tg = tid % kGroupsPerBlock, tr = tid / kGroupsPerBlock;
  const int groups = kv_dim / VW;
  const int grp = blockIdx.y * kGroupsPerBlock + tg;
  const int64_t s0 = cu[b];
  const int64_t len = (int64_t)cu[b + 1] - s0;
  const int64_t r0 = len * rc / row_chunks, r1 = len * (rc + 1) / row_chunks;
  float acc[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = 0.f;
  if (grp < groups) {
    const T* base = ks + s0 * kv_dim + (int64_t)grp * VW;
    int64_t r = r0 + tr;
    for (; r + (kUnroll - 1) * kRowLanes < r1; r += kUnroll * kRowLanes) {
      u32x4 raw[kUnroll];
      T vals[kUnroll][VW];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        load_row<T, VW>(base + (r + u * kRowLanes) * kv_dim, &raw[u], vals[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const T* v = (VW * sizeof(T) == 16) ? (const T*)&raw[u] : vals[u];
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[e] += to_f32(v[e]);
      }
    }
    for (; r < r1; r += kRowLanes) {
      u32x4 raw;
      T vals[VW];
      load_row<T, VW>(base + r * kv_dim, &raw, vals);
      const T* v = (VW * sizeof(T) == 16) ? (const T*)&raw : vals;
#pragma unroll
      for (int e = 0; e < VW; ++e) acc[e] += to_f32(v[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < VW; ++e) red[tr][tg * VW + e] = acc[e];
  __syncthreads();
  const int col_base = blockIdx.y * kGroupsPerBlock * VW;
  for (int c = tid; c < kGroupsPerBlock * VW; c += kPoolThreads) {
    if (col_base + c >= kv_dim) continue;
    float s = 0.f;
    for (int t = 0; t < kRowLanes; ++t) s += red[t][c];
    partial[((int64_t)b * row_chunks + rc) * kv_dim + col_base + c] = s;
  }
}

// x[b, c] = (sum over row chunks of partial[b, chunk, c]) / len_b; 16 columns x 16
// chunk lanes per workgroup, the lane sums added in lane order.
__global__ __launch_bounds__(256) void route_mean(const float* __restrict__ partial,
                                                  int row_chunks, const int32_t* __restrict__ cu,
                                                  int kv_dim, float* __restrict__ x) {
  __shared__ float red[16][17];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int col = blockIdx.x * 16 + tid % 16, lane = tid / 16;
  float s = 0.f;
  if (col < kv_dim) {
    const float* p = partial + (int64_t)b * row_chunks * kv_dim + col;
#pragma unroll 8
    for (int ch = lane; ch < row_chunks; ch += 16) s += p[(int64_t)ch * kv_dim];
  }
  red[lane][tid % 16] = s;
  __syncthreads();
  if (tid < 16 && col < kv_dim) {
    float t = 0.f;
    for (int l = 0; l < 16; ++l) t += red[l][tid];
    const int len = cu[b + 1] - cu[b];
    x[(int64_t)b * kv_dim + col] = len > 0 ? t / (float)len : 0.f;
  }
}

__device__ __forceinline__ float wave_sum(float x) {
  // butterfly over the 64 lanes; every lane ends with the same, order-fixed sum
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// One wavefront per output: the lanes stride over the inputs with every load of a lane
// issued before the first add (one memory round trip per output), then a butterfly sum.
template <int kPerLane>
__device__ __forceinline__ float wave_dot(const float* __restrict__ w, const float* __restrict__ x,
                                          int n) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
  for (int base = 0; base < n; base += 64 * kPerLane) {
    float wv[kPerLane], xv[kPerLane];
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const int c = base + u * 64 + lane;
      wv[u] = c < n ? w[c] : 0.f;
      xv[u] = c < n ? x[c] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) s += wv[u] * xv[u];
  }
  return wave_sum(s);
}

constexpr int kWavesPerBlock = 4;

// hv[b, j] = SiLU(W1[j, :] . x[b, :] + b1[j]); one wavefront per hidden unit.
__global__ __launch_bounds__(256) void route_hidden(const float* __restrict__ x, int kv_dim,
                                                    const float* __restrict__ w1,
                                                    const float* __restrict__ b1, int hidden,
                                                    float* __restrict__ hv) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (j >= hidden) return;
  const float u = wave_dot<16>(w1 + (int64_t)j * kv_dim, x + (int64_t)b * kv_dim, kv_dim) + b1[j];
  if ((threadIdx.x & 63) == 0) hv[(int64_t)b * hidden + j] = u / (1.0f + expf(-u));  // SiLU
}

// z[b, h] = W2[h, :] . hv[b, :] + b2[h]; route = z > 0 (z == 0 routes to full); one
// wavefront per head.
__global__ __launch_bounds__(256) void route_out(const float* __restrict__ hv, int hidden,
                                                 const float* __restrict__ w2,
                                                 const float* __restrict__ b2, int n_heads,
                                                 float* __restrict__ logits,
                                                 uint8_t* __restrict__ route) {
  const int b = blockIdx.y;
  const int h = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (h >= n_heads) return;
  const float z = wave_dot<4>(w2 + (int64_t)h * hidden, hv + (int64_t)b * hidden, hidden) + b2[h];
  if ((threadIdx.x & 63) == 0) {
    if (logits) logits[(int64_t)b * n_heads + h] = z;
    route[(int64_t)b * n_heads + h] = z > 0.f ? 1 : 0;
  }
}

}  // namespace

int router_chunks(int32_t batch) {
  // about 1024 pooling workgroups in all (8 column chunks of a 1024-wide bf16 row)
  int c = 128 / (batch > 0 ? batch : 1);
  return c < 4 ? 4 : c;
}

hipError_t launch_route(const void* ks, int kdt, int kv_dim, const int32_t* cu, int batch,
                        const float* w1, const float* b1, int hidden, const float* w2,
                        const float* b2, int n_heads_q, float* logits, uint8_t* route,
                        float* partial, int chunks, float* x, float* hv, hipStream_t stream) {
  const bool vec = kdt == 0 ? (kv_dim % 8 == 0) : (kv_dim % 4 == 0);
  const int vw = vec ? (kdt == 0 ? 8 : 4) : 1;
  const int groups = kv_dim / vw;
  dim3 grid(chunks, (groups + kGroupsPerBlock - 1) / kGroupsPerBlock, batch);
  if (kdt == 0) {
    if (vec)
      route_pool<__bf16, 8><<<grid, kPoolThreads, 0, stream>>>((const __bf16*)ks, kv_dim, cu,
                                                               chunks, partial);
    else
      route_pool<__bf16, 1><<<grid, kPoolThreads, 0, stream>>>((const __bf16*)ks, kv_dim, cu,
                                                               chunks, partial);
  } else {
    if (vec)
      route_pool<float, 4><<<grid, kPoolThreads, 0, stream>>>((const float*)ks, kv_dim, cu,
                                                              chunks, partial);
    else
      route_pool<float, 1><<<grid, kPoolThreads, 0, stream>>>((const float*)ks, kv_dim, cu,
                                                              chunks, partial);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  route_mean<<<dim3((kv_dim + 15) / 16, batch), 256, 0, stream>>>(partial, chunks, cu, kv_dim, x);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  route_hidden<<<dim3((hidden + kWavesPerBlock - 1) / kWavesPerBlock, batch), 256, 0, stream>>>(
      x, kv_dim, w1, b1, hidden, hv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  route_out<<<dim3((n_heads_q + kWavesPerBlock - 1) / kWavesPerBlock, batch), 256, 0, stream>>>(
      hv, hidden, w2, b2, n_heads_q, logits, route);
  return hipGetLastError();
}

}  // namespace ea
