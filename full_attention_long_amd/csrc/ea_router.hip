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
// The pre-activation u goes to u_out as well when that is given (the backward needs it).
__global__ __launch_bounds__(256) void route_hidden(const float* __restrict__ x, int kv_dim,
                                                    const float* __restrict__ w1,
                                                    const float* __restrict__ b1, int hidden,
                                                    float* __restrict__ hv,
                                                    float* __restrict__ u_out) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (j >= hidden) return;
  const float u = wave_dot<16>(w1 + (int64_t)j * kv_dim, x + (int64_t)b * kv_dim, kv_dim) + b1[j];
  if ((threadIdx.x & 63) == 0) {
    hv[(int64_t)b * hidden + j] = u / (1.0f + expf(-u));  // SiLU
    if (u_out) u_out[(int64_t)b * hidden + j] = u;
  }
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

// ---------------------------------------------------------------------------------------
// Backward of the router through its straight-through decision (blog post section 2.1,
// "training trick": a Gumbel-Softmax relaxation with a straight-through estimator keeps the
// 0/1 decision trainable).  The forward output of head h is r O_sparse + (1 - r) O_full with
// the hard r; the backward takes the relaxed r_soft = sigmoid((z + g) / tau), so
//   dr[b, h] = sum over the sequence's rows t of <dO[t, h], O_sparse[t, h] - O_full[t, h]>,
//   dz = dr r_soft (1 - r_soft) / tau,
// then the MLP and the mean pool backward (chain rule, SiLU'(u) = s + u s (1 - s)).
// Launches, all in fixed summation orders:
//   route_dr_partial  grid (row chunks, column chunks, batch): each thread owns 8 adjacent
//                     columns of the [Hq * D] row and adds dO * (Os - Of) over its rows; the
//                     columns of one head are then added in lane order -> partial[b][chunk][h]
//                     (HBM bound: three streamed reads of the outputs).
//   route_dz          one wavefront per (b, h): dr = sum of the chunk partials, z = W2 h + b2
//                     again, dz.
//   route_bwd_hidden  du[b, j] = (sum_h dz[b, h] W2[h, j]) SiLU'(u[b, j]).
//   route_bwd_w2      dW2[h, j] = sum_b dz[b, h] hs[b, j];  db2[h] = sum_b dz[b, h].
//   route_bwd_w1      dW1[j, c] = sum_b du[b, j] x[b, c];  db1[j] = sum_b du[b, j].
//   route_bwd_x       dx[b, c] = sum_j du[b, j] W1[j, c] (hidden units split in four).
//   route_bwd_spread  dkey_states[t, c] = dx[b, c] / n_b for the n_b rows t of sequence b.

constexpr int kDrCols = 8;  // columns per thread in route_dr_partial

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 raw = *(const u32x4*)p;
    const T* v = (const T*)&raw;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
  } else {
    const float4 a = *(const float4*)p, c = *(const float4*)(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = c.x; out[5] = c.y; out[6] = c.z; out[7] = c.w;
  }
}

// Rows [r0, r1) of sequence blockIdx.z, columns blockIdx.x' * 2048 + 8 * tid .. + 7 of the
// [n_heads * head_dim] rows; head_dim is a multiple of 8 and divides 2048 or equals it.
template <typename T>
__global__ __launch_bounds__(256) void route_dr_partial(const T* __restrict__ of,
                                                        const T* __restrict__ os,
                                                        const T* __restrict__ go,
                                                        const int32_t* __restrict__ cu,
                                                        int n_heads, int head_dim, int row_chunks,
                                                        float* __restrict__ partial) {
  const int rc = blockIdx.x, b = blockIdx.z, tid = threadIdx.x;
  const int width = n_heads * head_dim;
  const int col = blockIdx.y * 256 * kDrCols + tid * kDrCols;
  const int64_t s0 = cu[b];
  const int64_t len = (int64_t)cu[b + 1] - s0;
  const int64_t r0 = len * rc / row_chunks, r1 = len * (rc + 1) / row_chunks;
  float acc = 0.f;
  if (col < width) {
    int64_t r = r0;
    for (; r + 3 < r1; r += 4) {
      float f[4][8], s[4][8], g[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t at = (s0 + r + u) * width + col;
        load8(of + at, f[u]);
        load8(os + at, s[u]);
        load8(go + at, g[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(g[u][e], s[u][e] - f[u][e], acc);
    }
    for (; r < r1; ++r) {
      float f[8], s[8], g[8];
      const int64_t at = (s0 + r) * width + col;
      load8(of + at, f);
      load8(os + at, s);
      load8(go + at, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(g[e], s[e] - f[e], acc);
    }
  }
  // the head_dim / 8 lanes of one head are adjacent (head_dim / 8 <= 64 divides 64)
  const int per_head = head_dim / kDrCols;
  for (int m = 1; m < per_head; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (col < width && (tid % per_head) == 0)
    partial[((int64_t)b * row_chunks + rc) * n_heads + col / head_dim] = acc;
}

// dr, dz for (b, h) = (blockIdx.y, wavefront of blockIdx.x)
__global__ __launch_bounds__(256) void route_dz(const float* __restrict__ partial, int row_chunks,
                                                const float* __restrict__ hs, int hidden,
                                                const float* __restrict__ w2,
                                                const float* __restrict__ b2, int n_heads,
                                                const float* __restrict__ noise, float tau,
                                                float* __restrict__ dr_out,
                                                float* __restrict__ dz_out) {
  const int b = blockIdx.y, lane = threadIdx.x & 63;
  const int h = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (h >= n_heads) return;
  float s = 0.f;
  for (int c = lane; c < row_chunks; c += 64) s += partial[((int64_t)b * row_chunks + c) * n_heads + h];
  const float dr = wave_sum(s);
  const float z = wave_dot<4>(w2 + (int64_t)h * hidden, hs + (int64_t)b * hidden, hidden) + b2[h];
  if (lane == 0) {
    const float g = noise ? noise[(int64_t)b * n_heads + h] : 0.f;
    const float rs = 1.0f / (1.0f + expf(-(z + g) / tau));
    if (dr_out) dr_out[(int64_t)b * n_heads + h] = dr;
    dz_out[(int64_t)b * n_heads + h] = dr * rs * (1.0f - rs) / tau;
  }
}

// du[b, j]: thread j of grid (ceil(hidden / 256), batch)
__global__ __launch_bounds__(256) void route_bwd_hidden(const float* __restrict__ dz, int n_heads,
                                                        const float* __restrict__ w2,
                                                        const float* __restrict__ u, int hidden,
                                                        float* __restrict__ du) {
  const int b = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= hidden) return;
  float dh = 0.f;
  for (int h = 0; h < n_heads; ++h)
    dh = __builtin_fmaf(dz[(int64_t)b * n_heads + h], w2[(int64_t)h * hidden + j], dh);
  const float uu = u[(int64_t)b * hidden + j];
  const float sg = 1.0f / (1.0f + expf(-uu));
  du[(int64_t)b * hidden + j] = dh * (sg + uu * sg * (1.0f - sg));
}

// dW2[h, j] (thread per j, blockIdx.y = h) and db2[h]
__global__ __launch_bounds__(256) void route_bwd_w2(const float* __restrict__ dz,
                                                    const float* __restrict__ hs, int batch,
                                                    int hidden, int n_heads,
                                                    float* __restrict__ dw2,
                                                    float* __restrict__ db2) {
  const int h = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j < hidden) {
    float s = 0.f;
    for (int b = 0; b < batch; ++b)
      s = __builtin_fmaf(dz[(int64_t)b * n_heads + h], hs[(int64_t)b * hidden + j], s);
    dw2[(int64_t)h * hidden + j] = s;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    float s = 0.f;
    for (int b = 0; b < batch; ++b) s += dz[(int64_t)b * n_heads + h];
    db2[h] = s;
  }
}

// dW1[j, c] (thread per c, blockIdx.y = j) and db1[j]
__global__ __launch_bounds__(256) void route_bwd_w1(const float* __restrict__ du,
                                                    const float* __restrict__ x, int batch,
                                                    int kv_dim, int hidden,
                                                    float* __restrict__ dw1,
                                                    float* __restrict__ db1) {
  const int j = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  if (c < kv_dim) {
    float s = 0.f;
    for (int b = 0; b < batch; ++b)
      s = __builtin_fmaf(du[(int64_t)b * hidden + j], x[(int64_t)b * kv_dim + c], s);
    dw1[(int64_t)j * kv_dim + c] = s;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    float s = 0.f;
    for (int b = 0; b < batch; ++b) s += du[(int64_t)b * hidden + j];
    db1[j] = s;
  }
}

// dx[b, c] (blockIdx.y = b): 64 columns per workgroup, its four wavefronts each summing a
// quarter of the hidden units; the quarters are added in order (fixed, deterministic)
__global__ __launch_bounds__(256) void route_bwd_x(const float* __restrict__ du,
                                                   const float* __restrict__ w1, int kv_dim,
                                                   int hidden, float* __restrict__ dx) {
  __shared__ float part[4][64];
  const int b = blockIdx.y, lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int j0 = hidden * q / 4, j1 = hidden * (q + 1) / 4;
  float s = 0.f;
  if (c < kv_dim)
    for (int j = j0; j < j1; ++j)
      s = __builtin_fmaf(du[(int64_t)b * hidden + j], w1[(int64_t)j * kv_dim + c], s);
  part[q][lane] = s;
  __syncthreads();
  if (q == 0 && c < kv_dim)
    dx[(int64_t)b * kv_dim + c] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

// dkey_states rows of sequence blockIdx.z, chunk blockIdx.x, columns 4 * thread of
// column block blockIdx.y (kv_dim % 4 == 0: float4 stores)
__global__ __launch_bounds__(256) void route_bwd_spread(const float* __restrict__ dx,
                                                        const int32_t* __restrict__ cu,
                                                        int kv_dim, int row_chunks,
                                                        float* __restrict__ dks) {
  const int rc = blockIdx.x, b = blockIdx.z;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= kv_dim) return;
  const int64_t s0 = cu[b];
  const int64_t len = (int64_t)cu[b + 1] - s0;
  if (len <= 0) return;
  const int64_t r0 = len * rc / row_chunks, r1 = len * (rc + 1) / row_chunks;
  const float inv = 1.0f / (float)len;
  const float* x = dx + (int64_t)b * kv_dim + c;
  const float4 v = make_float4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
  for (int64_t r = r0; r < r1; ++r) *(float4*)(dks + (s0 + r) * kv_dim + c) = v;
}

}  // namespace

int route_bwd_chunks(int32_t batch, int32_t width) {
  // about 2048 workgroups for the dr reduction
  const int colblocks = (width + 256 * kDrCols - 1) / (256 * kDrCols);
  int c = 2048 / ((batch > 0 ? batch : 1) * (colblocks > 0 ? colblocks : 1));
  return c < 4 ? 4 : c;
}

hipError_t launch_route_backward(const RouteBwdArgs& a, hipStream_t stream) {
  // mean pool and the hidden layer again (the same kernels and order as the forward)
  const bool vec = a.kdt == 0 ? (a.kv_dim % 8 == 0) : (a.kv_dim % 4 == 0);
  const int vw = vec ? (a.kdt == 0 ? 8 : 4) : 1;
  const int groups = a.kv_dim / vw;
  dim3 grid(a.pool_chunks, (groups + kGroupsPerBlock - 1) / kGroupsPerBlock, a.batch);
  if (a.kdt == 0) {
    if (vec)
      route_pool<__bf16, 8><<<grid, kPoolThreads, 0, stream>>>((const __bf16*)a.key_states,
                                                               a.kv_dim, a.cu, a.pool_chunks,
                                                               a.pool_partial);
    else
      route_pool<__bf16, 1><<<grid, kPoolThreads, 0, stream>>>((const __bf16*)a.key_states,
                                                               a.kv_dim, a.cu, a.pool_chunks,
                                                               a.pool_partial);
  } else {
    if (vec)
      route_pool<float, 4><<<grid, kPoolThreads, 0, stream>>>((const float*)a.key_states,
                                                              a.kv_dim, a.cu, a.pool_chunks,
                                                              a.pool_partial);
    else
      route_pool<float, 1><<<grid, kPoolThreads, 0, stream>>>((const float*)a.key_states,
                                                              a.kv_dim, a.cu, a.pool_chunks,
                                                              a.pool_partial);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  route_mean<<<dim3((a.kv_dim + 15) / 16, a.batch), 256, 0, stream>>>(a.pool_partial,
                                                                      a.pool_chunks, a.cu,
                                                                      a.kv_dim, a.x);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  route_hidden<<<dim3((a.hidden + kWavesPerBlock - 1) / kWavesPerBlock, a.batch), 256, 0,
                 stream>>>(a.x, a.kv_dim, a.w1, a.b1, a.hidden, a.hs, a.u);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int width = a.n_heads_q * a.head_dim;
  const dim3 gdr(a.dr_chunks, (width + 256 * kDrCols - 1) / (256 * kDrCols), a.batch);
  if (a.odt == 0)
    route_dr_partial<__bf16><<<gdr, 256, 0, stream>>>(
        (const __bf16*)a.o_full, (const __bf16*)a.o_sparse, (const __bf16*)a.dout, a.cu,
        a.n_heads_q, a.head_dim, a.dr_chunks, a.dr_partial);
  else
    route_dr_partial<float><<<gdr, 256, 0, stream>>>(
        (const float*)a.o_full, (const float*)a.o_sparse, (const float*)a.dout, a.cu,
        a.n_heads_q, a.head_dim, a.dr_chunks, a.dr_partial);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  route_dz<<<dim3((a.n_heads_q + kWavesPerBlock - 1) / kWavesPerBlock, a.batch), 256, 0,
             stream>>>(a.dr_partial, a.dr_chunks, a.hs, a.hidden, a.w2, a.b2, a.n_heads_q,
                       a.noise, a.tau, a.dr, a.dz);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  route_bwd_hidden<<<dim3((a.hidden + 255) / 256, a.batch), 256, 0, stream>>>(
      a.dz, a.n_heads_q, a.w2, a.u, a.hidden, a.du);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  route_bwd_w2<<<dim3((a.hidden + 255) / 256, a.n_heads_q), 256, 0, stream>>>(
      a.dz, a.hs, a.batch, a.hidden, a.n_heads_q, a.dw2, a.db2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  route_bwd_w1<<<dim3((a.kv_dim + 255) / 256, a.hidden), 256, 0, stream>>>(
      a.du, a.x, a.batch, a.kv_dim, a.hidden, a.dw1, a.db1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!a.dkey_states) return hipSuccess;
  route_bwd_x<<<dim3((a.kv_dim + 63) / 64, a.batch), 256, 0, stream>>>(a.du, a.w1, a.kv_dim,
                                                                       a.hidden, a.dx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  route_bwd_spread<<<dim3(a.dr_chunks, (a.kv_dim / 4 + 255) / 256, a.batch), 256, 0, stream>>>(
      a.dx, a.cu, a.kv_dim, a.dr_chunks, a.dkey_states);
  return hipGetLastError();
}

namespace {
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
      x, kv_dim, w1, b1, hidden, hv, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  route_out<<<dim3((n_heads_q + kWavesPerBlock - 1) / kWavesPerBlock, batch), 256, 0, stream>>>(
      hv, hidden, w2, b2, n_heads_q, logits, route);
  return hipGetLastError();
}

}  // namespace ea
