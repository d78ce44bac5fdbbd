// Dense decode attention over all t keys: the baseline the sparse path is
// measured against (page "Near-Oracle KV Selection via Pre-hoc Sparsity for
// Long-Context Inference", Table IV: attention-operator latency against the
// dense FlashAttention kernel; the Abstract's speedup over the dense
// baseline).
//
// Split over keys, as flash decoding does: one 256-thread workgroup per
// (b, h_kv, chunk of kDecodeRows keys). The workgroup scores its chunk's K
// rows against the G query heads of the group exactly as the scan does (16-byte
// lane loads, fp32 dot products, DPP row sums), keeps the scores in LDS, turns
// them into chunk-local softmax weights per head, then streams the chunk's V
// rows once for all G heads and leaves a (max, sum, o[d]) partial per head.
// The split-decode merge combines the partials exactly. K and V are each read
// once (non-temporally); nothing else of size reaches HBM.
#include "prhs_device.hpp"
#include "prhs_launch.hpp"

namespace prhs {
namespace {

constexpr int kDenseThreads = 256;

template <typename T, int D, int G>
__global__ __launch_bounds__(kDenseThreads) void dense_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int Hq, int Hkv,
    int t, long long sb, long long sh, long long st, float scale, float* __restrict__ part,
    int nsplit, int g_off) {
  constexpr int NW = kDenseThreads / kWave;
  constexpr int ROWS = kDecodeRows;
  constexpr int E = Elem<T>::kPer16B;
  constexpr int LPR = D / E;
  constexpr int RPW = kWave / LPR;
  constexpr int RW = ROWS / NW;                    // rows per wave
  constexpr int U = RW / RPW < 16 ? RW / RPW : 16;  // K loads in flight per lane
  constexpr int IT = RW / (U * RPW);
  constexpr int UV = U < 8 ? U : 8;                  // V loads in flight per lane
  constexpr int ITV = RW / (UV * RPW);
  static_assert(G <= LPR, "one lane per head in a row group");
  static_assert(RW % (U * RPW) == 0 && RW % (UV * RPW) == 0, "chunk tiling");
  static_assert(ROWS == kDenseThreads, "the weights map one row per thread");

  constexpr int PITCH = ROWS + (RPW > 4 ? RPW : 4);  // distinct banks for the G heads' writes
  __shared__ float sc[G][PITCH];
  __shared__ float smax[G][NW];
  __shared__ float ssum[G][NW];
  __shared__ __align__(16) float so[G][NW][D];

  const int chunk = blockIdx.x;
  const int unit = blockIdx.y;
  const int b = unit / Hkv;
  const int g = unit - b * Hkv;
  const int h0 = g * (Hq / Hkv) + g_off;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int c = lane % LPR;
  const int rr = lane / LPR;
  const int beg = chunk * ROWS;

  uint4 qv[G];
#pragma unroll
  for (int j = 0; j < G; ++j) qv[j] = load16(q + ((size_t)(b * Hq + h0 + j) * D + c * E));

  const size_t kv_off = (size_t)b * sb + (size_t)g * sh;
  const size_t row_bytes = (size_t)st * sizeof(T);
  const char* kbase = reinterpret_cast<const char*>(k + kv_off) + c * 16;
  const char* vbase = reinterpret_cast<const char*>(v + kv_off) + c * 16;

  // scores of the chunk for every head of the group (-inf past t)
#pragma unroll 1
  for (int it = 0; it < IT; ++it) {
    uint4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = beg + w * RW + (it * U + u) * RPW + rr;
      kv[u] = r < t ? load16_stream(kbase + (size_t)r * row_bytes) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = w * RW + (it * U + u) * RPW + rr;
      float acc[G];
#pragma unroll
      for (int j = 0; j < G; ++j) acc[j] = group_sum<LPR>(dot16(kv[u], qv[j], 0.f, T()));
      float val = acc[0];
#pragma unroll
      for (int j = 1; j < G; ++j) val = (c == j) ? acc[j] : val;
      if (c < G) sc[c][i] = beg + i < t ? val * scale : -INFINITY;
    }
  }

  // the first batch of V rows goes out before the weights are formed
  uint4 vv[UV];
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int r = beg + w * RW + u * RPW + rr;
    vv[u] = r < t ? load16_stream(vbase + (size_t)r * row_bytes) : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  // chunk maximum and softmax weights per head (thread tid owns row tid)
  float mj[G], lj[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float m = wave_max(sc[j][tid]);
    if (lane == 0) smax[j][w] = m;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float m = smax[j][0];
#pragma unroll
    for (int u = 1; u < NW; ++u) m = fmaxf(m, smax[j][u]);
    mj[j] = m;
    const float p = m == -INFINITY ? 0.f : __expf(sc[j][tid] - m);
    sc[j][tid] = p;
    const float l = wave_sum(p);
    if (lane == 0) ssum[j][w] = l;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < NW; ++u) l += ssum[j][u];
    lj[j] = l;
  }

  // weighted V rows, all heads of the group at once
  float acc[G][E];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[j][e] = 0.f;
#pragma unroll 1
  for (int it = 0; it < ITV; ++it) {
    if (it > 0) {
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        const int r = beg + w * RW + (it * UV + u) * RPW + rr;
        vv[u] = r < t ? load16_stream(vbase + (size_t)r * row_bytes) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int i = w * RW + (it * UV + u) * RPW + rr;
#pragma unroll
      for (int j = 0; j < G; ++j) axpy16(sc[j][i], vv[u], acc[j], T());
    }
  }
  // sum the RPW row slots of the wave, then the waves through LDS
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
#pragma unroll
      for (int o = LPR; o < kWave; o <<= 1) acc[j][e] += __shfl_xor(acc[j][e], o);
    }
    if (rr == 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) so[j][w][c * E + e] = acc[j][e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    // written through the L2, like the scan's outputs: they land inside the
    // K and V read streams
    float* dst = part + ((size_t)(b * Hq + h0 + j) * nsplit + chunk) * (D + 2);
    constexpr uint32_t kBytes = (D + 2) * 4;
    for (int col = tid; col < D; col += kDenseThreads) {
      float s = 0.f;
#pragma unroll
      for (int u = 0; u < NW; ++u) s += so[j][u][col];
      store_through(dst, kBytes, (uint32_t)col * 4u, __float_as_uint(s));
    }
    if (tid == 0) {
      store_through(dst, kBytes, (uint32_t)D * 4u, __float_as_uint(mj[j]));
      store_through(dst, kBytes, (uint32_t)(D + 1) * 4u, __float_as_uint(lj[j]));
    }
  }
}

template <typename T, int D, int G>
void launch_dense_split(const prhs_dims& d, const void* q, const void* k, const void* v,
                        float* part, int nsplit, int g_off, hipStream_t stream) {
  dim3 grid(nsplit, d.batch * d.n_kv_heads);
  const float scale = (float)(1.0 / __builtin_sqrt((double)d.head_dim));
  hipLaunchKernelGGL((dense_split_kernel<T, D, G>), grid, dim3(kDenseThreads), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     d.n_q_heads, d.n_kv_heads, d.ctx_len, (long long)d.kv_stride_b,
                     (long long)d.kv_stride_h, (long long)d.kv_stride_t, scale, part, nsplit, g_off);
}

template <typename T, int D>
void launch_dense_group(const prhs_dims& d, const void* q, const void* k, const void* v,
                        float* part, int nsplit, hipStream_t stream) {
  // Power-of-two sub-groups of the query heads that share one KV head, up to
  // one lane per head of a row group (16 heads at fp16 d = 128): each
  // sub-group reads K and V once.
  constexpr int kMaxSub = D / Elem<T>::kPer16B < 16 ? D / Elem<T>::kPer16B : 16;
  const int G = d.n_q_heads / d.n_kv_heads;
  int off = 0;
  while (off < G) {
    int sub = 1;
    while (sub * 2 <= G - off && sub * 2 <= kMaxSub) sub *= 2;
    switch (sub) {
      case 16:
        if constexpr (kMaxSub >= 16) launch_dense_split<T, D, 16>(d, q, k, v, part, nsplit, off, stream);
        break;
      case 8: launch_dense_split<T, D, 8>(d, q, k, v, part, nsplit, off, stream); break;
      case 4: launch_dense_split<T, D, 4>(d, q, k, v, part, nsplit, off, stream); break;
      case 2: launch_dense_split<T, D, 2>(d, q, k, v, part, nsplit, off, stream); break;
      default: launch_dense_split<T, D, 1>(d, q, k, v, part, nsplit, off, stream); break;
    }
    off += sub;
  }
}

}  // namespace

hipError_t launch_dense(const prhs_dims& d, const void* q, const void* k, const void* v,
                        float* out, float* lse, void* ws, hipStream_t stream) {
  const int nsplit = decode_nsplit(d.ctx_len);
  float* part = static_cast<float*>(ws);
  if (d.dtype == PRHS_F16) {
    if (d.head_dim == 128) launch_dense_group<__half, 128>(d, q, k, v, part, nsplit, stream);
    else launch_dense_group<__half, 64>(d, q, k, v, part, nsplit, stream);
  } else {
    if (d.head_dim == 128) launch_dense_group<float, 128>(d, q, k, v, part, nsplit, stream);
    else launch_dense_group<float, 64>(d, q, k, v, part, nsplit, stream);
  }
  return launch_merge(d, part, nsplit, out, lse, nullptr, nullptr, nullptr, stream);
}

}  // namespace prhs
