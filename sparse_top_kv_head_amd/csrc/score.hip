// K-scan scoring kernel: s[b,h,i] = q[b,h,:] . K[b,h/G,i,:] / sqrt(d) for every
// cached key, plus per-chunk (max, sum-of-exp) partials of the dense softmax
// (page "Near-Oracle KV Selection via Pre-hoc Sparsity for Long-Context
// Inference", Table I: query q, keys K, per-head dimension d, attention weight A).
//
// HBM-bound GEMV: every K row is read exactly once, by one wave, with 16-byte
// loads, and is scored against all G query heads of its group. Layout on the
// wave: LPR lanes cover one row (LPR = 16 for d=128 fp16), so one load
// instruction covers RPW = 64/LPR rows. Scores are staged in LDS and written
// back coalesced; the chunk's softmax partials come from the staged values.
//
// Two kernels. For fp16 rows of d = 128 (every LLaMA/Mistral-shaped layer),
// score_scan_mfma_kernel: each wave passes its loaded rows, 16 at a time,
// through a 4 KiB LDS tile into the operand layout of v_mfma_f32_16x16x32_f16
// and scores them on the matrix cores. Otherwise (fp32 rows, d = 64, or a
// KV head whose rows span 4 GiB or more)
// score_scan_kernel: the LPR partial dot products of a row are summed with
// DPP row operations.
#include "prhs_device.hpp"
#include "prhs_launch.hpp"

namespace prhs {
namespace {

constexpr int kScoreThreads = 256;

// The G partial dot products of a 16-lane row group (lane c holds its slice's
// share of every head) reduced and scattered: exchanges between lanes c and
// 15 - c, then c and 7 - c, then c and c ^ 2, each halving the heads a lane
// carries, until every lane holds one head's sum over the lanes it met; the
// lanes of that head then finish with plain exchanges. Every lane ends with
// the full sum of head rs16_head(c) = c / (16 / G). 5 DPP additions for
// G = 4 and 8 for G = 8, against 4 G for separate sums.
template <int G>
__device__ __forceinline__ int rs16_head(int c) {
  return G == 1 ? 0 : c / (16 / G);
}

// The query head in acc[j] of lane c. Each exchange keeps the first half of
// a lane's heads and sends the second half, with no selects, when the heads
// run in this order: XOR-ing the group index of c with
// tau = (0, 1, 3, 2, 7, 6, 4, 5) pairs head j of one lane with head j + G/2 of
// its 15 - c partner (group index ^ (G - 1)), head j with head j + G/4 of its
// 7 - c partner (^ (G/2 - 1)), and head 0 with head 1 of its c ^ 2 partner
// (^ 1).
template <int G>
__device__ __forceinline__ int rs16_qorder(int j, int c) {
  constexpr int kTau[8] = {0, 1, 3, 2, 7, 6, 4, 5};
  return G == 1 ? 0 : (rs16_head<G>(c) ^ kTau[j]);
}

template <int G>
__device__ __forceinline__ float rs16(const float (&acc)[G]) {
  if constexpr (G == 1) {
    return group_sum<16>(acc[0]);
  } else {
    constexpr int H1 = G / 2;
    float k1[H1];
#pragma unroll
    for (int i = 0; i < H1; ++i) k1[i] = acc[i] + dpp<kDppRowMirror>(acc[H1 + i]);
    float x;
    if constexpr (G == 2) {
      x = k1[0];
      x += dpp<kDppRowHalfMirror>(x);
      x += dpp<kDppXor2>(x);
    } else {
      constexpr int H2 = H1 / 2;
      float k2[H2];
#pragma unroll
      for (int i = 0; i < H2; ++i) k2[i] = k1[i] + dpp<kDppRowHalfMirror>(k1[H2 + i]);
      x = k2[0];
      if constexpr (G == 4) x += dpp<kDppXor2>(x);
      else x += dpp<kDppXor2>(k2[1]);
    }
    x += dpp<kDppXor1>(x);
    return x;
  }
}
// dot16 from a zero accumulator. For fp16 the first pair goes through the
// three-operand v_dot2_f32_f16 with an inline-constant 0, which the compiler
// would otherwise form as a register clear plus the two-operand v_dot2c.
__device__ __forceinline__ float dot16_zero(const uint4 a, const uint4 b, float /*tag*/) {
  return dot16(a, b, 0.f, 0.f);
}

__device__ __forceinline__ float dot16_zero(const uint4 a, const uint4 b, __half /*tag*/) {
  const half2_t* x = reinterpret_cast<const half2_t*>(&a);
  const half2_t* y = reinterpret_cast<const half2_t*>(&b);
  float acc;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(acc) : "v"(x[0]), "v"(y[0]));
  acc = __builtin_amdgcn_fdot2(x[1], y[1], acc, false);
  acc = __builtin_amdgcn_fdot2(x[2], y[2], acc, false);
  acc = __builtin_amdgcn_fdot2(x[3], y[3], acc, false);
  return acc;
}

constexpr int kScoreLoads = 16;  // 16-byte loads in flight per lane

// The chunk's outputs from the staged scores sc[j][0:CHUNK) of its G heads,
// all written through the L2 (store_through):
// the scores themselves (not for heads with a finite theta under
// skip_hinted), the keys >= theta as (score bits, index) candidates
// (index-ordered: a ballot per wave, then the waves' counts give each wave its
// offset), and the (max, sum-of-exp) partial of each head. Contains one
// barrier; the caller has synchronised after filling sc.
template <int G, int NW, int CHUNK, int PITCH>
__device__ __forceinline__ void scan_tail(const float (&sc)[G][PITCH], uint32_t (&wcnt)[G][NW],
                                          const float (&th)[G], float* __restrict__ scores,
                                          float2* __restrict__ part, uint2* __restrict__ cand,
                                          uint32_t* __restrict__ cand_cnt, const bool use_theta,
                                          int b, int Hq, int h0, int t, int ld, int nchunks,
                                          int chunk, int w, int lane, bool skip_hinted = false,
                                          int nq = G) {
  // heads j >= nq pad the matrix-core operand and have no outputs
  const int base_row = chunk * CHUNK;
  const int nrows = min(CHUNK, t - base_row);
  // write-back: one float4 of one head's row per thread and pass
  constexpr int V4 = CHUNK / 4;
  static_assert(V4 == kWave, "one head's row segment per wave");
#pragma unroll
  for (int e = threadIdx.x; e < G * V4; e += kScoreThreads) {
    // V4 = 64: one head per wave and pass, so j is wave-uniform
    const int j = __builtin_amdgcn_readfirstlane(e / V4);
    const int i = (e - j * V4) * 4;
    if (j >= nq || (skip_hinted && __builtin_isfinite(th[j]))) continue;
    float* dst = scores + (size_t)(b * Hq + h0 + j) * ld + base_row;  // wave-uniform
    if (i + 4 <= nrows) {
      store_through(dst, (uint32_t)nrows * 4u, (uint32_t)i * 4u,
                    *reinterpret_cast<const float4*>(&sc[j][i]));
    } else {
      for (int x = i; x < nrows; ++x) dst[x] = sc[j][x];
    }
  }
  if (use_theta) {
    uint64_t hits[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int r = w * kWave + lane;
      const bool hit = j < nq && __builtin_isfinite(th[j]) && r < nrows && sc[j][r] >= th[j];
      hits[j] = __ballot(hit);
      if (lane == 0) wcnt[j][w] = (uint32_t)__popcll(hits[j]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (j >= nq) continue;
      const size_t hc = (size_t)(b * Hq + h0 + j) * nchunks + chunk;
      if (!__builtin_isfinite(th[j])) {
        if (threadIdx.x == 0) store_through(cand_cnt + hc, 4u, 0u, kNoCand);
        continue;
      }
      uint32_t base = 0, total = 0;
#pragma unroll
      for (int u = 0; u < NW; ++u) {
        const uint32_t c = wcnt[j][u];
        base += u < w ? c : 0u;
        total += c;
      }
      const int r = w * kWave + lane;
      if ((hits[j] >> lane) & 1ull) {
        const uint32_t pos = base + (uint32_t)__popcll(hits[j] & ((1ull << lane) - 1ull));
        store_through(cand + hc * CHUNK, CHUNK * 8u, pos * 8u,
                      make_uint2(__float_as_uint(sc[j][r]), (uint32_t)(base_row + r)));
      }
      if (threadIdx.x == 0) store_through(cand_cnt + hc, 4u, 0u, total);
    }
  }
  if (part != nullptr) {
    // L lanes per head: with G >= 4 heads (L <= 64) every head's partial is
    // formed at once by its own lanes, G values each, and reduced by lane
    // exchanges inside the wave; fewer heads take one wave per head in turn
    constexpr int L = (NW * kWave) / G;
    if constexpr (G >= 4 && L * G == NW * kWave && L * G == CHUNK) {
      const int j = (int)threadIdx.x / L;
      const int sub = (int)threadIdx.x % L;
      float v[G];
      float m = -INFINITY;
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const int i = sub + k * L;
        v[k] = i < nrows ? sc[j][i] : -INFINITY;
        m = fmaxf(m, v[k]);
      }
      m = group_max<L>(m);
      float l = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int k = 0; k < G; ++k) l += __expf(v[k] - m);
      }
      l = group_sum<L>(l);
      if (sub == 0 && j < nq)
        store_through(part + (size_t)(b * Hq + h0 + j) * nchunks + chunk, 8u, 0u,
                      make_uint2(__float_as_uint(m), __float_as_uint(l)));
    } else {
      for (int j = w; j < nq; j += NW) {
        float m = -INFINITY;
        for (int i = lane; i < nrows; i += kWave) m = fmaxf(m, sc[j][i]);
        m = group_max<kWave>(m);
        float l = 0.f;
        if (m != -INFINITY)
          for (int i = lane; i < nrows; i += kWave) l += __expf(sc[j][i] - m);
        l = group_sum<kWave>(l);
        if (lane == 0)
          store_through(part + (size_t)(b * Hq + h0 + j) * nchunks + chunk, 8u, 0u,
                        make_uint2(__float_as_uint(m), __float_as_uint(l)));
      }
    }
  }
}

// With `active` (per query head), a workgroup whose group has no active head
// does nothing. With `theta` (a per-head threshold per unit query norm), the
// chunk's keys whose score is >= theta * |q| are also written, in index order,
// as (score bits, index) pairs to cand[head][chunk][0:n] with n in
// cand_cnt[head][chunk]; a head whose theta * |q| is not finite gets the count
// kNoCand.
template <typename T, int D, int G, int CHUNK = kScoreChunk, int UMAX = kScoreLoads>
__global__ __launch_bounds__(kScoreThreads) void score_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, float* __restrict__ scores,
    float2* __restrict__ part, const float* __restrict__ theta, uint2* __restrict__ cand,
    uint32_t* __restrict__ cand_cnt, const int* __restrict__ active, int Hq, int Hkv, int t,
    long long sb, long long sh, long long st, int ld, int nchunks, int g_off, float scale) {
  constexpr int NW = kScoreThreads / kWave;
  constexpr int E = Elem<T>::kPer16B;
  constexpr int LPR = D / E;
  constexpr int RPW = kWave / LPR;
  constexpr int RW = CHUNK / NW;
  constexpr int U = RW / RPW < UMAX ? RW / RPW : UMAX;
  constexpr int ITERS = RW / (U * RPW);
  static_assert(G <= LPR, "one lane per head in a row group");
  static_assert(RW % (U * RPW) == 0, "chunk tiling");
  static_assert(CHUNK == kScoreThreads, "candidate compaction maps one row per thread");

  // Each head's staging row is padded by RPW (at least 4) floats, so the
  // lanes that write one wave-load's RPW rows for G heads hit distinct banks
  // (and the rows stay 16-byte aligned for the vector read-back).
  constexpr int PITCH = CHUNK + (RPW > 4 ? RPW : 4);
  __shared__ __align__(16) float sc[G][PITCH];
  __shared__ uint32_t wcnt[G][NW];

  const int chunk = blockIdx.x;
  const int unit = blockIdx.y;
  const int b = unit / Hkv;
  const int g = unit - b * Hkv;
  const int h0 = g * (Hq / Hkv) + g_off;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int c = lane % LPR;
  const int rr = lane / LPR;
  if (active != nullptr) {
    // the whole workgroup leaves when no head of the group is active
    bool any = false;
#pragma unroll
    for (int j = 0; j < G; ++j) any |= active[b * Hq + h0 + j] != 0;
    if (!any) return;
  }

  // The thresholds are read now, so that their latency hides behind the K
  // loads instead of stalling the workgroup's tail; each is scaled by its
  // head's query norm after the scoring loop.
  float th[G] = {};
  if (theta != nullptr) {
#pragma unroll
    for (int j = 0; j < G; ++j) th[j] = theta[b * Hq + h0 + j];
  }

  uint4 qv[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int hj = LPR == 16 ? rs16_qorder<G>(j, c) : j;
    qv[j] = load16(q + ((size_t)(b * Hq + h0 + hj) * D + c * E));
  }

  const char* kbase = reinterpret_cast<const char*>(k + b * sb + g * sh) + c * 16;
  const size_t row_bytes = (size_t)st * sizeof(T);
  const int wrow0 = w * RW;
  const int grow0 = chunk * CHUNK + wrow0;
  // every chunk but the last lies inside [0, t): its loads need no checks
  const bool full = (chunk + 1) * CHUNK <= t;

#pragma unroll 1
  for (int it = 0; it < ITERS; ++it) {
    uint4 kv[U];
    const char* p0 = kbase + (size_t)(grow0 + it * U * RPW + rr) * row_bytes;
    const size_t step = (size_t)RPW * row_bytes;
    if (full) {
#pragma unroll
      for (int u = 0; u < U; ++u) kv[u] = load16_stream(p0 + u * step);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = grow0 + it * U * RPW + u * RPW + rr;
        kv[u] = r < t ? load16_stream(p0 + u * step) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc[G];
      if constexpr (LPR == 16) {
#pragma unroll
        for (int j = 0; j < G; ++j) acc[j] = dot16_zero(kv[u], qv[j], T());
        float val = rs16<G>(acc);
        // The last exchange must run on every lane (its DPP source lanes
        // are the other lanes of the head): keep it ahead of the branch.
        asm volatile("" : "+v"(val));
        // lanes holding the same head carry the same sum: one writes it
        if ((c & (16 / G - 1)) == 0)
          sc[rs16_head<G>(c)][wrow0 + it * U * RPW + u * RPW + rr] = val * scale;
      } else {
#pragma unroll
        for (int j = 0; j < G; ++j) acc[j] = group_sum<LPR>(dot16(kv[u], qv[j], 0.f, T()));
        float val = acc[0];
#pragma unroll
        for (int j = 1; j < G; ++j) val = (c == j) ? acc[j] : val;
        if (c < G) sc[c][wrow0 + it * U * RPW + u * RPW + rr] = val * scale;
      }
    }
  }
  if (theta != nullptr) {
#pragma unroll
    for (int j = 0; j < G; ++j) th[j] *= query_norm<T, D>(q + (size_t)(b * Hq + h0 + j) * D, lane);
  }
  __syncthreads();

  scan_tail<G, NW, CHUNK, PITCH>(sc, wcnt, th, scores, part, cand, cand_cnt, theta != nullptr, b,
                                 Hq, h0, t, ld, nchunks, chunk, w, lane);
}

// Matrix-core scan of fp16 rows with d = 128; same outputs and grid as
// score_scan_kernel (one 256-key chunk per workgroup, 64 rows per wave),
// scored 16 keys at a time by mfma_score16 (query heads as the rows of A,
// keys as the columns of B). Rows at or past t (last chunk only) load row
// t - 1 instead, so every load is in bounds and branch-free; their scores are
// never written. The sub-group has nq <= G heads (G the operand's rows): a
// group of up to 16 heads is one launch, so K is read once for all of them.
// With skip_hinted, a head whose threshold is finite gets its
// candidates but no score row (the selection recomputes the row with the same
// helpers if the candidates do not hold its answer).
template <int G>
__global__ __launch_bounds__(kScoreThreads) void score_scan_mfma_kernel(
    const __half* __restrict__ q, const __half* __restrict__ k, float* __restrict__ scores,
    float2* __restrict__ part, const float* __restrict__ theta, uint2* __restrict__ cand,
    uint32_t* __restrict__ cand_cnt, const int* __restrict__ active, int Hq, int Hkv, int t,
    long long sb, long long sh, long long st, int ld, int nchunks, int g_off, int nq, float scale,
    int skip_hinted) {
  constexpr int D = 128;
  constexpr int NW = kScoreThreads / kWave;
  constexpr int CHUNK = kScoreChunk;
  constexpr int RW = CHUNK / NW;  // rows per wave and chunk
  constexpr int U = RW / 4;       // 16-byte loads per lane and chunk
  constexpr int PITCH = CHUNK + 4;
  constexpr int NR = G < 4 ? G : 4;  // heads per lane in the product
  static_assert(U == 16, "four 16-key groups per wave and chunk");
  __shared__ __align__(16) float sc[G][PITCH];
  __shared__ uint32_t wcnt[G][NW];
  __shared__ __align__(16) uint4 xt[NW][256];

  const int unit = blockIdx.y;
  const int b = unit / Hkv;
  const int g = unit - b * Hkv;
  const int h0 = g * (Hq / Hkv) + g_off;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c = lane & 15;   // segment of the loaded row; key of the operand
  const int rr = lane >> 4;  // row of the load; k-block of the operand
  if (active != nullptr) {
    bool any = false;
#pragma unroll
    for (int j = 0; j < G; ++j) any |= j < nq && active[b * Hq + h0 + j] != 0;
    if (!any) return;
  }
  float th[G] = {};
  if (theta != nullptr) {
#pragma unroll
    for (int j = 0; j < G; ++j) th[j] = j < nq ? theta[b * Hq + h0 + j] : 0.f;
  }

  half8_t qa[4];
  mfma_query_operand(q + (size_t)(b * Hq + h0) * D, nq, lane, qa);

  // The unit's rows span less than 4 GiB (checked by the launcher), so a
  // load address is the unit's base plus a 32-bit byte offset.
  const char* kunit = reinterpret_cast<const char*>(k + b * sb + g * sh);
  const uint32_t rb = (uint32_t)st * (uint32_t)sizeof(__half);
  const int chunk = blockIdx.x;
  const int row0 = chunk * CHUNK + w * RW + rr;
  uint4 kv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = min(row0 + 4 * u, t - 1);
    kv[u] = load16_stream(kunit + ((uint32_t)c * 16u + (uint32_t)r * rb));
  }
  // Each lane's two fp16 elements of every head's query row, for the norms
  // that scale the thresholds; requested after the K loads and summed just
  // before they are needed, so nothing waits for them.
  uint32_t qw[G] = {};
  if (theta != nullptr) {
#pragma unroll
    for (int j = 0; j < G; ++j)
      if (j < nq)
        qw[j] = reinterpret_cast<const uint32_t*>(q + (size_t)(b * Hq + h0 + j) * D)[lane];
  }

  uint4* tile = xt[w];
#pragma unroll
  for (int a = 0; a < U / 4; ++a) {
    const float4_t acc = mfma_score16(kv[4 * a], kv[4 * a + 1], kv[4 * a + 2], kv[4 * a + 3], qa,
                                      tile, lane);
    // lane l holds heads 4 (l / 16) + r of key l % 16
    if (rr < (G + 3) / 4) {
      const int row = w * RW + 16 * a + c;
#pragma unroll
      for (int r = 0; r < NR; ++r) sc[4 * rr + r][row] = acc[r] * scale;
    }
  }
  if (theta != nullptr) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const __half2 h = __builtin_bit_cast(__half2, qw[j]);
      const float x = __low2float(h), y = __high2float(h);
      th[j] *= __builtin_sqrtf(wave_sum(__builtin_fmaf(x, x, y * y)));
    }
  }
  __syncthreads();
  scan_tail<G, NW, CHUNK, PITCH>(sc, wcnt, th, scores, part, cand, cand_cnt, theta != nullptr, b,
                                 Hq, h0, t, ld, nchunks, chunk, w, lane,
                                 skip_hinted != 0 && theta != nullptr, nq);
}

// Merge the per-chunk partials of each head into its dense log-sum-exp: one
// wave per head, the lanes reading the partials in parallel.
__global__ __launch_bounds__(256) void lse_merge_kernel(const float2* __restrict__ part,
                                                        float* __restrict__ lse_all, int nheads,
                                                        int nchunks) {
  const int h = blockIdx.x * (256 / kWave) + (int)(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  if (h >= nheads) return;
  float m = -INFINITY, l = 0.f;
  for (int c = lane; c < nchunks; c += kWave) {
    const float2 p = part[(size_t)h * nchunks + c];
    ml_combine(m, l, p.x, p.y);
  }
  wave_ml(m, l);
  if (lane == 0) lse_all[h] = (l > 0.f) ? m + __logf(l) : -INFINITY;
}

template <int G>
void launch_scan_mfma(const prhs_dims& d, const void* q, const void* k, float* scores,
                      float2* part, const ScanCand& cd, int g_off, int nq, hipStream_t stream) {
  const int nchunks = score_nchunks(d);
  dim3 grid(nchunks, d.batch * d.n_kv_heads);
  const float scale = (float)(1.0 / __builtin_sqrt((double)d.head_dim));
  hipLaunchKernelGGL((score_scan_mfma_kernel<G>), grid, dim3(kScoreThreads), 0, stream,
                     static_cast<const __half*>(q), static_cast<const __half*>(k), scores, part,
                     cd.theta, cd.cand, cd.cand_cnt, cd.active, d.n_q_heads, d.n_kv_heads,
                     d.ctx_len, (long long)d.kv_stride_b, (long long)d.kv_stride_h,
                     (long long)d.kv_stride_t, d.scores_ld, nchunks, g_off, nq, scale,
                     cd.skip_hinted ? 1 : 0);
}

template <typename T, int D, int G>
void launch_scan_dot(const prhs_dims& d, const void* q, const void* k, float* scores,
                     float2* part, const ScanCand& cd, int g_off, hipStream_t stream) {
  const int nchunks = score_nchunks(d);
  dim3 grid(nchunks, d.batch * d.n_kv_heads);
  const float scale = (float)(1.0 / __builtin_sqrt((double)d.head_dim));
  hipLaunchKernelGGL((score_scan_kernel<T, D, G>), grid, dim3(kScoreThreads), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), scores, part, cd.theta,
                     cd.cand, cd.cand_cnt, cd.active, d.n_q_heads, d.n_kv_heads, d.ctx_len,
                     (long long)d.kv_stride_b, (long long)d.kv_stride_h, (long long)d.kv_stride_t,
                     d.scores_ld, nchunks, g_off, scale);
}

template <typename T, int D>
void launch_scan_group(const prhs_dims& d, const void* q, const void* k, float* scores,
                       float2* part, const ScanCand& cd, int G, hipStream_t stream) {
  if (scan_uses_mfma(d)) {
    // Runs of up to 16 query heads per launch, each padded to a power-of-two
    // operand: every group of at most 16 heads reads K once.
    for (int off = 0; off < G; off += kMfmaMaxGroup) {
      const int nq = G - off < kMfmaMaxGroup ? G - off : kMfmaMaxGroup;
      switch (mfma_rows(nq)) {
        case 16: launch_scan_mfma<16>(d, q, k, scores, part, cd, off, nq, stream); break;
        case 8: launch_scan_mfma<8>(d, q, k, scores, part, cd, off, nq, stream); break;
        case 4: launch_scan_mfma<4>(d, q, k, scores, part, cd, off, nq, stream); break;
        case 2: launch_scan_mfma<2>(d, q, k, scores, part, cd, off, nq, stream); break;
        default: launch_scan_mfma<1>(d, q, k, scores, part, cd, off, nq, stream); break;
      }
    }
    return;
  }
  // Power-of-two sub-groups of at most 8 heads on the dot-product path.
  for (int off = 0; off < G;) {
    const int sub = dot_subgroup_size(G - off);
    switch (sub) {
      case 8: launch_scan_dot<T, D, 8>(d, q, k, scores, part, cd, off, stream); break;
      case 4: launch_scan_dot<T, D, 4>(d, q, k, scores, part, cd, off, stream); break;
      case 2: launch_scan_dot<T, D, 2>(d, q, k, scores, part, cd, off, stream); break;
      default: launch_scan_dot<T, D, 1>(d, q, k, scores, part, cd, off, stream); break;
    }
    off += sub;
  }
}

}  // namespace

hipError_t launch_score(const prhs_dims& d, const void* q, const void* k, float* scores,
                        float* lse_all, void* ws, hipStream_t stream, const ScanCand* cand) {
  float2* part = static_cast<float2*>(ws);
  const ScanCand cd = cand ? *cand : ScanCand{};
  const int G = d.n_q_heads / d.n_kv_heads;
  if (d.dtype == PRHS_F16) {
    if (d.head_dim == 128) launch_scan_group<__half, 128>(d, q, k, scores, part, cd, G, stream);
    else launch_scan_group<__half, 64>(d, q, k, scores, part, cd, G, stream);
  } else {
    if (d.head_dim == 128) launch_scan_group<float, 128>(d, q, k, scores, part, cd, G, stream);
    else launch_scan_group<float, 64>(d, q, k, scores, part, cd, G, stream);
  }
  if (lse_all) {
    const int nheads = d.batch * d.n_q_heads;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((nheads + 3) / 4), dim3(256), 0, stream, part,
                       lse_all, nheads, score_nchunks(d));
  }
  return hipGetLastError();
}

}  // namespace prhs
