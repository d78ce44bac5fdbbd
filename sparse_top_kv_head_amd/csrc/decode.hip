// Sparse attention over the selected entries (page "Near-Oracle KV Selection
// via Pre-hoc Sparsity for Long-Context Inference": Abstract and the Table V
// caption's fused sparse-attention kernel; Table I tau(.) / delta(.)).
//
// Two shapes of the same computation:
//
// Split-budget decode (few heads): the selected list of a head is cut into
// splits of kDecodeRows entries, one 256-thread workgroup each, so even a few
// heads fill the chip. A workgroup reads its entries' scores (compact from the
// selection, gathered from the score scan, or recomputed from gathered K rows
// on steps without a scan), requests its first V rows with 16-byte lane loads
// (LPR lanes per row, 8 rows in flight per lane) while it turns the scores into
// weights, and accumulates weight * v in fp32. Each split leaves a partial
// (max, sum, output) triple; the merge kernel combines them exactly as the
// online softmax does and, when the dense log-sum-exp is given, writes the
// dropped mass delta and the retained mass tau of the set.
//
// One workgroup per head (decode_head_kernel), when the heads alone fill the
// chip or a set fits one split: the same sources and outputs without partials
// or a merge launch; in its dilation modes it also builds the CIS-dilated set
// itself.
#include "prhs_device.hpp"
#include "prhs_launch.hpp"

namespace prhs {
namespace {

constexpr int kDecThreads = 256;

// Merge the split partials of one head (thread `col` owns output column col):
// splits are taken eight at a time with all their loads issued together.
template <int D>
__device__ __forceinline__ void merge_head(const float* __restrict__ p, int nsplit, int col,
                                           float* __restrict__ out, float* __restrict__ lse_sel,
                                           const float* __restrict__ lse_all,
                                           float* __restrict__ delta, float* __restrict__ tau,
                                           const int* __restrict__ mix, int head) {
  float m = -INFINITY, l = 0.f, o = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float ms[8], ls[8], os[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = s0 + i;
      if (s < nsplit) {
        const float* ps = p + (size_t)s * (D + 2);
        ms[i] = ps[D];
        ls[i] = ps[D + 1];
        os[i] = ps[col];
      } else {
        ms[i] = -INFINITY;
        ls[i] = 0.f;
        os[i] = 0.f;
      }
    }
    float mg = m;
#pragma unroll
    for (int i = 0; i < 8; ++i) mg = fmaxf(mg, ms[i]);
    if (mg == -INFINITY) continue;
    const float f = m == -INFINITY ? 0.f : __expf(m - mg);
    l *= f;
    o *= f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (ms[i] != -INFINITY) {
        const float fi = __expf(ms[i] - mg);
        l += ls[i] * fi;
        o += os[i] * fi;
      }
    }
    m = mg;
  }
  out[(size_t)head * D + col] = l > 0.f ? o / l : 0.f;
  if (col == 0) {
    const float lse = l > 0.f ? m + __logf(l) : -INFINITY;
    lse_sel[head] = lse;
    if (lse_all != nullptr && delta != nullptr && (mix == nullptr || mix[head] != 0)) {
      const float dlt = fminf(fmaxf(-expm1f(lse - lse_all[head]), 0.f), 1.f);
      delta[head] = dlt;
      if (tau != nullptr) tau[head] = 1.f - dlt;
    }
  }
}

constexpr int kModeScores = 0;  // scores of the selected rows are given
constexpr int kModeGather = 1;  // scores are computed from gathered K rows
constexpr int kModeMixed = 2;   // per head, by mix[head]: given (idx) or gathered (idx2)
constexpr int kModeDilate = 3;  // idx: anchor sets, dilated in the kernel; K rows gathered
constexpr int kModeMixedDilate = 4;  // per head, by mix[head]: idx with its scores, or idx
                                     // dilated in the kernel with K rows gathered

// One split of one head. With given scores, the scores of the selected rows are
// read from sel_scores (compact, in idx order) when it is given, else gathered
// from `scores`; otherwise they are computed from gathered K rows. In the mixed
// mode a head with mix[head] != 0 takes (idx, count, sel_scores) and any other
// head (idx2, count2) with gathered K rows. Each wave owns
// 64 consecutive rows of the split; their V rows are requested as soon as the
// indices are known, before the split's weights are formed. The split leaves
// (max, sum, o[D]) for the merge kernel. (Merging in the last split to arrive
// needs a device-scope fence per workgroup, which costs far more on this chip
// than the separate merge launch.)
template <typename T, int D, int MODE>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int* __restrict__ idx, int idx_cap, const int* __restrict__ count,
    const float* __restrict__ sel_scores, const float* __restrict__ scores,
    const int* __restrict__ idx2, int idx2_cap, const int* __restrict__ count2,
    const int* __restrict__ mix, int Hq, int Hkv, int t, long long sb, long long sh,
    long long st, int ld, float scale, float* __restrict__ part, int nsplit) {
  constexpr int NW = kDecThreads / kWave;
  constexpr int ROWS = kDecodeRows;
  constexpr int E = Elem<T>::kPer16B;
  constexpr int LPR = D / E;
  constexpr int RPW = kWave / LPR;
  constexpr int RW = ROWS / NW;                    // rows per wave
  constexpr int U = RW / RPW < 8 ? RW / RPW : 8;  // loads in flight per lane
  constexpr int IT = RW / (U * RPW);
  static_assert(RW % (U * RPW) == 0, "split tiling");

  __shared__ int sidx[ROWS];
  __shared__ float sp[ROWS];
  __shared__ float sred[NW];
  __shared__ __align__(16) float so[NW][D];

  const int split = blockIdx.x;
  const int head = blockIdx.y;
  const int b = head / Hq;
  const int h = head - b * Hq;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int c = lane % LPR;
  const int rr = lane / LPR;

  const bool has_scores = MODE == kModeScores || (MODE == kModeMixed && mix[head] != 0);
  const int* ih = has_scores || MODE == kModeGather ? idx : idx2;
  const int icap = has_scores || MODE == kModeGather ? idx_cap : idx2_cap;
  const int* ch = has_scores || MODE == kModeGather ? count : count2;
  const int n = max(0, min(ch[head], icap));
  const int beg = split * ROWS;
  const int nr = max(0, min(ROWS, n - beg));
  const int* irow = ih + (size_t)head * icap + beg;

  for (int i = tid; i < nr; i += kDecThreads) {
    const int id = irow[i];
    const bool ok = id >= 0 && id < t;
    PRHS_CHECK(ok, kCheckIndex);
    sidx[i] = ok ? id : -1;
    if (has_scores)
      sp[i] = !ok ? -INFINITY
                  : sel_scores ? sel_scores[(size_t)head * idx_cap + beg + i]
                               : scores[(size_t)head * ld + id];
  }
  __syncthreads();

  const size_t kv_off = (size_t)b * sb + (size_t)g * sh;
  const size_t row_bytes = (size_t)st * sizeof(T);
  if (MODE != kModeScores && !has_scores) {
    const uint4 qv = load16(q + (size_t)head * D + c * E);
    const char* kbase = reinterpret_cast<const char*>(k + kv_off) + c * 16;
#pragma unroll 1
    for (int it = 0; it < IT; ++it) {
      uint4 kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = w * RW + (it * U + u) * RPW + rr;
        const int id = i < nr ? sidx[i] : -1;
        kv[u] = id >= 0 ? load16_stream(kbase + (size_t)id * row_bytes) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = w * RW + (it * U + u) * RPW + rr;
        const float s = group_sum<LPR>(dot16(kv[u], qv, 0.f, T()));
        if (c == 0 && i < nr) sp[i] = sidx[i] >= 0 ? s * scale : -INFINITY;
      }
    }
    __syncthreads();
  }

  // request the first batch of V rows before the weights are formed
  const char* vbase = reinterpret_cast<const char*>(v + kv_off) + c * 16;
  uint4 vv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = w * RW + u * RPW + rr;
    const int id = i < nr ? sidx[i] : -1;
    vv[u] = id >= 0 ? load16_stream(vbase + (size_t)id * row_bytes) : make_uint4(0, 0, 0, 0);
  }

  // split maximum
  float m = -INFINITY;
  for (int i = tid; i < nr; i += kDecThreads) m = fmaxf(m, sp[i]);
  m = wave_max(m);
  if (lane == 0) sred[w] = m;
  __syncthreads();
  m = sred[0];
#pragma unroll
  for (int k2 = 1; k2 < NW; ++k2) m = fmaxf(m, sred[k2]);
  __syncthreads();
  // weights and their sum
  float l = 0.f;
  for (int i = tid; i < nr; i += kDecThreads) {
    const float p = (m == -INFINITY) ? 0.f : __expf(sp[i] - m);
    sp[i] = p;
    l += p;
  }
  l = wave_sum(l);
  if (lane == 0) sred[w] = l;
  __syncthreads();
  l = 0.f;
#pragma unroll
  for (int k2 = 0; k2 < NW; ++k2) l += sred[k2];

  // weighted V rows
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll 1
  for (int it = 0; it < IT; ++it) {
    if (it > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = w * RW + (it * U + u) * RPW + rr;
        const int id = i < nr ? sidx[i] : -1;
        vv[u] = id >= 0 ? load16_stream(vbase + (size_t)id * row_bytes) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = w * RW + (it * U + u) * RPW + rr;
      const float pw = (i < nr && sidx[i] >= 0) ? sp[i] : 0.f;
      axpy16(pw, vv[u], acc, T());
    }
  }
  // sum the RPW row slots of the wave (lanes c, c+LPR, ...)
#pragma unroll
  for (int e = 0; e < E; ++e) {
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1) acc[e] += __shfl_xor(acc[e], o);
  }
  if (rr == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) so[w][c * E + e] = acc[e];
  }
  __syncthreads();
  float* dst = part + ((size_t)head * nsplit + split) * (D + 2);
  for (int col = tid; col < D; col += kDecThreads) {
    float s = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < NW; ++k2) s += so[k2][col];
    dst[col] = s;
  }
  if (tid == 0) {
    dst[D] = m;
    dst[D + 1] = l;
  }
}

// Merge of one head's split partials: thread `col` owns one output column.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ part, int nsplit,
                                                         float* __restrict__ out,
                                                         float* __restrict__ lse_sel,
                                                         const float* __restrict__ lse_all,
                                                         float* __restrict__ delta,
                                                         float* __restrict__ tau,
                                                         const int* __restrict__ mix) {
  const int head = blockIdx.x;
  merge_head<D>(part + (size_t)head * nsplit * (D + 2), nsplit, threadIdx.x, out, lse_sel,
                lse_all, delta, tau, mix, head);
}

// The whole decode of one head in one 1024-thread workgroup, used when the
// heads alone fill the chip (or a set fits one split): no partials and no
// merge launch. The index list is staged in LDS first. Wave w takes a
// contiguous share of the head's rows: it forms their scores (given, gathered
// from the score row, or computed from gathered K rows, kHeadLoads rows in
// flight per lane) into LDS, then at once gathers their V rows and weighs them
// by exp(s - m_w) with its own maximum m_w, so no barrier separates the two
// phases. The 16 wave partials are then rescaled to the head's maximum and
// added, as the online softmax merges. Sources, index checks and outputs are
// those of the split kernel and its merge.
constexpr int kHeadThreads = 1024;
constexpr int kHeadLoads = 8;
constexpr int kShortWindow = 64;

// CIS dilation of one head's anchor list src[0:n) into the LDS list
// sidx[0:out_cap), as the dilation kernel defines it: anchor i
// proposes [i - r, i + r] clipped to [0, t), starting after the largest end of
// every earlier window (a running maximum over the list), so the output is the
// sorted union for an ascending list and strictly ascending for any list;
// prefix sums of the window lengths give the offsets. Windows of at most
// kShortWindow keys, written by their own thread. out_cap must not exceed the
// LDS list. Returns min(total, out_cap).
// `first` is src[threadIdx.x] (or anything past n), loaded by the caller
// together with the count.
__device__ __forceinline__ int dilate_to_lds(const int* __restrict__ src, int n, int first, int r,
                                             int t, int* sidx, int out_cap,
                                             int (*s_wmax)[kHeadThreads / kWave],
                                             uint32_t (*s_wsum)[kHeadThreads / kWave]) {
  constexpr int NT = kHeadThreads, NW = NT / kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  int base = 0;
  int prev_end = -1;
  int next = tid < n ? first : -1;
  for (int tile = 0, par = 0; tile < n; tile += NT, par ^= 1) {
    const int j = tile + tid;
    const int i = next;
    next = j + NT < n ? src[j + NT] : -1;
    PRHS_CHECK(j >= n || (i >= 0 && i < t), kCheckIndex);
    PRHS_CHECK(j >= n || j == 0 || src[j - 1] < i, kCheckOrder);
    int lo = 0, hi = -1;
    if (j < n && i >= 0 && i < t) {
      lo = i - r > 0 ? i - r : 0;
      hi = i < t - 1 - r ? i + r : t - 1;
    }
    const int incl_max = wave_inclusive_max(hi);
    if (lane == kWave - 1) s_wmax[par][w] = incl_max;
    __syncthreads();
    int before = prev_end;
    int tile_max = prev_end;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int v = s_wmax[par][k];
      if (k < w) before = before > v ? before : v;
      tile_max = tile_max > v ? tile_max : v;
    }
    int excl_max = __shfl_up(incl_max, 1);
    if (lane == 0) excl_max = -1;
    if (excl_max > before) before = excl_max;
    if (lo < before + 1) lo = before + 1;
    const uint32_t len = hi >= lo ? (uint32_t)(hi - lo + 1) : 0u;
    const uint32_t incl = wave_scan_u32(len);
    if (lane == kWave - 1) s_wsum[par][w] = incl;
    __syncthreads();
    uint32_t off = 0, tile_total = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const uint32_t v = s_wsum[par][k];
      if (k < w) off += v;
      tile_total += v;
    }
    off += incl - len;
    for (uint32_t k = 0; k < len; ++k) {
      const uint32_t o = (uint32_t)base + off + k;
      if (o < (uint32_t)out_cap) sidx[o] = lo + (int)k;
    }
    base += (int)tile_total;
    prev_end = tile_max;
  }
  return base < out_cap ? base : out_cap;
}

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kHeadThreads) void decode_head_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int* __restrict__ idx, int idx_cap, const int* __restrict__ count,
    const float* __restrict__ sel_scores, const float* __restrict__ scores,
    const int* __restrict__ idx2, int idx2_cap, const int* __restrict__ count2,
    const int* __restrict__ mix, int Hq, int Hkv, int t, long long sb, long long sh,
    long long st, int ld, float scale, float* __restrict__ out, float* __restrict__ lse_sel,
    const float* __restrict__ lse_all, float* __restrict__ delta, float* __restrict__ tau,
    int radius, int* __restrict__ dil_idx, int dil_cap, int* __restrict__ dil_count) {
  constexpr int NW = kHeadThreads / kWave;
  constexpr int E = Elem<T>::kPer16B;
  constexpr int LPR = D / E;
  constexpr int RPW = kWave / LPR;
  constexpr int U = kHeadLoads;
  __shared__ int sidx[kDecodeHeadRows];
  __shared__ float sp[kDecodeHeadRows];
  __shared__ float sm[NW];
  __shared__ float sl[NW];
  __shared__ __align__(16) float so[NW][D];
  __shared__ int s_wmax[2][NW];
  __shared__ uint32_t s_wsum[2][NW];

  const int head = blockIdx.x;
  const int b = head / Hq;
  const int g = (head - b * Hq) / (Hq / Hkv);
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int c = lane % LPR;
  const int rr = lane / LPR;

  const bool has_scores =
      MODE == kModeScores ||
      ((MODE == kModeMixed || MODE == kModeMixedDilate) && mix[head] != 0);
  const bool primary =
      has_scores || MODE == kModeGather || MODE == kModeDilate || MODE == kModeMixedDilate;
  const bool dilate = MODE == kModeDilate || (MODE == kModeMixedDilate && !has_scores);
  const int* ih = primary ? idx : idx2;
  const int icap = primary ? idx_cap : idx2_cap;
  const int* ch = primary ? count : count2;
  const int* irow = ih + (size_t)head * icap;
  // the list's first entries are requested with the count (the capacity
  // bounds the buffer), so the two loads share one round trip
  const int first = (int)threadIdx.x < icap ? irow[threadIdx.x] : -1;
  int n = max(0, min(ch[head], icap));
  // the index list in LDS (indices outside [0, t) become -1): the given list,
  // or the dilation of the anchor list
  if (dilate) {  // uniform over the workgroup
    n = dilate_to_lds(irow, n, first, radius < t ? radius : t, t, sidx, dil_cap, s_wmax, s_wsum);
    if (threadIdx.x == 0) dil_count[head] = n;
  } else {
    // the rest of the list, four entries per thread requested together
    for (int r0 = 0; r0 < n; r0 += 4 * kHeadThreads) {
      int ids[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u * kHeadThreads + (int)threadIdx.x;
        ids[u] = r >= n ? -1 : r < kHeadThreads ? first : irow[r];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u * kHeadThreads + (int)threadIdx.x;
        if (r < n) {
          PRHS_CHECK(ids[u] >= 0 && ids[u] < t, kCheckIndex);
          sidx[r] = ids[u] >= 0 && ids[u] < t ? ids[u] : -1;
        }
      }
    }
  }
  __syncthreads();
  if (dilate) {
    // the dilated list goes out from LDS in whole rows, through the L2, while
    // the K and V rows are gathered
    int* dst = dil_idx + (size_t)head * dil_cap;
    for (int r = threadIdx.x; r < n; r += kHeadThreads)
      store_through(dst, (uint32_t)dil_cap * 4u, (uint32_t)r * 4u, (uint32_t)sidx[r]);
  }
  const int rw = ((n + NW - 1) / NW + RPW - 1) / RPW * RPW;
  const int rb = w * rw;
  const int re = min(n, rb + rw);
  const size_t kv_off = (size_t)b * sb + (size_t)g * sh;
  const size_t row_bytes = (size_t)st * sizeof(T);

  // the scores of the wave's rows
  float mw = -INFINITY;
  if (has_scores) {
    for (int r = rb + lane; r < re; r += kWave) {
      const int id = sidx[r];
      const float sv = id < 0 ? -INFINITY
                              : sel_scores ? sel_scores[(size_t)head * idx_cap + r]
                                           : scores[(size_t)head * ld + id];
      sp[r] = sv;
      mw = fmaxf(mw, sv);
    }
  } else {
    const uint4 qv = load16(q + (size_t)head * D + c * E);
    const char* kbase = reinterpret_cast<const char*>(k + kv_off) + c * 16;
    for (int r0 = rb; r0 < re; r0 += U * RPW) {
      uint4 kv[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * RPW + rr;
        const int id = r < re ? sidx[r] : -1;
        ok[u] = id >= 0;
        kv[u] = ok[u] ? load16_stream(kbase + (size_t)id * row_bytes) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * RPW + rr;
        const float sv = ok[u] ? group_sum<LPR>(dot16(kv[u], qv, 0.f, T())) * scale : -INFINITY;
        if (c == 0 && r < re) sp[r] = sv;
        mw = fmaxf(mw, sv);
      }
    }
  }
  const float m = wave_max(mw);
  // the wave reads back rows that other lanes of the same wave scored
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // weighted V rows against the wave's own maximum (rows with a skipped index
  // carry -inf, so weight 0)
  const char* vbase = reinterpret_cast<const char*>(v + kv_off) + c * 16;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float l = 0.f;
  for (int r0 = rb; r0 < re; r0 += U * RPW) {
    uint4 vv[U];
    float p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RPW + rr;
      const float sv = r < re ? sp[r] : -INFINITY;
      const bool ok = sv != -INFINITY;
      const int id = ok ? sidx[r] : 0;
      vv[u] = ok ? load16_stream(vbase + (size_t)id * row_bytes) : make_uint4(0, 0, 0, 0);
      p[u] = ok ? __expf(sv - m) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      axpy16(p[u], vv[u], acc, T());
      if (c == 0) l += p[u];
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1) acc[e] += __shfl_xor(acc[e], o);
  }
  l = wave_sum(l);
  if (rr == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) so[w][c * E + e] = acc[e];
  }
  if (lane == 0) {
    sm[w] = m;
    sl[w] = l;
  }
  __syncthreads();
  // the wave partials, rescaled to the head's maximum
  if ((int)threadIdx.x < D) {
    float mh = sm[0];
#pragma unroll
    for (int k2 = 1; k2 < NW; ++k2) mh = fmaxf(mh, sm[k2]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < NW; ++k2) {
      const float f = sm[k2] == -INFINITY ? 0.f : __expf(sm[k2] - mh);
      o += so[k2][threadIdx.x] * f;
      L += sl[k2] * f;
    }
    out[(size_t)head * D + threadIdx.x] = L > 0.f ? o / L : 0.f;
    if (threadIdx.x == 0) {
      const float lse = L > 0.f ? mh + __logf(L) : -INFINITY;
      lse_sel[head] = lse;
      if (lse_all != nullptr && delta != nullptr && (mix == nullptr || mix[head] != 0)) {
        const float dlt = fminf(fmaxf(-expm1f(lse - lse_all[head]), 0.f), 1.f);
        delta[head] = dlt;
        if (tau != nullptr) tau[head] = 1.f - dlt;
      }
    }
  }
}

__global__ __launch_bounds__(256) void dropped_mass_kernel(const float* __restrict__ lse_sel,
                                                           const float* __restrict__ lse_all,
                                                           float* __restrict__ delta,
                                                           float* __restrict__ tau, int nheads) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= nheads) return;
  const float dlt = fminf(fmaxf(-expm1f(lse_sel[h] - lse_all[h]), 0.f), 1.f);
  delta[h] = dlt;
  if (tau != nullptr) tau[h] = 1.f - dlt;
}

struct SplitArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* idx;
  int idx_cap;
  const int* count;
  const float* sel_scores;
  const float* scores;
  const int* idx2;
  int idx2_cap;
  const int* count2;
  const int* mix;
};

template <typename T, int D, int MODE>
void launch_split_mode(const prhs_dims& d, const SplitArgs& a, float* part, int nsplit,
                       hipStream_t stream) {
  dim3 grid(nsplit, d.batch * d.n_q_heads);
  const float scale = (float)(1.0 / __builtin_sqrt((double)d.head_dim));
  hipLaunchKernelGGL((decode_split_kernel<T, D, MODE>), grid, dim3(kDecThreads), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), a.idx, a.idx_cap, a.count, a.sel_scores, a.scores,
                     a.idx2, a.idx2_cap, a.count2, a.mix, d.n_q_heads, d.n_kv_heads, d.ctx_len,
                     (long long)d.kv_stride_b, (long long)d.kv_stride_h, (long long)d.kv_stride_t,
                     d.scores_ld, scale, part, nsplit);
}

// Dilation output of the fused reuse step (kModeDilate only).
struct DilateArgs {
  int radius = 0;
  int* idx = nullptr;
  int cap = 0;
  int* count = nullptr;
};

template <typename T, int D, int MODE>
void launch_head_mode(const prhs_dims& d, const SplitArgs& a, float* out, float* lse_sel,
                      const float* lse_all, float* delta, float* tau, hipStream_t stream,
                      const DilateArgs& dl = DilateArgs()) {
  const float scale = (float)(1.0 / __builtin_sqrt((double)d.head_dim));
  hipLaunchKernelGGL((decode_head_kernel<T, D, MODE>), dim3(d.batch * d.n_q_heads),
                     dim3(kHeadThreads), 0, stream, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.idx, a.idx_cap,
                     a.count, a.sel_scores, a.scores, a.idx2, a.idx2_cap, a.count2, a.mix,
                     d.n_q_heads, d.n_kv_heads, d.ctx_len, (long long)d.kv_stride_b,
                     (long long)d.kv_stride_h, (long long)d.kv_stride_t, d.scores_ld, scale, out,
                     lse_sel, lse_all, delta, tau, dl.radius, dl.idx, dl.cap, dl.count);
}

template <typename T, int D>
void launch_reuse_head(const prhs_dims& d, const SplitArgs& a, float* out, float* lse_sel,
                       const DilateArgs& dl, hipStream_t stream) {
  launch_head_mode<T, D, kModeDilate>(d, a, out, lse_sel, nullptr, nullptr, nullptr, stream, dl);
}

template <typename T, int D>
void launch_head(const prhs_dims& d, const SplitArgs& a, float* out, float* lse_sel,
                 const float* lse_all, float* delta, float* tau, hipStream_t stream) {
  if (a.mix != nullptr)
    launch_head_mode<T, D, kModeMixed>(d, a, out, lse_sel, lse_all, delta, tau, stream);
  else if (a.scores || a.sel_scores)
    launch_head_mode<T, D, kModeScores>(d, a, out, lse_sel, lse_all, delta, tau, stream);
  else
    launch_head_mode<T, D, kModeGather>(d, a, out, lse_sel, lse_all, delta, tau, stream);
}

void launch_head_any(const prhs_dims& d, const SplitArgs& a, float* out, float* lse_sel,
                     const float* lse_all, float* delta, float* tau, hipStream_t stream) {
  if (d.dtype == PRHS_F16) {
    if (d.head_dim == 128) launch_head<__half, 128>(d, a, out, lse_sel, lse_all, delta, tau, stream);
    else launch_head<__half, 64>(d, a, out, lse_sel, lse_all, delta, tau, stream);
  } else {
    if (d.head_dim == 128) launch_head<float, 128>(d, a, out, lse_sel, lse_all, delta, tau, stream);
    else launch_head<float, 64>(d, a, out, lse_sel, lse_all, delta, tau, stream);
  }
}

template <typename T, int D>
void launch_split(const prhs_dims& d, const SplitArgs& a, float* part, int nsplit,
                  hipStream_t stream) {
  if (a.mix != nullptr) launch_split_mode<T, D, kModeMixed>(d, a, part, nsplit, stream);
  else if (a.scores || a.sel_scores) launch_split_mode<T, D, kModeScores>(d, a, part, nsplit, stream);
  else launch_split_mode<T, D, kModeGather>(d, a, part, nsplit, stream);
}

void launch_split_any(const prhs_dims& d, const SplitArgs& a, float* part, int nsplit,
                      hipStream_t stream) {
  if (d.dtype == PRHS_F16) {
    if (d.head_dim == 128) launch_split<__half, 128>(d, a, part, nsplit, stream);
    else launch_split<__half, 64>(d, a, part, nsplit, stream);
  } else {
    if (d.head_dim == 128) launch_split<float, 128>(d, a, part, nsplit, stream);
    else launch_split<float, 64>(d, a, part, nsplit, stream);
  }
}

}  // namespace

hipError_t launch_decode(const prhs_dims& d, const void* q, const void* k, const void* v,
                         const int* idx, int idx_cap, const int* count, const float* sel_scores,
                         const float* scores, const float* lse_all, float* out, float* lse_sel,
                         float* delta, float* tau, void* ws, hipStream_t stream) {
  const SplitArgs a{q, k, v, idx, idx_cap, count, sel_scores, scores, nullptr, 0, nullptr, nullptr};
  if (decode_per_head(d, idx_cap)) {
    launch_head_any(d, a, out, lse_sel, lse_all, delta, tau, stream);
    return hipGetLastError();
  }
  const int nsplit = decode_nsplit(idx_cap);
  float* part = static_cast<float*>(ws);
  launch_split_any(d, a, part, nsplit, stream);
  return launch_merge(d, part, nsplit, out, lse_sel, lse_all, delta, tau, stream);
}

hipError_t launch_decode_mixed(const prhs_dims& d, const void* q, const void* k, const void* v,
                               const int* mix, const int* idx, int idx_cap, const int* count,
                               const float* sel_scores, const int* idx2, int idx2_cap,
                               const int* count2, const float* lse_all, float* out,
                               float* lse_sel, float* delta, float* tau, void* ws,
                               hipStream_t stream) {
  const int cap = idx_cap > idx2_cap ? idx_cap : idx2_cap;
  const SplitArgs a{q, k, v, idx, idx_cap, count, sel_scores, nullptr, idx2, idx2_cap, count2, mix};
  if (decode_per_head(d, cap)) {
    launch_head_any(d, a, out, lse_sel, lse_all, delta, tau, stream);
    return hipGetLastError();
  }
  const int nsplit = decode_nsplit(cap);
  float* part = static_cast<float*>(ws);
  launch_split_any(d, a, part, nsplit, stream);
  return launch_merge(d, part, nsplit, out, lse_sel, lse_all, delta, tau, stream, mix);
}

hipError_t launch_adaptive_decode(const prhs_dims& d, const void* q, const void* k,
                                  const void* v, const int* mix, const int* anchor_idx,
                                  int anchor_cap, const int* anchor_count,
                                  const float* sel_scores, int radius, int* dil_idx, int dil_cap,
                                  int* dil_count, const float* lse_all, float* out,
                                  float* lse_sel, float* delta, float* tau, void* ws,
                                  hipStream_t stream) {
  const int r = radius < d.ctx_len ? radius : d.ctx_len;
  const int cap = anchor_cap > dil_cap ? anchor_cap : dil_cap;
  if (decode_per_head(d, cap) && 2 * r + 1 <= kShortWindow) {
    const SplitArgs a{q, k, v, anchor_idx, anchor_cap, anchor_count, sel_scores, nullptr,
                      nullptr, 0, nullptr, mix};
    DilateArgs dl;
    dl.radius = radius;
    dl.idx = dil_idx;
    dl.cap = dil_cap;
    dl.count = dil_count;
    if (d.dtype == PRHS_F16) {
      if (d.head_dim == 128)
        launch_head_mode<__half, 128, kModeMixedDilate>(d, a, out, lse_sel, lse_all, delta, tau,
                                                        stream, dl);
      else
        launch_head_mode<__half, 64, kModeMixedDilate>(d, a, out, lse_sel, lse_all, delta, tau,
                                                       stream, dl);
    } else {
      if (d.head_dim == 128)
        launch_head_mode<float, 128, kModeMixedDilate>(d, a, out, lse_sel, lse_all, delta, tau,
                                                       stream, dl);
      else
        launch_head_mode<float, 64, kModeMixedDilate>(d, a, out, lse_sel, lse_all, delta, tau,
                                                      stream, dl);
    }
    return hipGetLastError();
  }
  hipError_t err = launch_cis(d, anchor_idx, anchor_cap, anchor_count, radius, nullptr, nullptr,
                              0.f, dil_idx, dil_cap, dil_count, nullptr, stream, mix);
  if (err != hipSuccess) return err;
  return launch_decode_mixed(d, q, k, v, mix, anchor_idx, anchor_cap, anchor_count, sel_scores,
                             dil_idx, dil_cap, dil_count, lse_all, out, lse_sel, delta, tau, ws,
                             stream);
}

hipError_t launch_reuse(const prhs_dims& d, const int* anchor_idx, int anchor_cap,
                        const int* anchor_count, int radius, const void* q, const void* k,
                        const void* v, int* out_idx, int out_cap, int* out_count, float* out,
                        float* lse_sel, void* ws, hipStream_t stream) {
  const int r = radius < d.ctx_len ? radius : d.ctx_len;
  if (decode_per_head(d, out_cap) && 2 * r + 1 <= kShortWindow) {
    const SplitArgs a{q, k, v, anchor_idx, anchor_cap, anchor_count, nullptr, nullptr,
                      nullptr, 0, nullptr, nullptr};
    DilateArgs dl;
    dl.radius = radius;
    dl.idx = out_idx;
    dl.cap = out_cap;
    dl.count = out_count;
    if (d.dtype == PRHS_F16) {
      if (d.head_dim == 128) launch_reuse_head<__half, 128>(d, a, out, lse_sel, dl, stream);
      else launch_reuse_head<__half, 64>(d, a, out, lse_sel, dl, stream);
    } else {
      if (d.head_dim == 128) launch_reuse_head<float, 128>(d, a, out, lse_sel, dl, stream);
      else launch_reuse_head<float, 64>(d, a, out, lse_sel, dl, stream);
    }
    return hipGetLastError();
  }
  hipError_t err = launch_cis(d, anchor_idx, anchor_cap, anchor_count, radius, nullptr, nullptr,
                              0.f, out_idx, out_cap, out_count, nullptr, stream);
  if (err != hipSuccess) return err;
  return launch_decode(d, q, k, v, out_idx, out_cap, out_count, nullptr, nullptr, nullptr, out,
                       lse_sel, nullptr, nullptr, ws, stream);
}

hipError_t launch_merge(const prhs_dims& d, const float* part, int nsplit, float* out,
                        float* lse_sel, const float* lse_all, float* delta, float* tau,
                        hipStream_t stream, const int* mix) {
  const int nheads = d.batch * d.n_q_heads;
  if (d.head_dim == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), dim3(nheads), dim3(128), 0, stream, part, nsplit,
                       out, lse_sel, lse_all, delta, tau, mix);
  else
    hipLaunchKernelGGL((decode_merge_kernel<64>), dim3(nheads), dim3(64), 0, stream, part, nsplit,
                       out, lse_sel, lse_all, delta, tau, mix);
  return hipGetLastError();
}

hipError_t launch_dropped_mass(const prhs_dims& d, const float* lse_sel, const float* lse_all,
                               float* delta, float* tau, hipStream_t stream) {
  const int nheads = d.batch * d.n_q_heads;
  hipLaunchKernelGGL(dropped_mass_kernel, dim3((nheads + 255) / 256), dim3(256), 0, stream,
                     lse_sel, lse_all, delta, tau, nheads);
  return hipGetLastError();
}

PRHS_CHECK_READER(take_checks_decode)

}  // namespace prhs
