// Per-head index selection (page "Near-Oracle KV Selection via Pre-hoc
// Sparsity for Long-Context Inference": Table I selector S / set S_t / budget
// N; the top-k oracle of Fig. 1, Fig. 2 and Fig. 9; the Abstract's control of
// the dropped mass delta before attention).
//
// One 1024-thread workgroup per (b, h). The head's t scores are held in
// registers as order-preserving 32-bit keys, KPT consecutive keys per thread.
// A three-pass most-significant-digit radix search (11 + 11 + 10 bits) over
// LDS histograms finds the exact boundary key T; later passes histogram only
// the keys still matching the boundary prefix. The result set is every key
// above T plus the lowest-index keys equal to T, written in ascending index
// order through one workgroup prefix sum.
//
// DELTA mode runs the same search on attention mass instead of counts: each
// histogram bin also sums the dense weights exp(s - lse) in 2^-40 fixed point,
// and the search walks up from the smallest keys to the first position whose
// suffix mass exceeds the target. That gives the smallest N whose dropped mass
// is within the target; when it exceeds the cap, a count search for the cap
// follows.
#include "prhs_device.hpp"
#include "prhs_launch.hpp"

#include <type_traits>

namespace prhs {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kBins = 2048;
constexpr double kMassScale = 1099511627776.0;  // 2^40

struct Pass {
  int shift;
  int bits;
};
__constant__ Pass kPasses[3] = {{21, 11}, {10, 11}, {0, 10}};

__device__ __forceinline__ float key_to_score(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ unsigned long long mass_fx(uint32_t key, float lse) {
  const float a = __expf(key_to_score(key) - lse);
  return (unsigned long long)__builtin_fmaf(a, (float)kMassScale, 0.5f);
}

template <int KPT>
struct Keys {
  uint32_t k[KPT];
};

// Histogram pass over keys matching (pre, pmask); bins of `bits` bits at `shift`.
template <int KPT, bool MASS>
__device__ __forceinline__ void histogram(const Keys<KPT>& K, int nvalid, uint32_t pre,
                                          uint32_t pmask, int shift, int bits, float lse,
                                          uint32_t* hist, unsigned long long* mhist) {
  for (int i = threadIdx.x; i < kBins; i += kSelThreads) {
    hist[i] = 0;
    if constexpr (MASS) mhist[i] = 0;
  }
  __syncthreads();
  const uint32_t dmask = (1u << bits) - 1u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t key = K.k[j];
    if (j < nvalid && (key & pmask) == pre) {
      const uint32_t dig = (key >> shift) & dmask;
      atomicAdd(&hist[dig], 1u);
      if constexpr (MASS) atomicAdd(&mhist[dig], mass_fx(key, lse));
    }
  }
  __syncthreads();
}

struct SelShared {
  uint32_t hist[kBins];
  unsigned long long scan64[kSelThreads / kWave];
  uint32_t scan32[kSelThreads / kWave];
  uint32_t digit;
  uint32_t above;
  unsigned long long below;
  int found;
};

struct DeltaShared {
  unsigned long long mhist[kBins];
};

// Count search: the krem-th largest key among the keys matching the prefix.
// On return pre holds the boundary key T and krem how many keys equal to T
// are taken.
template <int KPT>
__device__ __forceinline__ void count_search(const Keys<KPT>& K, int nvalid, uint32_t& pre, uint32_t& pmask,
                             uint32_t& krem, int first_pass, SelShared& sh) {
  for (int p = first_pass; p < 3; ++p) {
    const int shift = kPasses[p].shift, bits = kPasses[p].bits;
    const int nb = 1 << bits;
    histogram<KPT, false>(K, nvalid, pre, pmask, shift, bits, 0.f, sh.hist, nullptr);
    // Bins in descending order: thread i owns bins nb-1-2i and nb-2-2i.
    const int hi = nb - 1 - 2 * (int)threadIdx.x;
    const uint32_t c1 = hi >= 0 ? sh.hist[hi] : 0u;
    const uint32_t c0 = hi >= 1 ? sh.hist[hi - 1] : 0u;
    const uint32_t cnt = c1 + c0;
    uint32_t total;
    const uint32_t excl = block_exclusive_scan<kSelThreads>(cnt, sh.scan32, total);
    if (cnt > 0 && excl < krem && krem <= excl + cnt) {
      if (excl + c1 >= krem) {
        sh.digit = (uint32_t)hi;
        sh.above = excl;
      } else {
        sh.digit = (uint32_t)(hi - 1);
        sh.above = excl + c1;
      }
    }
    __syncthreads();
    krem -= sh.above;
    pre |= sh.digit << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
  }
}

// Mass search (DELTA): the first key, walking up from the smallest, whose
// suffix mass (itself and everything ranked below it) exceeds the remaining
// budget. Returns false when the whole set's mass is within the budget.
template <int KPT>
__device__ __forceinline__ bool mass_search(const Keys<KPT>& K, int nvalid, float lse, unsigned long long budget,
                            uint32_t& pre, uint32_t& pmask, uint32_t& above_total,
                            unsigned long long& drem, SelShared& sh, DeltaShared& dsh) {
  drem = budget;
  above_total = 0;
  for (int p = 0; p < 3; ++p) {
    const int shift = kPasses[p].shift, bits = kPasses[p].bits;
    const int nb = 1 << bits;
    histogram<KPT, true>(K, nvalid, pre, pmask, shift, bits, lse, sh.hist, dsh.mhist);
    // Bins in ascending order: thread i owns bins 2i and 2i+1.
    const int lo = 2 * (int)threadIdx.x;
    const uint32_t c0 = lo < nb ? sh.hist[lo] : 0u;
    const uint32_t c1 = lo + 1 < nb ? sh.hist[lo + 1] : 0u;
    const unsigned long long m0 = lo < nb ? dsh.mhist[lo] : 0ull;
    const unsigned long long m1 = lo + 1 < nb ? dsh.mhist[lo + 1] : 0ull;
    unsigned long long mtot;
    const unsigned long long mex = block_exclusive_scan<kSelThreads>(m0 + m1, sh.scan64, mtot);
    uint32_t ctot;
    const uint32_t cex = block_exclusive_scan<kSelThreads>(c0 + c1, sh.scan32, ctot);
    if (threadIdx.x == 0) sh.found = 0;
    __syncthreads();
    if (mex <= drem && drem < mex + m0 + m1) {
      sh.found = 1;
      if (mex + m0 > drem) {
        sh.digit = (uint32_t)lo;
        sh.below = mex;
        sh.above = ctot - (cex + c0);
      } else {
        sh.digit = (uint32_t)(lo + 1);
        sh.below = mex + m0;
        sh.above = ctot - (cex + c0 + c1);
      }
    }
    __syncthreads();
    if (!sh.found) return false;
    drem -= sh.below;
    above_total += sh.above;
    pre |= sh.digit << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    if (p == 2) {
      // Boundary key T = pre: its c_T keys carry identical mass a each. Keys
      // of rank j (by index) among them are taken while their suffix mass
      // (c_T - j + 1) * a exceeds drem.
      const uint32_t cT = sh.hist[sh.digit];
      const unsigned long long a = dsh.mhist[sh.digit] / cT;
      const unsigned long long keep_out = a ? drem / a : (unsigned long long)cT;
      const uint32_t dropped = keep_out < cT ? (uint32_t)keep_out : cT;
      above_total += cT - dropped;  // now the total count taken
    }
    __syncthreads();
  }
  return true;
}

// Write the keys above T and the first `take_eq` keys equal to T, ascending.
template <int KPT>
__device__ __forceinline__ void emit(const Keys<KPT>& K, int nvalid, int i0, uint32_t T, uint32_t take_eq,
                     int* __restrict__ out, uint32_t cap, SelShared& sh) {
  unsigned long long gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (j < nvalid) {
      if (K.k[j] > T) gt |= 1ull << j;
      else if (K.k[j] == T) eq |= 1ull << j;
    }
  }
  const unsigned long long packed =
      ((unsigned long long)__popcll(gt) << 32) | (unsigned long long)__popcll(eq);
  unsigned long long tot;
  const unsigned long long ex = block_exclusive_scan<kSelThreads>(packed, sh.scan64, tot);
  const uint32_t ex_gt = (uint32_t)(ex >> 32), ex_eq = (uint32_t)ex;
  uint32_t eq_take = take_eq > ex_eq ? take_eq - ex_eq : 0u;
  uint32_t pos = ex_gt + (ex_eq < take_eq ? ex_eq : take_eq);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    bool sel = (gt >> j) & 1ull;
    if ((eq >> j) & 1ull) {
      if (eq_take) {
        sel = true;
        --eq_take;
      }
    }
    if (sel) {
      if (pos < cap) out[pos] = i0 + j;  // never past the row, whatever the counts
      ++pos;
    }
  }
}

template <int KPT, int MODE>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ scores, const float* __restrict__ lse_all, int t, int ld,
    int n_budget, float delta_target, int* __restrict__ idx, int idx_cap,
    int* __restrict__ count, int* __restrict__ cap_hit) {
  __shared__ SelShared sh;
  __shared__ typename std::conditional<MODE == PRHS_DELTA, DeltaShared, char>::type dsh_raw;

  const int head = blockIdx.x;
  const float* row = scores + (size_t)head * ld;
  const int i0 = threadIdx.x * KPT;
  const int nvalid = max(0, min(KPT, t - i0));

  Keys<KPT> K;
  if constexpr (KPT >= 4) {
#pragma unroll
    for (int v = 0; v < KPT / 4; ++v) {
      if (4 * v + 4 <= nvalid) {
        const float4 x = *reinterpret_cast<const float4*>(row + i0 + 4 * v);
        K.k[4 * v] = score_key(x.x);
        K.k[4 * v + 1] = score_key(x.y);
        K.k[4 * v + 2] = score_key(x.z);
        K.k[4 * v + 3] = score_key(x.w);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          K.k[4 * v + e] = (4 * v + e < nvalid) ? score_key(row[i0 + 4 * v + e]) : 0u;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) K.k[j] = (j < nvalid) ? score_key(row[i0 + j]) : 0u;
  }

  uint32_t pre = 0, pmask = 0, take = 0;
  int n_sel = n_budget;
  int hit = 0;
  if constexpr (MODE == PRHS_DELTA) {
    DeltaShared& dsh = *reinterpret_cast<DeltaShared*>(&dsh_raw);
    const float lse = lse_all[head];
    const unsigned long long budget =
        (unsigned long long)((double)delta_target * kMassScale);
    uint32_t n_delta = 0;
    unsigned long long drem = 0;
    const bool found = mass_search<KPT>(K, nvalid, lse, budget, pre, pmask, n_delta, drem, sh, dsh);
    if (found && (int)n_delta <= n_budget) {
      n_sel = (int)n_delta;
      // pre is the boundary key; take the keys above it and enough equal keys.
      uint32_t above = 0;
#pragma unroll
      for (int j = 0; j < KPT; ++j) above += (j < nvalid && K.k[j] > pre) ? 1u : 0u;
      uint32_t tot;
      (void)block_exclusive_scan<kSelThreads>(above, sh.scan32, tot);
      take = n_delta - tot;
    } else {
      hit = found ? 1 : 0;
      n_sel = found ? n_budget : 1;
      pre = 0;
      pmask = 0;
      take = (uint32_t)n_sel;
      count_search<KPT>(K, nvalid, pre, pmask, take, 0, sh);
    }
  } else {
    take = (uint32_t)n_budget;
    count_search<KPT>(K, nvalid, pre, pmask, take, 0, sh);
  }
  emit<KPT>(K, nvalid, i0, pre, take, idx + (size_t)head * idx_cap, (uint32_t)idx_cap, sh);
  if (threadIdx.x == 0) {
    count[head] = n_sel;
    if (cap_hit) cap_hit[head] = hit;
  }
}

template <int MODE>
void launch_mode(int kpt, int nheads, const float* scores, const float* lse_all, int t, int ld,
                 int n_budget, float delta_target, int* idx, int idx_cap, int* count, int* cap_hit,
                 hipStream_t stream) {
#define PRHS_SEL(K)                                                                            \
  hipLaunchKernelGGL((select_kernel<K, MODE>), dim3(nheads), dim3(kSelThreads), 0, stream, scores, \
                     lse_all, t, ld, n_budget, delta_target, idx, idx_cap, count, cap_hit)
  switch (kpt) {
    case 1: PRHS_SEL(1); break;
    case 2: PRHS_SEL(2); break;
    case 4: PRHS_SEL(4); break;
    case 8: PRHS_SEL(8); break;
    case 16: PRHS_SEL(16); break;
    case 32: PRHS_SEL(32); break;
    default: PRHS_SEL(64); break;
  }
#undef PRHS_SEL
}

}  // namespace

hipError_t launch_select(const prhs_dims& d, const float* scores, const float* lse_all, int mode,
                         int n_budget, float delta_target, int* idx, int idx_cap, int* count,
                         int* cap_hit, hipStream_t stream) {
  int kpt = 1;
  while (kpt * kSelThreads < d.ctx_len) kpt *= 2;
  const int nheads = d.batch * d.n_q_heads;
  if (mode == PRHS_DELTA)
    launch_mode<PRHS_DELTA>(kpt, nheads, scores, lse_all, d.ctx_len, d.scores_ld, n_budget,
                            delta_target, idx, idx_cap, count, cap_hit, stream);
  else
    launch_mode<PRHS_TOPN>(kpt, nheads, scores, lse_all, d.ctx_len, d.scores_ld, n_budget,
                           delta_target, idx, idx_cap, count, cap_hit, stream);
  return hipGetLastError();
}

}  // namespace prhs
