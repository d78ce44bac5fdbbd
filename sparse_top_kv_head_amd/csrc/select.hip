// Per-head index selection (page "Near-Oracle KV Selection via Pre-hoc
// Sparsity for Long-Context Inference": Table I selector S / set S_t / budget
// N; the top-k oracle of Fig. 1, Fig. 2 and Fig. 9; the Abstract's control of
// the dropped mass delta before attention).
//
// One 1024-thread workgroup per (b, h), working on order-preserving 32-bit
// keys of the fp32 scores (-0 folded onto +0).
//
// TOPN, steady state: the score scan already wrote, per 256-key chunk, the
// keys at or above a per-head threshold carried from the previous anchor step,
// in index order. Their counts give each chunk its offset (one workgroup
// scan); the candidates are gathered into an LDS list, still in index order,
// and a radix search with 12-bit digits of key - min over that list finds the
// exact N-th largest key T (two passes for a typical range; one wave locates
// each boundary bin while the others wait). The selection is written in list
// order, with each row's score, and a threshold for the next step. When the
// carried threshold leaves fewer than N or more than kCandCap keys, the full
// path below runs; the result is exact either way.
//
// Full path: the head's keys are loaded into registers (wave w owns a
// contiguous range of 64*KPT keys, 16-byte loads, lane l holding granules of
// 4 consecutive keys at stride 256). A 1-in-8 sample is histogrammed on its
// top 11 bits to pick a threshold theta that at least N keys clear with a
// wide margin; the keys >= theta (a few thousand) are compacted with their
// indices into the LDS list and the same 12-bit radix search finds T. If the
// sample misleads, an 11 + 11 + 10-bit radix search streams the (L2-resident)
// score row instead of holding keys in registers, the first pass adding into
// kRep1 copies of the histogram because most keys land in a few crowded bins,
// the later ones over the boundary bin's keys compacted to LDS. Only candidate
// building holds keys in registers, so no path spills.
//
// The result is every key above T plus the lowest-index keys equal to T. The
// keys are marked in two LDS bitmaps (above T, equal to T) indexed by key
// position; one workgroup scan over the bitmap words gives each word its final
// selection and output offset, and the indices and scores are scattered from
// the LDS list (or the streamed row) in ascending index order.
//
// Contexts longer than the keys the registers hold (64K) take the streamed
// path from the start: the top key and the exact boundary come from passes
// over the row, and the selection is emitted in 64K-position tiles of the
// bitmaps, each tile continuing the previous one's output offset and its
// count of keys equal to T already taken.
//
// DELTA mode first finds the cap-th largest key Tc as above and sums the
// dense weights exp(s - lse) of the keys outside the top-cap set, in 2^-40
// fixed point (exact, order-free integer sums). If that dropped mass exceeds
// the target the cap binds. Otherwise the smallest N lies within the top-cap
// set: a radix search on mass over the keys >= Tc (each bin also sums their
// weights) walks up from the smallest of them, with the mass below Tc already
// spent, to the first position whose suffix mass exceeds the target.
#include "prhs_device.hpp"
#include "prhs_launch.hpp"

#include <type_traits>

namespace prhs {
namespace {

constexpr int kBins = 2048;
constexpr int kRep1 = 4;                 // copies of the first-pass count histogram
constexpr int kCandCap = 8192;           // LDS candidate list capacity (keys and indices)
// Positions the LDS bitmaps cover at once; longer rows are emitted in tiles.
constexpr int kTileKeys = 65536;
constexpr int kMaxWords = kTileKeys / 32;
// Threads per selection workgroup: 1024, or 512 for top-N rows of at most
// kShortCtx keys, where half the waves make the latency-bound phases cheaper
// and 8 keys per thread still hold the row (LLaMA2-shaped 4K step 19.0 ->
// 17.7 us with the two-chunk read-ahead of gather_candidates).
constexpr int kSelThreads = 1024;
constexpr int kShortSelThreads = 512;
constexpr int kShortCtx = 4096;
template <int NT>
constexpr int max_select_ctx() {
  return NT == kSelThreads ? PRHS_MAX_SELECT_CTX : kShortCtx;
}
constexpr double kMassScale = 1099511627776.0;  // 2^40

struct Pass {
  int shift;
  int bits;
};
constexpr Pass kPasses[3] = {{21, 11}, {10, 11}, {0, 10}};

__device__ __forceinline__ float key_to_score(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ unsigned long long mass_fx(uint32_t key, float lse) {
  const float a = __expf(key_to_score(key) - lse);
  return (unsigned long long)__builtin_fmaf(a, (float)kMassScale, 0.5f);
}

// Register-resident keys of one thread. Key j = v*GR + e sits at index
// w*64*KPT + v*64*GR + lane*GR + e (wave w, lane `lane`).
template <int KPT>
struct Keys {
  static constexpr int GR = KPT >= 4 ? 4 : KPT;
  static constexpr int NV = KPT / GR;
  uint32_t k[KPT];
  unsigned long long valid;
};

template <int KPT>
__device__ __forceinline__ int key_index(int w, int lane, int j) {
  constexpr int GR = Keys<KPT>::GR;
  return w * kWave * KPT + (j / GR) * kWave * GR + lane * GR + (j % GR);
}

template <int NT, bool MASS>
struct SelShared {
  uint32_t hist[kBins * kRep1];
  typename std::conditional<MASS, unsigned long long[kBins], char>::type mhist;
  // (key, index) of the fast path; key only otherwise; + dummies. Also the
  // waves' transpose tiles while a skipped score row is recomputed.
  __align__(16) uint2 cand[kCandCap + kWave];
  uint32_t gt_bits[kMaxWords];
  uint32_t eq_bits[kMaxWords];
  uint32_t wtot[NT / kWave];
  uint32_t wtot2[NT / kWave];
  unsigned long long wmass[NT / kWave];
  float lse;                      // dense log-sum-exp merged from the scan partials
  float qnorm;                    // |q| of the head, for the threshold hint
  uint32_t ncand;                 // candidate list length (keys and indices)
  uint32_t ncand_r;               // boundary-bin list length of the streamed searches (keys only)
  uint32_t kmax;
  uint32_t kmin;
  uint32_t digit;
  uint32_t above;
  uint32_t cT;
  uint32_t rT;                    // boundary key and its take from a ranked boundary bin
  uint32_t rTake;
  int found;
  unsigned long long below;
  unsigned long long mT;
};

__device__ __forceinline__ int hist_slot(int p, uint32_t dig, int lane) {
  return p == 0 ? (int)dig * kRep1 + (lane & (kRep1 - 1)) : (int)dig;
}

// Read a bin's count (summing the copies of the first pass) and clear it.
__device__ __forceinline__ uint32_t take_bin(uint32_t* hist, int p, int b) {
  if (p == 0) {
    uint4* q = reinterpret_cast<uint4*>(hist + b * kRep1);
    const uint4 a = *q;
    *q = make_uint4(0, 0, 0, 0);
    return a.x + a.y + a.z + a.w;
  }
  const uint32_t c = hist[b];
  hist[b] = 0;
  return c;
}

// Where the keys of a search come from: the first n entries of the LDS list
// (key in .x), or the score row itself, streamed (L2-resident after the
// first read). Only the fallback paths stream; they then hold no keys in
// registers, which keeps the kernel free of spills.
struct Src {
  const float* row;  // non-NULL: row[0:n]; NULL: the LDS list
  int n;
};

__device__ __forceinline__ uint32_t src_key(const Src& src, const uint2* cand, int c) {
  return src.row != nullptr ? score_key(src.row[c]) : cand[c].x;
}

// Atomics of pass p over the source keys >= klo matching (pre, pmask).
template <int NT, bool MASS>
__device__ __forceinline__ void hist_pass(const Src& src, int p, uint32_t pre, uint32_t pmask,
                                          float lse, SelShared<NT, MASS>& sh, uint32_t klo = 0) {
  const int shift = kPasses[p].shift;
  const uint32_t dmask = (1u << kPasses[p].bits) - 1u;
  const int lane = threadIdx.x & (kWave - 1);
  for (int c = threadIdx.x; c < src.n; c += NT) {
    const uint32_t key = src_key(src, sh.cand, c);
    if ((key & pmask) == pre && key >= klo) {
      const uint32_t dig = (key >> shift) & dmask;
      atomicAdd(&sh.hist[hist_slot(p, dig, lane)], 1u);
      if constexpr (MASS) atomicAdd(&sh.mhist[dig], mass_fx(key, lse));
    }
  }
  __syncthreads();
}

// Locate the bin holding the krem-th largest key of pass p (bins in
// descending order; thread i owns bins nb-1-(BPT*i+k)). Clears the bins.
template <int NT, bool MASS>
__device__ __forceinline__ void find_count(int p, uint32_t krem, SelShared<NT, MASS>& sh) {
  constexpr int NW = NT / kWave;
  constexpr int BPT = kBins / NT;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int nb = 1 << kPasses[p].bits;
  uint32_t c[BPT];
  uint32_t local = 0;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int b = nb - 1 - (BPT * (int)threadIdx.x + k);
    c[k] = b >= 0 ? take_bin(sh.hist, p, b) : 0u;
    local += c[k];
  }
  if constexpr (MASS) {
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int b = nb - 1 - (BPT * (int)threadIdx.x + k);
      if (b >= 0) sh.mhist[b] = 0;
    }
  }
  const uint32_t incl = wave_scan_u32(local);
  if (lane == kWave - 1) sh.wtot[w] = incl;
  __syncthreads();
  uint32_t before = 0;
  int wb = NW;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    const uint32_t x = sh.wtot[u];
    if (wb == NW) {
      if (before + x >= krem) wb = u;
      else before += x;
    }
  }
  if (w == wb) {
    uint32_t acc = before + incl - local;
    if (acc < krem && krem <= acc + local) {
#pragma unroll
      for (int k = 0; k < BPT; ++k) {
        if (acc < krem && krem <= acc + c[k]) {
          sh.digit = (uint32_t)(nb - 1 - (BPT * (int)threadIdx.x + k));
          sh.above = acc;
          sh.cT = c[k];
        }
        acc += c[k];
      }
    }
  }
  __syncthreads();
}

// Locate the bin, walking up from the smallest keys, where the suffix mass
// first exceeds drem (bins ascending; thread i owns bins BPT*i+k). Clears
// the bins. sh.found = 0 when the whole region's mass is within drem.
template <int NT>
__device__ __forceinline__ void find_mass(int p, unsigned long long drem, SelShared<NT, true>& sh) {
  constexpr int NW = NT / kWave;
  constexpr int BPT = kBins / NT;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int nb = 1 << kPasses[p].bits;
  uint32_t c[BPT];
  unsigned long long m[BPT];
  uint32_t lc = 0;
  unsigned long long lm = 0;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int b = BPT * (int)threadIdx.x + k;
    c[k] = b < nb ? take_bin(sh.hist, p, b) : 0u;
    m[k] = 0;
    if (b < nb) {
      m[k] = sh.mhist[b];
      sh.mhist[b] = 0;
    }
    lc += c[k];
    lm += m[k];
  }
  const uint32_t cinc = wave_scan_u32(lc);
  const unsigned long long minc = wave_inclusive_scan(lm);
  if (lane == kWave - 1) {
    sh.wtot[w] = cinc;
    sh.wmass[w] = minc;
  }
  if (threadIdx.x == 0) sh.found = 0;
  __syncthreads();
  unsigned long long mbefore = 0;
  uint32_t cbefore = 0, ctot = 0;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    ctot += sh.wtot[u];
    if (u < w) {
      mbefore += sh.wmass[u];
      cbefore += sh.wtot[u];
    }
  }
  unsigned long long mex = mbefore + minc - lm;
  uint32_t cex = cbefore + cinc - lc;
  if (mex <= drem && drem < mex + lm) {
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      if (mex <= drem && drem < mex + m[k]) {
        sh.found = 1;
        sh.digit = (uint32_t)(BPT * (int)threadIdx.x + k);
        sh.below = mex;
        sh.above = ctot - (cex + c[k]);
        sh.cT = c[k];
        sh.mT = m[k];
      }
      mex += m[k];
      cex += c[k];
    }
  }
  __syncthreads();
}

// Copy the row's keys >= klo matching (pre, pmask) into the LDS list (keys
// only, in no particular order); sh.ncand_r becomes their number. The caller
// knows that they fit.
template <int NT, bool MASS>
__device__ __forceinline__ void compact_row(const float* __restrict__ row, int t, uint32_t pre,
                                            uint32_t pmask, uint32_t klo,
                                            SelShared<NT, MASS>& sh) {
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x == 0) sh.ncand_r = 0;
  __syncthreads();
  for (int c0 = 0; c0 < t; c0 += NT) {  // whole waves iterate together
    const int c = c0 + (int)threadIdx.x;
    const uint32_t key = c < t ? score_key(row[c]) : 0u;
    const bool h = c < t && (key & pmask) == pre && key >= klo;
    const unsigned long long m = __ballot(h);
    if (m) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&sh.ncand_r, (uint32_t)__popcll(m));
      base = lane_read(base, 0);
      const uint32_t pos = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
      PRHS_CHECK(!h || pos < (uint32_t)kCandCap, kCheckList);  // the caller knows they fit
    if (h && pos < (uint32_t)kCandCap) sh.cand[pos].x = key;
    }
  }
  __syncthreads();
}

// Exact boundary of the krem-th largest key of the row. Returns T; krem
// becomes the number of keys equal to T that are taken.
template <int NT, bool MASS>
__device__ __forceinline__ uint32_t count_search(const float* __restrict__ row, int t,
                                                 uint32_t& krem, SelShared<NT, MASS>& sh) {
  uint32_t pre = 0, pmask = 0;
  Src src{row, t};
  hist_pass<NT, MASS>(src, 0, pre, pmask, 0.f, sh);
  find_count<NT, MASS>(0, krem, sh);
  krem -= sh.above;
  pre = sh.digit << kPasses[0].shift;
  pmask = (uint32_t)(kBins - 1) << kPasses[0].shift;
  if (sh.cT <= (uint32_t)kCandCap) {
    compact_row<NT, MASS>(row, t, pre, pmask, 0u, sh);
    src = Src{nullptr, (int)sh.ncand_r};
  }
#pragma unroll 1
  for (int p = 1; p < 3; ++p) {
    hist_pass<NT, MASS>(src, p, pre, pmask, 0.f, sh);
    find_count<NT, MASS>(p, krem, sh);
    krem -= sh.above;
    pre |= sh.digit << kPasses[p].shift;
    pmask |= (uint32_t)((1 << kPasses[p].bits) - 1) << kPasses[p].shift;
  }
  return pre;
}

// Mass search (DELTA) over the source keys >= klo: the boundary key T where
// the suffix mass (a key and everything ranked below it, down to klo) first
// exceeds drem, walking up from the smallest key. A streamed row is compacted
// to the LDS list after the first pass when the boundary bin fits. Returns
// false when the mass of all keys >= klo is within drem. Otherwise n_above is
// the number of keys above T and take_T the number of keys equal to T that
// are taken.
template <int NT>
__device__ __forceinline__ bool mass_search(Src src, float lse, unsigned long long drem,
                                            uint32_t klo, uint32_t& T, uint32_t& n_above,
                                            uint32_t& take_T, SelShared<NT, true>& sh) {
  uint32_t pre = 0, pmask = 0;
  n_above = 0;
#pragma unroll 1
  for (int p = 0; p < 3; ++p) {
    hist_pass<NT, true>(src, p, pre, pmask, lse, sh, klo);
    find_mass<NT>(p, drem, sh);
    if (!sh.found) return false;
    drem -= sh.below;
    n_above += sh.above;
    pre |= sh.digit << kPasses[p].shift;
    pmask |= (uint32_t)((1 << kPasses[p].bits) - 1) << kPasses[p].shift;
    if (p == 0 && src.row != nullptr && sh.cT <= (uint32_t)kCandCap) {
      compact_row<NT, true>(src.row, src.n, pre, pmask, klo, sh);
      src = Src{nullptr, (int)sh.ncand_r};
    }
  }
  // Boundary key T = pre: its c_T keys carry identical mass a each. The key
  // of rank j (by index) among them is taken while its suffix mass
  // (c_T - j + 1) * a exceeds drem.
  const uint32_t cT = sh.cT;
  const unsigned long long a = sh.mT / cT;
  const unsigned long long keep_out = a ? drem / a : (unsigned long long)cT;
  take_T = cT - (keep_out < cT ? (uint32_t)keep_out : cT);
  T = pre;
  return true;
}

// Block sums over the source keys: the mass of the keys below T (BELOW) or at
// or above T, and the number of keys equal to T.
template <int NT, bool BELOW>
__device__ __forceinline__ void mass_split(const Src& src, uint32_t T, float lse,
                                           unsigned long long& mass, uint32_t& n_eq,
                                           SelShared<NT, true>& sh) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  unsigned long long m = 0;
  uint32_t e = 0;
  for (int c = threadIdx.x; c < src.n; c += NT) {
    const uint32_t key = src_key(src, sh.cand, c);
    if (BELOW ? key < T : key >= T) m += mass_fx(key, lse);
    e += key == T;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    m += __shfl_xor(m, o);
    e += __shfl_xor(e, o);
  }
  if (lane == 0) {
    sh.wmass[w] = m;
    sh.wtot[w] = e;
  }
  __syncthreads();
  mass = 0;
  n_eq = 0;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    mass += sh.wmass[u];
    n_eq += sh.wtot[u];
  }
  __syncthreads();
}

// Mark the row's keys above T and equal to T in the LDS bitmaps.
template <int NT, bool MASS>
__device__ __forceinline__ void mark_row(const float* __restrict__ row, int t, uint32_t T,
                                         SelShared<NT, MASS>& sh) {
  for (int i = threadIdx.x; i < t; i += NT) {
    const uint32_t key = score_key(row[i]);
    if (key > T) atomicOr(&sh.gt_bits[i >> 5], 1u << (i & 31));
    else if (key == T) atomicOr(&sh.eq_bits[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
}

// Final selection of every bitmap word -- the keys above T plus the first
// take_eq keys equal to T in index order -- and the word's exclusive output
// offset, stored in place of gt_bits and eq_bits. Thread i owns WPT
// consecutive words.
template <int NT, bool MASS>
__device__ __forceinline__ void emit_offsets(int t, uint32_t take_eq, SelShared<NT, MASS>& sh,
                                             uint32_t out_base = 0u, uint32_t* n_out = nullptr,
                                             uint32_t* n_eq_taken = nullptr) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int nwords = (t + 31) >> 5;
  constexpr int WPT = (kMaxWords + NT - 1) / NT;
  uint32_t g[WPT], e[WPT];
  uint32_t ng = 0, ne = 0;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    const int wi = (int)threadIdx.x * WPT + q;
    g[q] = wi < nwords ? sh.gt_bits[wi] : 0u;
    e[q] = wi < nwords ? sh.eq_bits[wi] : 0u;
    ng += __popc(g[q]);
    ne += __popc(e[q]);
  }
  const uint32_t ginc = wave_scan_u32(ng);
  const uint32_t einc = wave_scan_u32(ne);
  if (lane == kWave - 1) {
    sh.wtot[w] = ginc;
    sh.wtot2[w] = einc;
  }
  __syncthreads();
  uint32_t gb = ginc - ng, eb = einc - ne, gtot = 0, etot = 0;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    if (u < w) {
      gb += sh.wtot[u];
      eb += sh.wtot2[u];
    }
    gtot += sh.wtot[u];
    etot += sh.wtot2[u];
  }
  if (n_out != nullptr) {
    // selected in this range: every key above T and the equal ones still due
    *n_eq_taken = etot < take_eq ? etot : take_eq;
    *n_out = gtot + *n_eq_taken;
  }
  uint32_t pos = out_base + gb + (eb < take_eq ? eb : take_eq);
  uint32_t eq_left = take_eq > eb ? take_eq - eb : 0u;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    uint32_t sel = g[q];
    uint32_t ew = e[q];
    while (eq_left && ew) {
      const uint32_t low = ew & (0u - ew);
      sel |= low;
      ew ^= low;
      --eq_left;
    }
    const int wi = (int)threadIdx.x * WPT + q;
    if (wi < nwords) {
      sh.gt_bits[wi] = sel;
      sh.eq_bits[wi] = pos;
    }
    pos += __popc(sel);
  }
  __syncthreads();
}

// Output slot of key index i, or -1 when it is not selected (after emit_offsets).
template <int NT, bool MASS>
__device__ __forceinline__ int out_slot(uint32_t i, const SelShared<NT, MASS>& sh) {
  const uint32_t m = sh.gt_bits[i >> 5];
  const uint32_t bit = i & 31u;
  if (!((m >> bit) & 1u)) return -1;
  return (int)(sh.eq_bits[i >> 5] + __popc(m & ((1u << bit) - 1u)));
}

// Write one selected entry to its slot, and to the LDS mirror of the fused
// decode (index, score bits) when there is one.
__device__ __forceinline__ void put_sel(int* __restrict__ out, float* __restrict__ out_s,
                                        uint2* mirror, uint32_t pos, uint32_t i, float s) {
  out[pos] = (int)i;
  if (out_s) out_s[pos] = s;
  if (mirror != nullptr && pos < (uint32_t)kFuseRows) mirror[pos] = make_uint2(i, __float_as_uint(s));
}

// Write the selected entries of the LDS list (key, index) to their slots.
template <int NT, bool MASS>
__device__ __forceinline__ void scatter_list(uint32_t C, int* __restrict__ out,
                                             float* __restrict__ out_s, uint32_t cap,
                                             const SelShared<NT, MASS>& sh, uint2* mirror) {
  for (int c = threadIdx.x; c < (int)C; c += NT) {
    const uint2 ki = sh.cand[c];
    const int pos = out_slot<NT, MASS>(ki.y, sh);
    if (pos >= 0 && (uint32_t)pos < cap) put_sel(out, out_s, mirror, pos, ki.y, key_to_score(ki.x));
  }
}

// Write the row's selected keys to their slots.
// Write the row's selected keys to their slots. `row` and the bitmaps start at
// key index i0 (a tile of a longer row).
template <int NT, bool MASS>
__device__ __forceinline__ void scatter_row(const float* __restrict__ row, int t,
                                            int* __restrict__ out, float* __restrict__ out_s,
                                            uint32_t cap, const SelShared<NT, MASS>& sh,
                                            uint2* mirror, int i0 = 0) {
  for (int i = threadIdx.x; i < t; i += NT) {
    const int pos = out_slot<NT, MASS>((uint32_t)i, sh);
    if (pos >= 0 && (uint32_t)pos < cap)
      put_sel(out, out_s, mirror, pos, (uint32_t)(i0 + i), key_to_score(score_key(row[i])));
  }
}

// The streamed row's selection in tiles of kTileKeys positions: each tile's
// bitmaps are cleared, marked and turned into offsets that continue the
// previous tiles' output count and their count of keys equal to T taken.
template <int NT, bool MASS>
__device__ __forceinline__ void emit_row_tiled(const float* __restrict__ row, int t, uint32_t T,
                                               uint32_t take_eq, int* __restrict__ out,
                                               float* __restrict__ out_s, uint32_t cap,
                                               SelShared<NT, MASS>& sh, uint2* mirror) {
  uint32_t out_base = 0, eq_left = take_eq;
  for (int t0 = 0; t0 < t; t0 += kTileKeys) {
    const int tt = t - t0 < kTileKeys ? t - t0 : kTileKeys;
    const int nw = (tt + 31) >> 5;
    __syncthreads();  // the previous tile's scatter has read the bitmaps
    for (int i = threadIdx.x; i < nw; i += NT) {
      sh.gt_bits[i] = 0;
      sh.eq_bits[i] = 0;
    }
    __syncthreads();
    mark_row<NT, MASS>(row + t0, tt, T, sh);
    uint32_t n_out = 0, n_eq = 0;
    emit_offsets<NT, MASS>(tt, eq_left, sh, out_base, &n_out, &n_eq);
    scatter_row<NT, MASS>(row + t0, tt, out, out_s, cap, sh, mirror, t0);
    out_base += n_out;
    eq_left -= n_eq;
  }
}

// The row's top key into sh.kmax, streamed (for rows whose keys the registers
// do not hold).
template <int NT, bool MASS>
__device__ __forceinline__ void stream_kmax(const float* __restrict__ row, int t,
                                            SelShared<NT, MASS>& sh) {
  if (threadIdx.x == 0) sh.kmax = 0;
  __syncthreads();
  uint32_t kmx = 0;
  for (int i = threadIdx.x; i < t; i += NT) {
    const uint32_t key = score_key(row[i]);
    kmx = key > kmx ? key : kmx;
  }
  kmx = wave_max_u32(kmx);
  if ((threadIdx.x & (kWave - 1)) == 0) atomicMax(&sh.kmax, kmx);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// TOPN fast path: sampled threshold, compacted candidates, 12-bit passes.
// ---------------------------------------------------------------------------

// Histogram layout of the one-wave find: NB bins, REP copies each. Lane l of
// the finding wave owns bins [NB - (l+1)*BPL, NB - l*BPL); bin b is stored at
// word ((b % BPL) * 64 + b / BPL) * REP, so that the lanes' k-th bins are
// adjacent words and every read of the find is free of bank conflicts.
template <int NB, int REP>
__device__ __forceinline__ int swz_slot(uint32_t b, int lane) {
  constexpr int BPL = NB / kWave;
  return ((int)(b % BPL) * kWave + (int)(b / BPL)) * REP + (REP > 1 ? (lane & (REP - 1)) : 0);
}

template <int NB, int REP>
__device__ __forceinline__ uint32_t swz_bin(const uint32_t* hist, int b) {
  constexpr int BPL = NB / kWave;
  const int w0 = ((b % BPL) * kWave + b / BPL) * REP;
  if constexpr (REP == 4) {
    const uint4 a = *reinterpret_cast<const uint4*>(hist + w0);
    return a.x + a.y + a.z + a.w;
  } else {
    return hist[w0];
  }
}

// Wave 0 locates, over NB bins taken in descending order, the bin holding the
// krem-th largest; it clears every bin. The result goes to sh.digit / above /
// cT (left unchanged when the bins hold fewer than krem keys).
template <int NB, int REP, int NT, bool MASS>
__device__ __forceinline__ void find_count_w0(uint32_t krem, SelShared<NT, MASS>& sh) {
  constexpr int BPL = NB / kWave;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int col = kWave - 1 - lane;  // = b / BPL for this lane's bins
    uint32_t local = 0;
#pragma unroll
    for (int k = 0; k < BPL; ++k) {
      const int w0 = (k * kWave + col) * REP;
      if constexpr (REP == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(sh.hist + w0);
        local += a.x + a.y + a.z + a.w;
      } else {
        local += sh.hist[w0];
      }
    }
    const uint32_t incl = wave_scan_u32(local);
    const uint32_t excl = incl - local;
    // the lane whose range crosses krem (at most one), then its bins one per lane
    const unsigned long long cross = __ballot(excl < krem && krem <= incl);
    if (cross) {
      const int L = __builtin_ctzll(cross);
      const uint32_t baseL = lane_read(excl, L);
      const int b = NB - (L + 1) * BPL + (BPL - 1 - lane);
      const uint32_t c = lane < BPL ? swz_bin<NB, REP>(sh.hist, b) : 0u;
      const uint32_t ce = wave_scan_u32(c) - c + baseL;
      if (lane < BPL && ce < krem && krem <= ce + c) {
        sh.digit = (uint32_t)b;
        sh.above = ce;
        sh.cT = c;
      }
    }
#pragma unroll
    for (int k = 0; k < BPL; ++k) {
      const int w0 = (k * kWave + col) * REP;
      if constexpr (REP == 4) *reinterpret_cast<uint4*>(sh.hist + w0) = make_uint4(0, 0, 0, 0);
      else sh.hist[w0] = 0;
    }
  }
  __syncthreads();
}

// Exact N-th largest key among the C candidate keys in sh.cand[].x, all of
// them in [lo, hi]: radix passes with 10-bit digits of key - lo until the
// boundary bin holds at most 64 keys (or no digits are left). Those keys are
// then compacted past the list and ranked by one wave, lane against lane.
// Returns the boundary key T and take_eq, the number of keys equal to T that
// are taken.
template <int NT, bool MASS>
__device__ __forceinline__ void cand_radix(uint32_t lo, uint32_t hi, uint32_t C, uint32_t N,
                                           uint32_t& T, uint32_t& take_eq,
                                           SelShared<NT, MASS>& sh) {
  constexpr int DB = 10, NB = 1 << DB;
  const uint32_t range = hi - lo;
  int shift = range ? 32 - __builtin_clz(range) - DB : 0;
  shift = shift > 0 ? shift : 0;
  uint32_t pre = 0, pmask = 0, krem = N;
#pragma unroll 1
  while (true) {
    if (threadIdx.x == 0) sh.ncand_r = 0;
    for (int c = threadIdx.x; c < (int)C; c += NT) {
      const uint32_t o = sh.cand[c].x - lo;
      if ((o & pmask) == pre)
        atomicAdd(&sh.hist[swz_slot<NB, 1>((o >> shift) & (uint32_t)(NB - 1), 0)], 1u);
    }
    __syncthreads();
    // 1 <= krem <= the keys counted, so the find always sets digit / above / cT
    find_count_w0<NB, 1, NT, MASS>(krem, sh);
    krem -= sh.above;
    pre |= sh.digit << shift;
    pmask |= (uint32_t)(NB - 1) << shift;
    if (shift == 0) break;
    if (sh.cT <= (uint32_t)kWave) {
      // the boundary bin's keys, ranked directly
      for (int c = threadIdx.x; c < (int)C; c += NT) {
        const uint32_t key = sh.cand[c].x;
        if (((key - lo) & pmask) == pre) sh.cand[kCandCap + atomicAdd(&sh.ncand_r, 1u)].x = key;
      }
      __syncthreads();
      if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        const int n = (int)sh.cT;
        const uint32_t x = lane < n ? sh.cand[kCandCap + lane].x : 0u;
        uint32_t gt = 0, eq = 0;
        for (int j = 0; j < n; ++j) {
          const uint32_t y = lane_read(x, j);
          gt += y > x;
          eq += y == x;
        }
        // lanes holding the same key write the same values
        if (lane < n && gt < krem && krem <= gt + eq) {
          sh.rT = x;
          sh.rTake = krem - gt;
        }
      }
      __syncthreads();
      T = sh.rT;
      take_eq = sh.rTake;
      return;
    }
    shift = shift > DB ? shift - DB : 0;
  }
  T = lo + pre;
  take_eq = krem;
}

// Sampled threshold: pick theta so that at least N keys clear it with a wide
// margin and compact the keys >= theta with their indices into sh.cand
// (sh.ncand of them, sh.kmax their largest). Returns false when the list does
// not hold between N and kCandCap keys; theta is returned in `theta`.
template <int KPT, int NT, bool MASS>
__device__ __forceinline__ bool build_candidates(const Keys<KPT>& K, int t, uint32_t N,
                                                 uint32_t& theta_key, SelShared<NT, MASS>& sh) {
  constexpr int SR = KPT >= 8 ? 8 : 1;  // sample one key in SR
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  uint32_t theta = 0;
  // sample whenever the list would otherwise hold far more keys than needed
  if (t > kCandCap || (SR > 1 && (uint32_t)t >= 8u * N)) {
    if (threadIdx.x == 0) {
      sh.digit = 0;
      sh.ncand = 0;
      sh.kmax = 0;
    }
#pragma unroll
    for (int j = 0; j < KPT; j += SR) {
      if ((K.valid >> j) & 1ull)
        atomicAdd(&sh.hist[swz_slot<kBins, kRep1>(K.k[j] >> 21, lane)], 1u);
    }
    __syncthreads();
    // enough sampled keys above the bin edge for N keys with a margin of
    // about two binomial standard deviations
    const float ns = (float)N / SR;
    const uint32_t target = (uint32_t)(ns + 2.f * sqrtf(ns) + 8.f);
    find_count_w0<kBins, kRep1, NT, MASS>(target, sh);
    theta = sh.digit << 21;
  } else {
    if (threadIdx.x == 0) {
      sh.ncand = 0;
      sh.kmax = 0;
    }
    __syncthreads();
  }
  // compact the keys >= theta with their indices; lanes without a hit write
  // their own dummy slot past the list, so the loop has no branches
  using Mask = typename std::conditional<(KPT > 32), unsigned long long, uint32_t>::type;
  Mask hit = 0;
  uint32_t kmx = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool h = ((K.valid >> j) & 1ull) && K.k[j] >= theta;
    hit |= (Mask)h << j;
    kmx = h && K.k[j] > kmx ? K.k[j] : kmx;
  }
  const uint32_t cnt = (uint32_t)__builtin_popcountll(hit);
  const uint32_t incl = wave_scan_u32(cnt);
  const uint32_t wtotal = lane_read(incl, kWave - 1);
  kmx = wave_max_u32(kmx);
  uint32_t base = 0;
  if (lane == 0 && wtotal) {
    base = atomicAdd(&sh.ncand, wtotal);
    atomicMax(&sh.kmax, kmx);
  }
  uint32_t pos = lane_read(base, 0) + incl - cnt;
  const uint32_t dummy = (uint32_t)kCandCap + (uint32_t)lane;
  const int ibase = key_index<KPT>(w, lane, 0);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool h = (hit >> j) & 1;
    const uint32_t slot = (h && pos < (uint32_t)kCandCap) ? pos : dummy;
    sh.cand[slot] = make_uint2(K.k[j], (uint32_t)(ibase + (j / Keys<KPT>::GR) * kWave * Keys<KPT>::GR + (j % Keys<KPT>::GR)));
    pos += h;
  }
  __syncthreads();
  theta_key = theta;
  const uint32_t C = sh.ncand;
  return C >= N && C <= (uint32_t)kCandCap;
}

// Mark the list entries above T and equal to T in the LDS bitmaps.
template <int NT, bool MASS>
__device__ __forceinline__ void mark_from_list(uint32_t C, uint32_t T, SelShared<NT, MASS>& sh) {
  for (int c = threadIdx.x; c < (int)C; c += NT) {
    const uint2 ki = sh.cand[c];
    if (ki.x > T) atomicOr(&sh.gt_bits[ki.y >> 5], 1u << (ki.y & 31));
    else if (ki.x == T) atomicOr(&sh.eq_bits[ki.y >> 5], 1u << (ki.y & 31));
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// TOPN from the scan's candidates (keys >= a per-head threshold hint).
// ---------------------------------------------------------------------------

// Write the candidates above T and the first take_eq equal to T, in the list's
// (index) order, with their scores. Thread i owns a contiguous block of the list.
template <int NT, bool MASS>
__device__ __forceinline__ void emit_list(uint32_t C, uint32_t T, uint32_t take_eq,
                                          int* __restrict__ out, float* __restrict__ out_s,
                                          uint32_t cap, SelShared<NT, MASS>& sh, uint2* mirror) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const uint32_t cpt = (C + NT - 1) / NT;
  const uint32_t beg = threadIdx.x * cpt;
  const uint32_t end = beg + cpt < C ? beg + cpt : C;
  uint32_t ng = 0, ne = 0;
  for (uint32_t c = beg; c < end; ++c) {
    const uint32_t key = sh.cand[c].x;
    ng += key > T;
    ne += key == T;
  }
  const uint32_t ginc = wave_scan_u32(ng);
  const uint32_t einc = wave_scan_u32(ne);
  if (lane == kWave - 1) {
    sh.wtot[w] = ginc;
    sh.wtot2[w] = einc;
  }
  __syncthreads();
  uint32_t gb = ginc - ng, eb = einc - ne;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    if (u < w) {
      gb += sh.wtot[u];
      eb += sh.wtot2[u];
    }
  }
  uint32_t pos = gb + (eb < take_eq ? eb : take_eq);
  uint32_t eq_left = take_eq > eb ? take_eq - eb : 0u;
  for (uint32_t c = beg; c < end; ++c) {
    const uint2 ki = sh.cand[c];
    bool sel = ki.x > T;
    if (ki.x == T && eq_left) {
      sel = true;
      --eq_left;
    }
    if (sel) {
      if (pos < cap) put_sel(out, out_s, mirror, pos, ki.y, key_to_score(ki.x));
      ++pos;
    }
  }
}

// Candidate chunks per wave: wave w owns chunks [w * cpw, (w + 1) * cpw) and
// lane l < cpw loads the count of chunk w * cpw + l at kernel start.
template <int NT>
__device__ __forceinline__ int cand_cpw(int nch) {
  return (nch + NT / kWave - 1) / (NT / kWave);
}

// Compact the scan's candidates of one head (keys >= its threshold hint, per
// chunk in index order) into sh.cand in index order, with their keys, and set
// sh.kmax / sh.kmin. `c` is this lane's chunk count (see cand_cpw). Each wave
// requests the first entries of its own chunks as soon as its counts are in,
// without waiting for the other waves: kSlots loads per lane cover R = 64-lane
// rows of every chunk (R = kSlots / cpw, at most the chunk's 4 rows); rows past
// that are fetched afterwards. The workgroup offsets are formed while those
// loads are in flight. Returns false (nothing written) when a chunk has no
// candidate list or the total is below N or above the LDS list capacity.
constexpr int kSlots = 16;
template <int NT, bool MASS>
__device__ __forceinline__ bool gather_candidates(const uint2* __restrict__ cand, uint32_t c,
                                                  int head, int nch, uint32_t N, uint32_t& C,
                                                  SelShared<NT, MASS>& sh) {
  constexpr int NW = NT / kWave;
  static_assert((max_select_ctx<NT>() / kScoreChunk + NW - 1) / NW <= kWave,
                "one lane per chunk count in a wave");
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int cpw = cand_cpw<NT>(nch);
  int rows = 1;  // 64-entry rows requested per chunk in the first round
  while (rows < 4 && rows * 2 * cpw <= kSlots) rows *= 2;
  // the wave's chunks start at a wave-uniform address: one scalar base, and a
  // 32-bit lane offset per load
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint2* src = cand + ((size_t)head * nch + (size_t)wu * cpw) * kScoreChunk;
  uint2 e[kSlots];
  // Up to 4K keys (one chunk per wave of the 1024-thread workgroup, two per
  // wave of the 512-thread one; all four rows of each in the first round) the
  // wave requests its whole chunks before their counts are in: 2 or 4 KiB per
  // wave read ahead, one dependent round trip saved. Slots past a count hold
  // stale entries and are never used.
  const bool ahead = cpw <= (NT == kShortSelThreads ? 2 : 1) && rows == 4;
  if (ahead) {
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int k = sl / 4, r = sl - k * 4;
      e[sl] = make_uint2(0u, 0u);
      if (k < cpw && wu * cpw + k < nch)
        e[sl] = src[(uint32_t)(k * kScoreChunk + lane + r * kWave)];
    }
  }
  const bool bad = __ballot(c == kNoCand) != 0ull;
  const uint32_t cc = c == kNoCand ? 0u : c;
  const uint32_t inc = wave_scan_u32(cc);
  const uint32_t ex = inc - cc;
  if (!ahead) {
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int k = sl / rows, r = sl - k * rows;
      e[sl] = make_uint2(0u, 0u);
      if (k < cpw) {
        const uint32_t j = (uint32_t)(lane + r * kWave);
        if (j < lane_read(cc, k)) e[sl] = src[(uint32_t)k * kScoreChunk + j];
      }
    }
  }
  if (lane == kWave - 1) {
    sh.wtot[w] = inc;
    sh.wtot2[w] = bad ? 1u : 0u;
  }
  __syncthreads();
  uint32_t base = 0, total = 0, anybad = 0;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    const uint32_t v = sh.wtot[u];
    if (u < w) base += v;
    total += v;
    anybad |= sh.wtot2[u];
  }
  if (threadIdx.x == 0) {
    sh.kmax = 0;
    sh.kmin = 0xFFFFFFFFu;
  }
  __syncthreads();  // every wave has read wtot; kmax / kmin are reset
  C = total;
  if (anybad || C < N || C > (uint32_t)kCandCap) return false;
  uint32_t kmx = 0, kmn = 0xFFFFFFFFu;
#pragma unroll
  for (int sl = 0; sl < kSlots; ++sl) {
    const int k = sl / rows, r = sl - k * rows;
    if (k < cpw) {
      const uint32_t j = (uint32_t)(lane + r * kWave);
      if (j < lane_read(cc, k)) {
        const uint32_t key = score_key(__uint_as_float(e[sl].x));
        sh.cand[base + lane_read(ex, k) + j] = make_uint2(key, e[sl].y);
        kmx = key > kmx ? key : kmx;
        kmn = key < kmn ? key : kmn;
      }
    }
  }
  // chunks past the first round's kSlots (more than 16 chunks per wave, i.e.
  // contexts beyond 64K): their first 64-entry rows, kSlots chunks per round
  const int first = kSlots / rows;  // chunks the first round covered
  for (int k0 = first; k0 < cpw; k0 += kSlots) {
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int k = k0 + sl;
      e[sl] = make_uint2(0u, 0u);
      if (k < cpw && (uint32_t)lane < lane_read(cc, k < cpw ? k : 0))
        e[sl] = src[(uint32_t)k * kScoreChunk + (uint32_t)lane];
    }
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int k = k0 + sl;
      if (k < cpw && (uint32_t)lane < lane_read(cc, k < cpw ? k : 0)) {
        const uint32_t key = score_key(__uint_as_float(e[sl].x));
        sh.cand[base + lane_read(ex, k) + (uint32_t)lane] = make_uint2(key, e[sl].y);
        kmx = key > kmx ? key : kmx;
        kmn = key < kmn ? key : kmn;
      }
    }
  }
  // rows past the first 64-entry row (or past the first round's rows)
  for (int k = 0; k < cpw; ++k) {
    const uint32_t n = lane_read(cc, k);
    const int done = k < first ? rows : 1;
    for (uint32_t j = (uint32_t)(lane + done * kWave); j < n; j += kWave) {
      const uint2 x = src[(size_t)k * kScoreChunk + j];
      const uint32_t key = score_key(__uint_as_float(x.x));
      sh.cand[base + lane_read(ex, k) + j] = make_uint2(key, x.y);
      kmx = key > kmx ? key : kmx;
      kmn = key < kmn ? key : kmn;
    }
  }
  kmx = wave_max_u32(kmx);
  kmn = wave_min_u32(kmn);
  if (lane == 0) {
    atomicMax(&sh.kmax, kmx);
    atomicMin(&sh.kmin, kmn);
  }
  __syncthreads();
  return true;
}

// Threshold hint for the next step of the same head: the boundary score less
// a margin that grows with the spread between the top score and the boundary,
// divided by the query norm (scores scale with |q| at a fixed direction, so
// the next scan multiplies it by its own query's norm). A zero norm gives NaN:
// no hint.
__device__ __forceinline__ float next_theta(uint32_t T, uint32_t kmax, float qnorm) {
  const float ts = key_to_score(T), ms = key_to_score(kmax);
  const float spread = ms - ts;
  const float th = ts - (0.1f * (spread > 0.f ? spread : 0.f) + 0.05f);
  return qnorm > 0.f ? th / qnorm : __builtin_nanf("");
}

// Load the head's scores (raw fp32 bits; finish_keys turns them into keys):
// wave w owns [w*64*KPT, (w+1)*64*KPT), lane `lane` the granules at
// w*64*KPT + v*64*GR + lane*GR. Split in two so that the loads stay in flight
// across unrelated work.
template <int KPT>
__device__ __forceinline__ void load_keys_raw(Keys<KPT>& K, const float* __restrict__ row, int t) {
  constexpr int GR = Keys<KPT>::GR, NV = Keys<KPT>::NV;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int base = w * kWave * KPT + lane * GR;
  if (GR == 4 && (w + 1) * kWave * KPT <= t) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint4 x = *reinterpret_cast<const uint4*>(row + base + v * kWave * GR);
      K.k[GR * v] = x.x;
      K.k[GR * v + 1 % GR] = x.y;
      K.k[GR * v + 2 % GR] = x.z;
      K.k[GR * v + 3 % GR] = x.w;
    }
    K.valid = KPT == 64 ? ~0ull : ((1ull << KPT) - 1ull);
    return;
  }
  K.valid = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int i = base + v * kWave * GR;
#pragma unroll
    for (int e = 0; e < GR; ++e) {
      const bool ok = i + e < t;
      K.k[v * GR + e] = ok ? __float_as_uint(row[i + e]) : 0u;
      if (ok) K.valid |= 1ull << (v * GR + e);
    }
  }
}

template <int KPT>
__device__ __forceinline__ void finish_keys(Keys<KPT>& K) {
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    K.k[j] = ((K.valid >> j) & 1ull) ? score_key(__uint_as_float(K.k[j])) : 0u;
}

template <int KPT>
__device__ __forceinline__ void load_keys(Keys<KPT>& K, const float* __restrict__ row, int t) {
  load_keys_raw<KPT>(K, row, t);
  finish_keys<KPT>(K);
}

// Write the selection once T and take are known and (up to kTileKeys
// positions) the bitmaps are marked:
// indices and scores in ascending index order, scattered from the LDS list
// (`list`) or from the streamed row, then the count, the cap flag and the
// threshold hint.
template <int NT, bool MASS>
__device__ __forceinline__ void finish_head(const SelectArgs& a, int head, const float* row,
                                            int* out, float* out_s, bool list, uint32_t C,
                                            uint32_t T, uint32_t take, int n_sel, int hit,
                                            SelShared<NT, MASS>& sh, uint2* mirror) {
  const uint32_t cap = (uint32_t)a.idx_cap;
  if (a.t > kTileKeys) {
    // longer rows are streamed (never listed): marked and emitted per tile
    emit_row_tiled<NT, MASS>(row, a.t, T, take, out, out_s, cap, sh, mirror);
  } else {
    emit_offsets<NT, MASS>(a.t, take, sh);
    if (list) scatter_list<NT, MASS>(C, out, out_s, cap, sh, mirror);
    else scatter_row<NT, MASS>(row, a.t, out, out_s, cap, sh, mirror);
  }
  if (threadIdx.x == 0) {
    a.count[head] = n_sel;
    if (a.cap_hit) a.cap_hit[head] = hit;
    if (!MASS && a.theta_out) a.theta_out[head] = next_theta(T, sh.kmax, sh.qnorm);
  }
}

// Fused decode: attention of one head over its own selection, read from the
// LDS mirror (index, score) that the emission filled in index order. Wave w
// gathers the fp16 V rows (128 wide, 16 lanes of 16 bytes per row) of a
// contiguous share of the selection, kFuseLoads rows in flight per lane, and
// weighs them by exp(s - m). m is the head's top score, which is always
// selected, so the waves share one maximum and their partials add without
// rescaling. Finishes like the split decode's merge: out, lse_sel, and the
// dropped mass from the dense log-sum-exp lse_all.
constexpr int kFuseLoads = 8;
template <int NT, bool MASS>
__device__ __forceinline__ void fused_decode(const SelectArgs& a, int head, int n, uint32_t kmax,
                                             float lse_all, SelShared<NT, MASS>& sh) {
  constexpr int D = 128, LPR = 16, RPW = kWave / LPR, U = kFuseLoads, NW = NT / kWave;
  static_assert(2 * kFuseRows + NW * (D + 1) <= kBins * kRep1, "fused decode overlays the histogram");
  const uint2* sel = reinterpret_cast<const uint2*>(sh.hist);
  float* so = reinterpret_cast<float*>(sh.hist) + 2 * kFuseRows;  // [NW][D] wave partials
  float* sl = so + NW * D;                                        // [NW] wave weight sums
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int c = lane % LPR, rr = lane / LPR;
  const int b = head / a.hq;
  const int g = (head - b * a.hq) / (a.hq / a.hkv);
  const char* vbase = static_cast<const char*>(a.v) +
                      ((size_t)b * a.kv_sb + (size_t)g * a.kv_sh) * sizeof(__half) + c * 16;
  const size_t row_bytes = (size_t)a.kv_st * sizeof(__half);
  const float m = key_to_score(kmax);
  const bool none = m == -INFINITY;
  const int rw = ((n + NW - 1) / NW + RPW - 1) / RPW * RPW;
  const int rb = w * rw;
  const int re = min(n, rb + rw);
  __syncthreads();  // the mirror is complete
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float l = 0.f;
  for (int r0 = rb; r0 < re; r0 += U * RPW) {
    uint4 x[U];
    float p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * RPW + rr;
      const uint2 e = r < re ? sel[r] : make_uint2(0u, 0u);
      const bool ok = r < re && e.x < (uint32_t)a.t;  // every mirrored index is < t
      x[u] = ok ? load16(vbase + (size_t)e.x * row_bytes) : make_uint4(0u, 0u, 0u, 0u);
      p[u] = ok && !none ? __expf(__uint_as_float(e.y) - m) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      axpy16(p[u], x[u], acc, __half());
      if (c == 0) l += p[u];
    }
  }
  // the RPW row slots of the wave (lanes c, c + LPR, ...) hold one column block
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1) acc[e] += __shfl_xor(acc[e], o);
  }
  l = wave_sum(l);
  if (rr == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) so[w * D + c * 8 + e] = acc[e];
  }
  if (lane == 0) sl[w] = l;
  __syncthreads();
  if ((int)threadIdx.x < D) {
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      o += so[k * D + threadIdx.x];
      L += sl[k];
    }
    a.out[(size_t)head * D + threadIdx.x] = L > 0.f ? o / L : 0.f;
    if (threadIdx.x == 0) {
      const float lse = L > 0.f ? m + __logf(L) : -INFINITY;
      a.lse_sel[head] = lse;
      if (a.delta != nullptr) {
        const float dlt = fminf(fmaxf(-expm1f(lse - lse_all), 0.f), 1.f);
        a.delta[head] = dlt;
        if (a.tau != nullptr) a.tau[head] = 1.f - dlt;
      }
    }
  }
}

// Recompute the score row of `head` that a hinted matrix-core scan skipped,
// with the scan's own operands and helpers (the same query sub-group in the
// rows of A, the same products and scaling), so the row is bit-identical to
// the one the scan would have written. Wave w scores RG consecutive 16-key
// groups per pass (4 RG loads in flight per lane) through its 4 KiB tile;
// RG is one group, so that this rare path needs few registers (the few it
// spills in the largest instantiations stay on this path).
template <int NT>
__device__ __forceinline__ void rescore_row(const SelectArgs& a, int head, uint4* tiles) {
  constexpr int NWV = NT / kWave;
  constexpr int RG = 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int c = lane & 15;
  const int rr = lane >> 4;
  const int t = a.t;
  const int b = head / a.hq;
  const int h = head - b * a.hq;
  const int G = a.hq / a.hkv;
  const int g = h / G;
  int off, sub;
  mfma_subgroup(G, h - g * G, off, sub);
  const int m = h - g * G - off;  // the head's row of A
  half8_t qa[4];
  mfma_query_operand(static_cast<const __half*>(a.rescore_q) + (size_t)(b * a.hq + g * G + off) * 128,
                     sub, lane, qa);
  const char* kunit = reinterpret_cast<const char*>(static_cast<const __half*>(a.rescore_k) +
                                                    b * a.kv_sb + g * a.kv_sh);
  const uint32_t rb = (uint32_t)a.kv_st * 2u;
  float* row = a.rescore_row + (size_t)head * a.ld;
  uint4* tile = tiles + w * 256;
  const int ngroups = (t + 15) / 16;
  for (int g0 = RG * w; g0 < ngroups; g0 += RG * NWV) {
    uint4 kv[4 * RG];
#pragma unroll
    for (int i = 0; i < RG; ++i)
#pragma unroll
      for (int mq = 0; mq < 4; ++mq) {
        const int r = min((g0 + i) * 16 + 4 * mq + rr, t - 1);
        kv[4 * i + mq] = load16_stream(kunit + ((uint32_t)c * 16u + (uint32_t)r * rb));
      }
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const float4_t acc = mfma_score16(kv[4 * i], kv[4 * i + 1], kv[4 * i + 2], kv[4 * i + 3], qa,
                                        tile, lane);
      const int key = (g0 + i) * 16 + c;
      if (rr == (m >> 2) && key < t) {
        const int e = m & 3;
        const float v = e == 0 ? acc[0] : e == 1 ? acc[1] : e == 2 ? acc[2] : acc[3];
        row[key] = v * a.rescore_scale;
      }
    }
  }
}

// Heads with a zero `active` flag (when given) are left untouched.
// lse_all is read (DELTA) unless `part` is given: then the head's per-chunk
// (max, sum) partials of the score scan are merged here, the result used and
// written to lse_all. TOPN with scan candidates (cand != NULL) selects from
// them when they hold the answer and otherwise falls back to the full path.
// FUSE: the workgroup then decodes its head (fused_decode), over the top-N
// or the delta-budgeted set.
template <int KPT, int NT, int MODE, bool FUSE>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  constexpr bool MASS = MODE == PRHS_DELTA;
  __shared__ SelShared<NT, MASS> sh;
  // LDS mirror of the selection for the fused decode; the histogram is free
  // once the emission starts
  uint2* const mirror = FUSE ? reinterpret_cast<uint2*>(sh.hist) : nullptr;

  const int head = blockIdx.x;
  if (a.active != nullptr && a.active[head] == 0) return;
  const int t = a.t;
  const float* row = a.scores + (size_t)head * a.ld;
  int* out = a.idx + (size_t)head * a.idx_cap;
  float* out_s = a.sel_scores ? a.sel_scores + (size_t)head * a.idx_cap : nullptr;
  // Without scan candidates the scores are needed in registers: their loads
  // go out first and complete under the partial merge and the LDS clearing.
  const bool from_scan = !MASS && a.cand != nullptr;
  // rows longer than the registers hold take the streamed path throughout
  const bool regs = t <= KPT * NT;
  Keys<KPT> K;
  K.valid = 0;
  if (!from_scan && regs) load_keys_raw<KPT>(K, row, t);
  // the chunk counts of the scan's candidates (lane l of wave w: chunk
  // w * cpw + l), in flight under the partial merge
  uint32_t ccount = 0u;
  if (from_scan) {
    const int cpw = cand_cpw<NT>(a.nchunks);
    const int lane = threadIdx.x & (kWave - 1);
    const int ch = (int)(threadIdx.x / kWave) * cpw + lane;
    if (lane < cpw && ch < a.nchunks) ccount = a.cand_cnt[(size_t)head * a.nchunks + ch];
  }
  if (a.part != nullptr && threadIdx.x < kWave) {
    float m = -INFINITY, l = 0.f;
    for (int c = threadIdx.x; c < a.nchunks; c += kWave) {
      const float2 pc = a.part[(size_t)head * a.nchunks + c];
      ml_combine(m, l, pc.x, pc.y);
    }
    wave_ml(m, l);
    if (threadIdx.x == 0) {
      const float lse = l > 0.f ? m + __logf(l) : -INFINITY;
      sh.lse = lse;
      a.lse_all[head] = lse;
    }
  }

  // the query norm for the threshold hint, by the last wave (the first merges
  // the partials): its loads go out now and are summed after the LDS
  // clearing; read only after the barriers that follow
  const bool qwave = !MASS && a.theta_out != nullptr && threadIdx.x / kWave == NT / kWave - 1;
  uint2 qshare = make_uint2(0u, 0u);
  if (qwave) qshare = query_share(a.hint_q, (size_t)head, a.hint_d, a.hint_q_f16 != 0,
                                  (int)(threadIdx.x & (kWave - 1)));

  for (int i = threadIdx.x; i < kBins * kRep1; i += NT) sh.hist[i] = 0;
  if constexpr (MASS)
    for (int i = threadIdx.x; i < kBins; i += NT) sh.mhist[i] = 0;
  const int nwords = t < kTileKeys ? (t + 31) >> 5 : kMaxWords;
  for (int i = threadIdx.x; i < nwords; i += NT) {
    sh.gt_bits[i] = 0;
    sh.eq_bits[i] = 0;
  }
  if (qwave) {
    const float qn = query_share_norm(qshare, a.hint_q_f16 != 0);
    if ((threadIdx.x & (kWave - 1)) == 0) sh.qnorm = qn;
  }

  if constexpr (!MASS) {
    if (from_scan) {
      uint32_t C = 0;
      if (gather_candidates<NT, MASS>(a.cand, ccount, head, a.nchunks, (uint32_t)a.n_budget, C,
                                      sh)) {
        uint32_t T, take;
        cand_radix<NT, MASS>(sh.kmin, sh.kmax, C, (uint32_t)a.n_budget, T, take, sh);
        emit_list<NT, MASS>(C, T, take, out, out_s, (uint32_t)a.idx_cap, sh, mirror);
        if (threadIdx.x == 0) {
          a.count[head] = a.n_budget;
          if (a.cap_hit) a.cap_hit[head] = 0;
          if (a.theta_out) a.theta_out[head] = next_theta(T, sh.kmax, sh.qnorm);
        }
        if constexpr (FUSE) fused_decode<NT, MASS>(a, head, a.n_budget, sh.kmax, sh.lse, sh);
        return;
      }
      // the candidates do not hold the answer: the full path, on keys loaded
      // now (inside this branch, so that the keys of the other branch are not
      // live across the gather). A hinted head's row is not written by the
      // scan and is recomputed first (the list's LDS serves as the tiles).
      if (a.rescore_k != nullptr && a.cand_cnt[(size_t)head * a.nchunks] != kNoCand) {
        __syncthreads();
        rescore_row<NT>(a, head, reinterpret_cast<uint4*>(sh.cand));
        __syncthreads();
      }
      if (regs) load_keys_raw<KPT>(K, row, t);
    }
  }

  finish_keys<KPT>(K);
  __syncthreads();

  // The nb-th largest key Tn (TOPN: N; DELTA: the cap), `taken` of the keys
  // equal to it in the top-nb set: from the sampled candidate list when it
  // holds them (the register keys die here), else by a radix search that
  // streams the row. sh.kmax is the top key either way.
  const uint32_t nb = (uint32_t)a.n_budget;
  uint32_t theta = 0;
  bool list = false;
  if (regs) list = build_candidates<KPT, NT, MASS>(K, t, nb, theta, sh);
  else stream_kmax<NT, MASS>(row, t, sh);
  const uint32_t C = sh.ncand;
  uint32_t Tn = 0, taken = nb;
  if (list) cand_radix<NT, MASS>(theta, sh.kmax, C, nb, Tn, taken, sh);
  else Tn = count_search<NT, MASS>(row, t, taken, sh);
  uint32_t T = Tn, take = taken;
  int n_sel = (int)nb, hit = 0;
  if constexpr (MASS) {
    // Dropped mass of the top-cap set: above the target the cap binds;
    // otherwise the smallest N lies within the top-cap set, and the mass
    // search runs over the keys >= Tn only, with the mass below Tn spent. On
    // the list path (which holds every key >= Tn) the mass below Tn is the
    // whole -- the dense weights sum to one -- less the listed keys >= Tn,
    // which avoids weighing every key.
    const float lse = a.part != nullptr ? sh.lse : a.lse_all[head];
    const unsigned long long budget = (unsigned long long)((double)a.delta_target * kMassScale);
    const Src src = list ? Src{nullptr, (int)C} : Src{row, t};
    unsigned long long below = 0;
    uint32_t n_eq = 0;
    if (list) {
      unsigned long long top = 0;
      mass_split<NT, false>(src, Tn, lse, top, n_eq, sh);
      const unsigned long long one = (unsigned long long)kMassScale;
      below = top < one ? one - top : 0ull;
    } else {
      mass_split<NT, true>(src, Tn, lse, below, n_eq, sh);
    }
    hit = 1;
    if (below + (unsigned long long)(n_eq - taken) * mass_fx(Tn, lse) <= budget) {
      hit = 0;
      uint32_t n_above = 0, take_T = 0;
      if (mass_search<NT>(src, lse, budget - below, Tn, T, n_above, take_T, sh)) {
        n_sel = (int)(n_above + take_T);
        take = take_T;
      } else {
        // all of the mass is within the target: the single top key (the
        // lowest index among equal ones)
        n_sel = 1;
        take = 1;
        T = sh.kmax;
      }
    }
  }
  if (t <= kTileKeys) {
    if (list) mark_from_list<NT, MASS>(C, T, sh);
    else mark_row<NT, MASS>(row, t, T, sh);
  }
  finish_head<NT, MASS>(a, head, row, out, out_s, list, C, T, take, n_sel, hit, sh, mirror);
  if constexpr (FUSE) fused_decode<NT, MASS>(a, head, n_sel, sh.kmax, sh.lse, sh);
}

static_assert(64 * kSelThreads == kTileKeys, "the largest register instantiation fills one tile");
static_assert(kShortCtx <= kTileKeys && kShortCtx % kShortSelThreads == 0, "short rows fit one tile");

// Short top-N rows: the 512-thread workgroup, kShortCtx / 512 keys per thread.
template <bool FUSE>
void launch_short(int nheads, const SelectArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((select_kernel<kShortCtx / kShortSelThreads, kShortSelThreads, PRHS_TOPN, FUSE>),
                     dim3(nheads), dim3(kShortSelThreads), 0, stream, a);
}

template <int MODE, bool FUSE>
void launch_mode(int kpt, int nheads, const SelectArgs& a, hipStream_t stream) {
#define PRHS_SEL(K)                                                                    \
  hipLaunchKernelGGL((select_kernel<K, kSelThreads, MODE, FUSE>), dim3(nheads),          \
                     dim3(kSelThreads), 0, stream, a)
  switch (kpt) {
    case 1: PRHS_SEL(1); break;
    case 2: PRHS_SEL(2); break;
    case 4: PRHS_SEL(4); break;
    case 8: PRHS_SEL(8); break;
    case 16: PRHS_SEL(16); break;
    case 32: PRHS_SEL(32); break;
    case 64: PRHS_SEL(64); break;
    // longer rows hold no keys in registers (streamed throughout): the
    // smallest instantiation, whose register budget leaves the candidate and
    // streamed paths free of spills
    default: PRHS_SEL(1); break;
  }
#undef PRHS_SEL
}

}  // namespace

hipError_t launch_select(const prhs_dims& d, const SelectArgs& args, hipStream_t stream) {
  int kpt = 1;
  while (kpt * kSelThreads < d.ctx_len) kpt *= 2;
  const int nheads = d.batch * d.n_q_heads;
  SelectArgs a = args;
  // the hint is stored per unit query norm: it needs the queries
  if (a.theta_out != nullptr && (a.hint_q == nullptr || (a.hint_d != 64 && a.hint_d != 128)))
    return hipErrorInvalidValue;
  a.t = d.ctx_len;
  a.ld = d.scores_ld;
  a.nchunks = score_nchunks(d);
  if (a.mode == PRHS_TOPN && d.ctx_len <= kShortCtx) {
    if (a.v != nullptr) launch_short<true>(nheads, a, stream);
    else launch_short<false>(nheads, a, stream);
  } else if (a.mode == PRHS_DELTA) {
    if (a.v != nullptr) launch_mode<PRHS_DELTA, true>(kpt, nheads, a, stream);
    else launch_mode<PRHS_DELTA, false>(kpt, nheads, a, stream);
  } else if (a.v != nullptr) {
    launch_mode<PRHS_TOPN, true>(kpt, nheads, a, stream);
  } else {
    launch_mode<PRHS_TOPN, false>(kpt, nheads, a, stream);
  }
  return hipGetLastError();
}

PRHS_CHECK_READER(take_checks_select)

}  // namespace prhs
