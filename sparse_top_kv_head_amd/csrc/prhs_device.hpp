// Device-side helpers shared by the PrHS kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace prhs {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element types: one 16-byte lane load holds kElems elements.
// ---------------------------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kPer16B = 4; };
template <> struct Elem<__half> { static constexpr int kPer16B = 8; };

// Dot product of one 16-byte slice of a key row with the matching slice of a
// query (kept as raw 16 bytes), accumulated in fp32.
__device__ __forceinline__ float dot16(const uint4 a, const uint4 b, float acc, float /*tag*/) {
  const float* x = reinterpret_cast<const float*>(&a);
  const float* y = reinterpret_cast<const float*>(&b);
  acc = __builtin_fmaf(x[0], y[0], acc);
  acc = __builtin_fmaf(x[1], y[1], acc);
  acc = __builtin_fmaf(x[2], y[2], acc);
  acc = __builtin_fmaf(x[3], y[3], acc);
  return acc;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot16(const uint4 a, const uint4 b, float acc, __half /*tag*/) {
  const half2_t* x = reinterpret_cast<const half2_t*>(&a);
  const half2_t* y = reinterpret_cast<const half2_t*>(&b);
  acc = __builtin_amdgcn_fdot2(x[0], y[0], acc, false);
  acc = __builtin_amdgcn_fdot2(x[1], y[1], acc, false);
  acc = __builtin_amdgcn_fdot2(x[2], y[2], acc, false);
  acc = __builtin_amdgcn_fdot2(x[3], y[3], acc, false);
  return acc;
}

// Widen one 16-byte slice to fp32 and accumulate w * slice into acc[kPer16B].
__device__ __forceinline__ void axpy16(float w, const uint4 a, float* acc, float /*tag*/) {
  const float* x = reinterpret_cast<const float*>(&a);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(w, x[i], acc[i]);
}

__device__ __forceinline__ void axpy16(float w, const uint4 a, float* acc, __half /*tag*/) {
  const half2_t* x = reinterpret_cast<const half2_t*>(&a);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = __builtin_fmaf(w, (float)x[i].x, acc[2 * i]);
    acc[2 * i + 1] = __builtin_fmaf(w, (float)x[i].y, acc[2 * i + 1]);
  }
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streaming load: the data is read once, so mark it non-temporal.
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// Matrix-core scoring of fp16 key rows with d = 128 (the scan, and the
// selection's recomputation of a row the scan did not write; both use these
// helpers, so their scores are bit-identical).
//
// A 16x16x32 product takes from lane l the 8 consecutive k-elements
// 8 (l / 16) .. + 7 of A's row l % 16 and of B's column l % 16, and returns
// D[4 (l / 16) + r][l % 16] in element r. A holds up to 16 query heads (one
// per row, the rest zero) and B 16 keys (key n in column n); feature block j
// (features 32 j .. 32 j + 31, i.e. 16-byte segments 4 j .. 4 j + 3) is the
// j-th of four chained products.
// ---------------------------------------------------------------------------
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// The A operands of the nq (<= 16) consecutive query rows starting at q0:
// lane l holds head min(l % 16, nq - 1) (zeroed when l % 16 >= nq), segment
// 4 j + l / 16 of feature block j.
__device__ __forceinline__ void mfma_query_operand(const __half* q0, int nq, int lane,
                                                   half8_t (&qa)[4]) {
  const int c = lane & 15;
  const int rr = lane >> 4;
  const int m = c < nq ? c : nq - 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint4 v = *reinterpret_cast<const uint4*>(q0 + (size_t)m * 128 + (4 * j + rr) * 8);
    if (c >= nq) v = make_uint4(0, 0, 0, 0);
    qa[j] = __builtin_bit_cast(half8_t, v);
  }
}

// Scores of one 16-key group against the heads of qa. On entry lane l holds,
// in k[mq], segment l % 16 of key 4 mq + l / 16 (the coalesced load layout:
// one load instruction covers four whole rows). The keys pass through the
// wave's own 4 KiB LDS tile, segment s of key n at 16-byte slot 16 n + (s ^ n),
// so the 16 lanes of one row write and the 16 lanes of one operand read each
// hit 16 distinct slots of a 256-byte bank row. Returns D (heads x keys) in
// the product's layout, unscaled.
__device__ __forceinline__ float4_t mfma_score16(const uint4 k0, const uint4 k1, const uint4 k2,
                                                 const uint4 k3, const half8_t (&qa)[4],
                                                 uint4* tile, int lane) {
  const int c = lane & 15;
  const int rr = lane >> 4;
  const uint4 kk[4] = {k0, k1, k2, k3};
#pragma unroll
  for (int mq = 0; mq < 4; ++mq) {
    const int nk = 4 * mq + rr;
    tile[nk * 16 + (c ^ nk)] = kk[mq];
  }
  // The tile is shared by the lanes of this wave only, and LDS operations of
  // one wave complete in order: a wave-scope fence, which only orders the
  // compiler's accesses, is all the exchange needs.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half8_t bk = __builtin_bit_cast(half8_t, tile[c * 16 + ((4 * j + rr) ^ c)]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[j], bk, acc, 0, 0, 0);
  }
  // the next group may overwrite the tile only after these reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return acc;
}

// Query sub-groups of a GQA group of G heads, as the scans launch them. The
// matrix-core scan takes up to 16 heads per launch (the rows of its A
// operand; a group of 12 is one launch, padded to 16 rows), in consecutive
// runs of 16. The dot-product scan takes power-of-two sub-groups of at most 8,
// largest first.
constexpr int kMfmaMaxGroup = 16;
constexpr int kDotMaxGroup = 8;

// Size of the next dot-product sub-group when `rest` heads are left.
__host__ __device__ inline int dot_subgroup_size(int rest) {
  int sub = 1;
  while (sub * 2 <= rest && sub * 2 <= kDotMaxGroup) sub *= 2;
  return sub;
}

// The matrix-core sub-group of head h_local: its first head (within the
// group) and its size.
__host__ __device__ inline void mfma_subgroup(int G, int h_local, int& off, int& sub) {
  off = h_local / kMfmaMaxGroup * kMfmaMaxGroup;
  sub = G - off < kMfmaMaxGroup ? G - off : kMfmaMaxGroup;
}

// Rows of the A operand (and template size) for a sub-group of nq heads: the
// next power of two.
__host__ __device__ inline int mfma_rows(int nq) {
  int r = 1;
  while (r < nq) r *= 2;
  return r;
}

// ---------------------------------------------------------------------------
// Device checks. Built with -DPRHS_DEVICE_CHECKS (the checked library), a
// kernel that meets a broken input contract or internal invariant sets a bit
// in its source file's check word with a vector atomic and carries on as the
// unchecked build does (nothing traps); the library reads and clears the
// words after each call and reports the bits as an error. Without the macro
// every check compiles to nothing.
// ---------------------------------------------------------------------------
#ifdef PRHS_DEVICE_CHECKS
static __device__ unsigned int g_check_word = 0u;
#define PRHS_CHECK(cond, bit)                                        \
  do {                                                               \
    if (!(cond)) __hip_atomic_fetch_or(&g_check_word, (bit), __ATOMIC_RELAXED, \
                                       __HIP_MEMORY_SCOPE_AGENT);    \
  } while (0)
// Host side: this source file's check word, read and cleared (synchronous).
#define PRHS_CHECK_READER(fn)                                                      \
  uint32_t fn() {                                                                  \
    uint32_t v = 0u, zero = 0u;                                                    \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_check_word), sizeof v) != hipSuccess) \
      return 0x80000000u;                                                          \
    if (v != 0u) (void)hipMemcpyToSymbol(HIP_SYMBOL(g_check_word), &zero, sizeof zero); \
    return v;                                                                      \
  }
#else
#define PRHS_CHECK(cond, bit) \
  do {                        \
  } while (0)
#define PRHS_CHECK_READER(fn) \
  uint32_t fn() { return 0u; }
#endif

// ---------------------------------------------------------------------------
// Write-through stores: the system-scope cache policy (sc0 sc1) sends the data
// through the L2 to memory at once instead of leaving dirty lines behind. The
// scan's outputs are written this way: interleaved with its K read stream,
// lines that would later be written back cost more (measured: the 32K GQA scan
// 49.5-50.3 -> 47.2-47.8 us with its score rows, 48.9-49.9 -> 48.1-48.6 us with
// candidates). Raw buffer stores over [base, base + bytes) with `base`
// wave-uniform; out-of-range offsets are dropped by the buffer bounds check.
// ---------------------------------------------------------------------------
constexpr int kStoreThrough = 17;  // sc0 | sc1 in the cache-policy operand
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void store_through(void* base, uint32_t bytes, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, buffer_rsrc(base, bytes), (int)off, 0, kStoreThrough);
}

__device__ __forceinline__ void store_through(void* base, uint32_t bytes, uint32_t off, uint2 v) {
  const u32x2_t x = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(x, buffer_rsrc(base, bytes), (int)off, 0, kStoreThrough);
}

__device__ __forceinline__ void store_through(void* base, uint32_t bytes, uint32_t off, float4 v) {
  const u32x4_t x = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                     __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(x, buffer_rsrc(base, bytes), (int)off, 0, kStoreThrough);
}

// ---------------------------------------------------------------------------
// Cross-lane data movement
// ---------------------------------------------------------------------------
// DPP controls (GFX9 encoding).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Every control used with this helper permutes lanes inside a 16-lane row, so
// each lane has a source lane; bound_ctrl only lets the compiler fold the move
// into the consuming VALU instruction (v_add_f32_dpp and the like).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPR consecutive lanes; every lane of the group
// receives the group total. LPR in {4, 8, 16, 32, 64}.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  if constexpr (LPR >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (LPR >= 32) {
    // swap the two 16-lane halves of each 32-lane group
    x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
  }
  if constexpr (LPR >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Maximum over aligned groups of L consecutive lanes, the exchanges of
// group_sum; every lane of the group receives it. L in {4, 8, 16, 32, 64}.
template <int L>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (L >= 8) x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  if constexpr (L >= 16) x = fmaxf(x, dpp<kDppRowMirror>(x));
  if constexpr (L >= 32)
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F)));
  if constexpr (L >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// Whole-wave reductions (every lane receives the result; called with the
// whole wave active): the DPP and swizzle exchanges of group_max/group_sum,
// which take a few cycles each, with one cross-half exchange at the end.
__device__ __forceinline__ float wave_max(float x) { return group_max<kWave>(x); }

__device__ __forceinline__ float wave_sum(float x) { return group_sum<kWave>(x); }

// fp32 Euclidean norm of one query row of D elements (lane-strided loads);
// every lane of the wave returns it.
template <typename T, int D>
__device__ __forceinline__ float query_norm(const T* __restrict__ row, int lane) {
  float s = 0.f;
#pragma unroll
  for (int e = lane; e < D; e += kWave) {
    const float x = static_cast<float>(row[e]);
    s = __builtin_fmaf(x, x, s);
  }
  return __builtin_sqrtf(wave_sum(s));
}

// The same in two halves, so that the loads can be issued early and summed
// later: this lane's elements e = lane, lane + 64 of a row of d (64 or 128)
// fp16 or fp32 elements, as raw bits (zero past the row).
__device__ __forceinline__ uint2 query_share(const void* __restrict__ q, size_t row, int d,
                                             bool f16, int lane) {
  uint2 r = make_uint2(0u, 0u);
  if (f16) {
    const uint16_t* p = static_cast<const uint16_t*>(q) + row * d;
    r.x = p[lane];
    if (lane + kWave < d) r.y = p[lane + kWave];
  } else {
    const uint32_t* p = static_cast<const uint32_t*>(q) + row * d;
    r.x = p[lane];
    if (lane + kWave < d) r.y = p[lane + kWave];
  }
  return r;
}

__device__ __forceinline__ float query_share_norm(uint2 r, bool f16) {
  float x, y;
  if (f16) {
    x = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)r.x));
    y = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)r.y));
  } else {
    x = __uint_as_float(r.x);
    y = __uint_as_float(r.y);
  }
  return __builtin_sqrtf(wave_sum(__builtin_fmaf(x, x, y * y)));
}

// Combine two (max, sum-of-exp) pairs: sum is relative to its max; an empty
// pair is (-inf, 0).
__device__ __forceinline__ void ml_combine(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) { m = mn; l = 0.f; return; }
  l = l * __expf(m - mn) + l2 * __expf(m2 - mn);
  m = mn;
}

// The (max, sum-of-exp) pair of the whole wave, through the exchanges of
// group_sum (each pairs every lane with a distinct partner, so all lanes end
// with the same pair).
__device__ __forceinline__ float swizzle_half(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
__device__ __forceinline__ void wave_ml(float& m, float& l) {
  ml_combine(m, l, dpp<kDppXor1>(m), dpp<kDppXor1>(l));
  ml_combine(m, l, dpp<kDppXor2>(m), dpp<kDppXor2>(l));
  ml_combine(m, l, dpp<kDppRowHalfMirror>(m), dpp<kDppRowHalfMirror>(l));
  ml_combine(m, l, dpp<kDppRowMirror>(m), dpp<kDppRowMirror>(l));
  ml_combine(m, l, swizzle_half(m), swizzle_half(l));
  ml_combine(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32));
}

// Inclusive prefix sum of 32-bit values over the 64 lanes of a wave, with DPP
// row shifts inside each 16-lane row and row broadcasts across rows.
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Inclusive running maximum over the 64 lanes of a wave: the DPP steps of
// wave_scan_u32, with the smallest int as the value of lanes that have no
// source.
__device__ __forceinline__ int wave_inclusive_max(int x) {
  constexpr int kLow = -2147483647 - 1;
  int y;
  y = __builtin_amdgcn_update_dpp(kLow, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x = x > y ? x : y;
  y = __builtin_amdgcn_update_dpp(kLow, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x = x > y ? x : y;
  y = __builtin_amdgcn_update_dpp(kLow, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x = x > y ? x : y;
  y = __builtin_amdgcn_update_dpp(kLow, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x = x > y ? x : y;
  y = __builtin_amdgcn_update_dpp(kLow, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x = x > y ? x : y;
  y = __builtin_amdgcn_update_dpp(kLow, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  x = x > y ? x : y;
  return x;
}

// Maximum and minimum of 32-bit unsigned values over the whole wave (every
// lane receives it; called with the whole wave active), through the
// exchanges of group_sum.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
template <bool MAX>
__device__ __forceinline__ uint32_t wave_extreme_u32(uint32_t x) {
  auto pick = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  x = pick(x, dpp_u32<kDppXor1>(x));
  x = pick(x, dpp_u32<kDppXor2>(x));
  x = pick(x, dpp_u32<kDppRowHalfMirror>(x));
  x = pick(x, dpp_u32<kDppRowMirror>(x));
  x = pick(x, (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F));
  x = pick(x, (uint32_t)__shfl_xor((int)x, 32));
  return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) { return wave_extreme_u32<true>(x); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return wave_extreme_u32<false>(x); }

__device__ __forceinline__ uint32_t lane_read(uint32_t x, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

// Inclusive prefix sum over the 64 lanes of a wave.
template <typename U>
__device__ __forceinline__ U wave_inclusive_scan(U x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const U y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive prefix sum over a whole workgroup of NT threads. `tmp` is LDS of
// at least NT / 64 elements. Returns the exclusive prefix; `total` receives the
// workgroup total. Contains two barriers.
template <int NT, typename U>
__device__ __forceinline__ U block_exclusive_scan(U x, U* tmp, U& total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const U inc = wave_inclusive_scan(x);
  if (lane == kWave - 1) tmp[w] = inc;
  __syncthreads();
  U base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const U v = tmp[i];
    if (i < w) base += v;
    tot += v;
  }
  __syncthreads();
  total = tot;
  return base + inc - x;
}

// ---------------------------------------------------------------------------
// Order-preserving 32-bit key of an fp32 score (larger score -> larger key).
// -0.0 is folded onto +0.0 so that the two compare equal.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __builtin_bit_cast(uint32_t, s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace prhs
