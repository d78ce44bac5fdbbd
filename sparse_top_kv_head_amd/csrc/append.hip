// Growing KV cache: append one decode step's key and value rows (page
// "Near-Oracle KV Selection via Pre-hoc Sparsity for Long-Context Inference",
// Table I: t counts the decode steps, so the cache gains one row per step).
//
// One wave per (b, KV head): the first LPR lanes copy the K row and the next
// LPR lanes the V row, 16 bytes each (LPR = row bytes / 16 <= 32).
#include "prhs_device.hpp"
#include "prhs_launch.hpp"

namespace prhs {
namespace {

__global__ __launch_bounds__(kWave) void append_kv_kernel(const uint4* __restrict__ k_new,
                                                           const uint4* __restrict__ v_new,
                                                           char* __restrict__ k,
                                                           char* __restrict__ v, int Hkv, int lpr,
                                                           long long sb, long long sh,
                                                           long long row_off) {
  const int unit = blockIdx.x;
  const int b = unit / Hkv;
  const int g = unit - b * Hkv;
  const int lane = threadIdx.x;
  if (lane >= 2 * lpr) return;
  const bool is_v = lane >= lpr;
  const int c = is_v ? lane - lpr : lane;
  const uint4 x = (is_v ? v_new : k_new)[(size_t)unit * lpr + c];
  char* dst = (is_v ? v : k) + (size_t)b * sb + (size_t)g * sh + row_off;
  reinterpret_cast<uint4*>(dst)[c] = x;
}

}  // namespace

hipError_t launch_append_kv(const prhs_dims& d, const void* k_new, const void* v_new, void* k,
                            void* v, int pos, hipStream_t stream) {
  const long long es = d.dtype == PRHS_F16 ? 2 : 4;
  const int lpr = (int)(d.head_dim * es / 16);
  hipLaunchKernelGGL(append_kv_kernel, dim3(d.batch * d.n_kv_heads), dim3(kWave), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     static_cast<char*>(k), static_cast<char*>(v), d.n_kv_heads, lpr,
                     (long long)d.kv_stride_b * es, (long long)d.kv_stride_h * es,
                     (long long)pos * d.kv_stride_t * es);
  return hipGetLastError();
}

}  // namespace prhs
