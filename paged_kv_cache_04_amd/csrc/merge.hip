// Log-sum-exp merge of partial attention states.
//
// Partial k of a row covers a disjoint set of keys and carries
// o_k = sum_t exp(s_t - m_k) V_t / sum_t exp(s_t - m_k) and
// lse_k = m_k + log sum_t exp(s_t - m_k).  The exact result over the union is
//   M = max_k lse_k,  w_k = exp(lse_k - M),
//   out = sum_k w_k o_k / sum_k w_k,  lse = M + log sum_k w_k,
// the same rescaling step the online softmax applies between key blocks
// (page 2, section 2.2).  Parts are combined in ascending k order, so the
// result does not depend on the schedule.
//
// One wavefront per row.  The lse values of a row are read lane-parallel for
// the maximum and the weight sum; the D outputs are spread over the lanes and
// each loops over the parts, reading o_k rows with coalesced loads.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, xor_f(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += xor_f(x, m);
  return x;
}

template <typename TT>
__global__ __launch_bounds__(64) void merge_kernel(const float* __restrict__ o_parts,
                                                   const float* __restrict__ lse_parts,
                                                   int32_t n_parts, int32_t head_dim,
                                                   void* __restrict__ out,
                                                   float* __restrict__ lse_out) {
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const float* lp = lse_parts + row * n_parts;
  const float* op = o_parts + row * n_parts * (int64_t)head_dim;

  float mx = -INFINITY;
  bool nan_seen = false;
  for (int k = lane; k < n_parts; k += 64) {
    const float l = lp[k];
    nan_seen |= (l != l);
    mx = fmaxf(mx, l);
  }
  if (__ballot(nan_seen) != 0) {  // a poisoned part poisons the row
    for (int d = lane; d < head_dim; d += 64)
      store_elem<TT>(out, row * head_dim + d, __builtin_nanf(""));
    if (lane == 0 && lse_out) lse_out[row] = __builtin_nanf("");
    return;
  }
  const float M = wave_max(mx);
  if (M == -INFINITY) {  // every part empty
    for (int d = lane; d < head_dim; d += 64) store_elem<TT>(out, row * head_dim + d, 0.f);
    if (lane == 0 && lse_out) lse_out[row] = -INFINITY;
    return;
  }
  float ws = 0.f;
  for (int k = lane; k < n_parts; k += 64) {
    const float l = lp[k];
    if (l != -INFINITY) ws += exp2_fast((l - M) * kLog2e);
  }
  const float wsum = wave_sum(ws);
  const float inv = 1.f / wsum;

  for (int d = lane; d < head_dim; d += 64) {
    float acc = 0.f;
    for (int k = 0; k < n_parts; ++k) {
      const float l = lp[k];
      if (l == -INFINITY) continue;
      acc = fmaf(exp2_fast((l - M) * kLog2e), op[(int64_t)k * head_dim + d], acc);
    }
    store_elem<TT>(out, row * head_dim + d, acc * inv);
  }
  if (lane == 0 && lse_out) lse_out[row] = M + log2_fast(wsum) * kLn2;
}

}  // namespace

hipError_t launch_merge(int out_dtype, int head_dim, const float* o_parts,
                        const float* lse_parts, int32_t rows, int32_t n_parts, void* out,
                        float* lse_out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)rows), block(64);
  switch (out_dtype) {
    case 0:
      hipLaunchKernelGGL(merge_kernel<TF32>, grid, block, 0, stream, o_parts, lse_parts,
                         n_parts, head_dim, out, lse_out);
      break;
    case 1:
      hipLaunchKernelGGL(merge_kernel<TF16>, grid, block, 0, stream, o_parts, lse_parts,
                         n_parts, head_dim, out, lse_out);
      break;
    case 2:
      hipLaunchKernelGGL(merge_kernel<TBF16>, grid, block, 0, stream, o_parts, lse_parts,
                         n_parts, head_dim, out, lse_out);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
