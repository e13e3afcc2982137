// Log-sum-exp merge of partial attention states.
//
// Partial k of a row covers a disjoint set of keys and carries
// o_k = sum_t exp(s_t - m_k) V_t / sum_t exp(s_t - m_k) and
// lse_k = m_k + log sum_t exp(s_t - m_k).  The exact result over the union is
//   M = max_k lse_k,  w_k = exp(lse_k - M),
//   out = sum_k w_k o_k / sum_k w_k,  lse = M + log sum_k w_k,
// the same rescaling step the online softmax applies between key blocks
// (page 2, section 2.2).  The combination order is fixed by (n_parts, D), so
// the result does not depend on the schedule.
//
// Two forms, the same sums in a fixed order for a given (n_parts, D):
// - up to 16 parts per row, one wavefront per row and four rows per
//   256-thread workgroup, no LDS and no barrier: the row's lse values are
//   reduced across the wave (maximum, weight sum); the o_k rows are read as
//   float4 by groups of D/4 lanes (two groups at D = 128, four at D = 64),
//   group j taking parts j, j + groups, ..., and the groups' sums are added
//   by lane exchanges;
// - more parts (a few long rows split many times), one 256-thread workgroup
//   per row: block-wide reductions, eight (D = 128) or sixteen (D = 64) part
//   groups, their sums added in LDS.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kMergeThreads = 256;
constexpr int kRowsPerBlock = kMergeThreads / 64;
constexpr int kWaveRowParts = 16;   // up to this many parts: one wavefront per row

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

template <typename TT, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int32_t n_parts,
    int64_t rows, void* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int LPP = D / 4;          // lanes per part row (float4 each)
  constexpr int NG = 64 / LPP;        // part groups per wave
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;            // the whole wave
  const float* lp = lse_parts + row * n_parts;
  const float* op = o_parts + row * n_parts * (int64_t)D;

  // row max and NaN check
  float mx = -INFINITY;
  int nan_seen = 0;
  for (int k = lane; k < n_parts; k += 64) {
    const float l = lp[k];
    nan_seen |= (l != l);
    mx = fmaxf(mx, l);
  }
  const float M = wave_max(mx);
  const bool any_nan = __ballot(nan_seen) != 0;
  if (any_nan || M == -INFINITY) {  // a poisoned part poisons the row; all empty gives 0
    const float o = any_nan ? __builtin_nanf("") : 0.f;
    for (int d = lane; d < D; d += 64) store_elem<TT>(out, row * D + d, o);
    if (lane == 0 && lse_out) lse_out[row] = any_nan ? __builtin_nanf("") : -INFINITY;
    return;
  }

  float ws = 0.f;
  for (int k = lane; k < n_parts; k += 64) {
    const float l = lp[k];
    ws += (l == -INFINITY) ? 0.f : exp2_fast((l - M) * kLog2e);
  }
  const float wsum = wave_sum(ws);

  const int grp = lane / LPP, li = lane % LPP;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int k = grp; k < n_parts; k += NG) {
    const float l = lp[k];
    const float4 o = *reinterpret_cast<const float4*>(op + (int64_t)k * D + li * 4);
    const bool skip = (l == -INFINITY);
    const float wk = skip ? 0.f : exp2_fast((l - M) * kLog2e);
    acc.x += skip ? 0.f : wk * o.x;
    acc.y += skip ? 0.f : wk * o.y;
    acc.z += skip ? 0.f : wk * o.z;
    acc.w += skip ? 0.f : wk * o.w;
  }
#pragma unroll
  for (int m = LPP; m < 64; m <<= 1) {   // add the other groups' sums, fixed order
    acc.x += xor_f(acc.x, m);
    acc.y += xor_f(acc.y, m);
    acc.z += xor_f(acc.z, m);
    acc.w += xor_f(acc.w, m);
  }
  if (grp == 0) {
    const float inv = 1.f / wsum;
    const int64_t base = row * D + li * 4;
    store_elem<TT>(out, base + 0, acc.x * inv);
    store_elem<TT>(out, base + 1, acc.y * inv);
    store_elem<TT>(out, base + 2, acc.z * inv);
    store_elem<TT>(out, base + 3, acc.w * inv);
  }
  if (lane == 0 && lse_out) lse_out[row] = M + log2_fast(wsum) * kLn2;
}

template <typename TT, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_block_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int32_t n_parts,
    void* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int LPP = D / 4;                    // lanes per part row (float4 each)
  constexpr int NG = kMergeThreads / LPP;       // part groups
  __shared__ float red[NG][D];
  __shared__ float wred[4];
  __shared__ int nan_red[4];

  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const float* lp = lse_parts + row * n_parts;
  const float* op = o_parts + row * n_parts * (int64_t)D;

  // block max and NaN check
  float mx = -INFINITY;
  int nan_seen = 0;
  for (int k = tid; k < n_parts; k += kMergeThreads) {
    const float l = lp[k];
    nan_seen |= (l != l);
    mx = fmaxf(mx, l);
  }
  mx = wave_max(mx);
  nan_seen = __ballot(nan_seen) != 0;
  if (lane == 0) {
    wred[wv] = mx;
    nan_red[wv] = nan_seen;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  const bool any_nan = (nan_red[0] | nan_red[1] | nan_red[2] | nan_red[3]) != 0;
  if (any_nan || M == -INFINITY) {  // a poisoned part poisons the row; all empty gives 0
    const float o = any_nan ? __builtin_nanf("") : 0.f;
    for (int d = tid; d < D; d += kMergeThreads) store_elem<TT>(out, row * D + d, o);
    if (tid == 0 && lse_out) lse_out[row] = any_nan ? __builtin_nanf("") : -INFINITY;
    return;
  }
  __syncthreads();  // wred is reused below

  float ws = 0.f;
  for (int k = tid; k < n_parts; k += kMergeThreads) {
    const float l = lp[k];
    ws += (l == -INFINITY) ? 0.f : exp2_fast((l - M) * kLog2e);
  }
  ws = wave_sum(ws);
  if (lane == 0) wred[wv] = ws;

  const int grp = tid / LPP, li = tid % LPP;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int k = grp; k < n_parts; k += NG) {
    const float l = lp[k];
    const float4 o = *reinterpret_cast<const float4*>(op + (int64_t)k * D + li * 4);
    const bool skip = (l == -INFINITY);
    const float wk = skip ? 0.f : exp2_fast((l - M) * kLog2e);
    acc.x += skip ? 0.f : wk * o.x;
    acc.y += skip ? 0.f : wk * o.y;
    acc.z += skip ? 0.f : wk * o.z;
    acc.w += skip ? 0.f : wk * o.w;
  }
  red[grp][li * 4 + 0] = acc.x;
  red[grp][li * 4 + 1] = acc.y;
  red[grp][li * 4 + 2] = acc.z;
  red[grp][li * 4 + 3] = acc.w;
  __syncthreads();
  const float wsum = wred[0] + wred[1] + wred[2] + wred[3];
  const float inv = 1.f / wsum;
  for (int d = tid; d < D; d += kMergeThreads) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NG; ++j) s += red[j][d];
    store_elem<TT>(out, row * D + d, s * inv);
  }
  if (tid == 0 && lse_out) lse_out[row] = M + log2_fast(wsum) * kLn2;
}

template <typename TT>
hipError_t launch_t(int head_dim, const float* o_parts, const float* lse_parts, int32_t rows,
                    int32_t n_parts, void* out, float* lse_out, hipStream_t stream) {
  const dim3 block(kMergeThreads);
  if (n_parts <= kWaveRowParts) {
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    switch (head_dim) {
      case 64:
        hipLaunchKernelGGL((merge_kernel<TT, 64>), grid, block, 0, stream, o_parts, lse_parts,
                           n_parts, (int64_t)rows, out, lse_out);
        break;
      case 128:
        hipLaunchKernelGGL((merge_kernel<TT, 128>), grid, block, 0, stream, o_parts, lse_parts,
                           n_parts, (int64_t)rows, out, lse_out);
        break;
      default:
        return hipErrorInvalidValue;
    }
  } else {
    const dim3 grid((unsigned)rows);
    switch (head_dim) {
      case 64:
        hipLaunchKernelGGL((merge_block_kernel<TT, 64>), grid, block, 0, stream, o_parts,
                           lse_parts, n_parts, out, lse_out);
        break;
      case 128:
        hipLaunchKernelGGL((merge_block_kernel<TT, 128>), grid, block, 0, stream, o_parts,
                           lse_parts, n_parts, out, lse_out);
        break;
      default:
        return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(int out_dtype, int head_dim, const float* o_parts,
                        const float* lse_parts, int32_t rows, int32_t n_parts, void* out,
                        float* lse_out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  switch (out_dtype) {
    case 0: return launch_t<TF32>(head_dim, o_parts, lse_parts, rows, n_parts, out, lse_out, stream);
    case 1: return launch_t<TF16>(head_dim, o_parts, lse_parts, rows, n_parts, out, lse_out, stream);
    case 2: return launch_t<TBF16>(head_dim, o_parts, lse_parts, rows, n_parts, out, lse_out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
