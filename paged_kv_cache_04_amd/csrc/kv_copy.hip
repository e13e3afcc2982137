// kv_append and gather: the paged address rule as plain copies.
//
// A token's K/V row for one KV head is D elements, 64 or 128 bytes for fp8,
// 128 or 256 bytes for the 16-bit types and 256 or 512 for f32: always a
// whole number of 16-byte vectors.  Each thread moves one 16-byte vector, so
// a wavefront moves 1 KiB with fully coalesced loads and stores.  The slot of a token (slot = page *
// P + offset) gives page = slot / P and offset = slot % P (page 3, section
// 3.2: the page of token t is page_table[t / PAGE_SIZE]).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kCopyThreads = 256;

// One thread per (K or V, token, head, 16-byte vector).
__global__ __launch_bounds__(kCopyThreads) void kv_append_kernel(
    char* __restrict__ k_cache, char* __restrict__ v_cache, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int32_t* __restrict__ slots, int32_t n_tokens,
    int32_t num_kv_heads, int32_t row_vecs, int64_t num_slots) {
  const int64_t per_tok = (int64_t)num_kv_heads * row_vecs;
  const int64_t total = 2 * (int64_t)n_tokens * per_tok;
  for (int64_t idx = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kCopyThreads) {
    const int which = idx >= (int64_t)n_tokens * per_tok;   // 0: K, 1: V
    const int64_t r = which ? idx - (int64_t)n_tokens * per_tok : idx;
    const int64_t i = r / per_tok;
    const int64_t rem = r - i * per_tok;
    const int64_t g = rem / row_vecs;
    const int64_t vec = rem - g * row_vecs;
    const int64_t s = slots[i];
    if (s < 0 || s >= num_slots) continue;
    const int64_t page = s / kPageSize;
    const int64_t off = s - page * kPageSize;
    const int64_t row_bytes = (int64_t)row_vecs * 16;
    const int64_t dst = ((page * num_kv_heads + g) * kPageSize + off) * row_bytes + vec * 16;
    const int64_t src = (i * num_kv_heads + g) * row_bytes + vec * 16;
    if (which)
      store16(v_cache + dst, load16(v_new + src));
    else
      store16(k_cache + dst, load16(k_new + src));
  }
}

// One thread per (K or V, token, head, 16-byte vector) of the output.
__global__ __launch_bounds__(kCopyThreads) void gather_kernel(
    const char* __restrict__ k_cache, const char* __restrict__ v_cache,
    const int32_t* __restrict__ table_row, int32_t len, int32_t num_kv_heads, int32_t row_vecs,
    int64_t num_pages, char* __restrict__ k_out, char* __restrict__ v_out, int elem_bytes) {
  const int64_t per_tok = (int64_t)num_kv_heads * row_vecs;
  const int64_t total = 2 * (int64_t)len * per_tok;
  for (int64_t idx = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kCopyThreads) {
    const int which = idx >= (int64_t)len * per_tok;
    const int64_t r = which ? idx - (int64_t)len * per_tok : idx;
    const int64_t t = r / per_tok;
    const int64_t rem = r - t * per_tok;
    const int64_t g = rem / row_vecs;
    const int64_t vec = rem - g * row_vecs;
    const int64_t page = table_row[t / kPageSize];
    const int64_t row_bytes = (int64_t)row_vecs * 16;
    const int64_t dst = (t * num_kv_heads + g) * row_bytes + vec * 16;
    char* out = which ? v_out : k_out;
    u32x4 val;
    if (page < 0 || page >= num_pages) {
      // out-of-range page id: write NaN (all-ones payload is NaN for f32/f16/bf16)
      val.w[0] = val.w[1] = val.w[2] = val.w[3] = 0xffffffffu;
    } else {
      const int64_t src = ((page * num_kv_heads + g) * kPageSize + t % kPageSize) * row_bytes +
                          vec * 16;
      val = load16((which ? v_cache : k_cache) + src);
    }
    store16(out + dst, val);
    (void)elem_bytes;
  }
}

// One thread per (K or V, token, head, group of 16 elements): reads the 16
// source elements, divides by the pool's scale in IEEE fp32, writes 16 fp8
// codes as one 16-byte store.
template <typename ST, bool E4M3>
__global__ __launch_bounds__(kCopyThreads) void kv_append_quant_kernel(
    char* __restrict__ k_cache, char* __restrict__ v_cache, const char* __restrict__ k_new,
    const char* __restrict__ v_new, float k_scale, float v_scale,
    const int32_t* __restrict__ slots, int32_t n_tokens, int32_t num_kv_heads, int32_t row_vecs,
    int64_t num_slots) {
  constexpr int SB = ST::bytes;          // source bytes per element
  const int64_t per_tok = (int64_t)num_kv_heads * row_vecs;
  const int64_t total = 2 * (int64_t)n_tokens * per_tok;
  for (int64_t idx = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * kCopyThreads) {
    const int which = idx >= (int64_t)n_tokens * per_tok;   // 0: K, 1: V
    const int64_t r = which ? idx - (int64_t)n_tokens * per_tok : idx;
    const int64_t i = r / per_tok;
    const int64_t rem = r - i * per_tok;
    const int64_t g = rem / row_vecs;
    const int64_t vec = rem - g * row_vecs;
    const int64_t s = slots[i];
    if (s < 0 || s >= num_slots) continue;
    const int64_t page = s / kPageSize;
    const int64_t off = s - page * kPageSize;
    const int64_t row_bytes = (int64_t)row_vecs * 16;          // fp8: D bytes
    const int64_t dst = ((page * num_kv_heads + g) * kPageSize + off) * row_bytes + vec * 16;
    const char* src =
        (which ? v_new : k_new) + ((i * num_kv_heads + g) * row_vecs + vec) * 16 * SB;
    const float scale = which ? v_scale : k_scale;
    u32x4 in[4];
#pragma unroll
    for (int j = 0; j < SB; ++j) in[j] = load16(src + 16 * j);
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = __fdiv_rn(src_elem<ST>(in, 4 * q + e), scale);
      out.w[q] = fp8_pack4<E4M3>(y);
    }
    store16((which ? v_cache : k_cache) + dst, out);
  }
}

int elem_size(int dtype) { return dtype == 0 ? 4 : (dtype >= 3 ? 1 : 2); }

unsigned grid_for(int64_t total) {
  int64_t blocks = (total + kCopyThreads - 1) / kCopyThreads;
  if (blocks > 65536) blocks = 65536;    // grid-stride loop covers the rest
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

template <typename ST>
hipError_t launch_quant_t(bool e4m3, int head_dim, int num_kv_heads, int64_t num_pages,
                          void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                          float k_scale, float v_scale, const int32_t* slots, int32_t n_tokens,
                          hipStream_t stream) {
  const int row_vecs = head_dim / 16;
  const int64_t total = 2 * (int64_t)n_tokens * num_kv_heads * row_vecs;
  const dim3 grid(grid_for(total)), block(kCopyThreads);
  if (e4m3)
    hipLaunchKernelGGL((kv_append_quant_kernel<ST, true>), grid, block, 0, stream,
                       (char*)k_cache, (char*)v_cache, (const char*)k_new, (const char*)v_new,
                       k_scale, v_scale, slots, n_tokens, num_kv_heads, row_vecs,
                       num_pages * kPageSize);
  else
    hipLaunchKernelGGL((kv_append_quant_kernel<ST, false>), grid, block, 0, stream,
                       (char*)k_cache, (char*)v_cache, (const char*)k_new, (const char*)v_new,
                       k_scale, v_scale, slots, n_tokens, num_kv_heads, row_vecs,
                       num_pages * kPageSize);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append_quant(int fp8_dtype, int src_dtype, int head_dim, int num_kv_heads,
                                  int64_t num_pages, void* k_cache, void* v_cache,
                                  const void* k_new, const void* v_new, float k_scale,
                                  float v_scale, const int32_t* slots, int32_t n_tokens,
                                  hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  if (fp8_dtype != 3 && fp8_dtype != 4) return hipErrorInvalidValue;
  const bool e4m3 = fp8_dtype == 3;
  switch (src_dtype) {
    case 0: return launch_quant_t<TF32>(e4m3, head_dim, num_kv_heads, num_pages, k_cache,
                                        v_cache, k_new, v_new, k_scale, v_scale, slots,
                                        n_tokens, stream);
    case 1: return launch_quant_t<TF16>(e4m3, head_dim, num_kv_heads, num_pages, k_cache,
                                        v_cache, k_new, v_new, k_scale, v_scale, slots,
                                        n_tokens, stream);
    case 2: return launch_quant_t<TBF16>(e4m3, head_dim, num_kv_heads, num_pages, k_cache,
                                         v_cache, k_new, v_new, k_scale, v_scale, slots,
                                         n_tokens, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_kv_append(int dtype, int head_dim, int num_kv_heads, int64_t num_pages,
                            void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* slots, int32_t n_tokens, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const int row_vecs = head_dim * elem_size(dtype) / 16;
  const int64_t total = 2 * (int64_t)n_tokens * num_kv_heads * row_vecs;
  hipLaunchKernelGGL(kv_append_kernel, dim3(grid_for(total)), dim3(kCopyThreads), 0, stream,
                     (char*)k_cache, (char*)v_cache, (const char*)k_new, (const char*)v_new,
                     slots, n_tokens, num_kv_heads, row_vecs, num_pages * kPageSize);
  return hipGetLastError();
}

hipError_t launch_gather(int dtype, int head_dim, int num_kv_heads, int64_t num_pages,
                         const void* k_cache, const void* v_cache, const int32_t* table_row,
                         int32_t len, void* k_out, void* v_out, hipStream_t stream) {
  if (len == 0) return hipSuccess;
  const int row_vecs = head_dim * elem_size(dtype) / 16;
  const int64_t total = 2 * (int64_t)len * num_kv_heads * row_vecs;
  hipLaunchKernelGGL(gather_kernel, dim3(grid_for(total)), dim3(kCopyThreads), 0, stream,
                     (const char*)k_cache, (const char*)v_cache, table_row, len, num_kv_heads,
                     row_vecs, num_pages, (char*)k_out, (char*)v_out, elem_size(dtype));
  return hipGetLastError();
}

}  // namespace pkv
