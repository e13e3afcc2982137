// C-ABI host layer of libpkv: argument checks, the decode split plan and
// kernel launches on the caller's stream.  See include/pkv.h for the contract.
#include "pkv.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "pkv_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return PKV_OK;
}

bool is_fp8(int dtype) { return dtype == PKV_FP8_E4M3 || dtype == PKV_FP8_E5M2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dtype(int dtype) {
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16 && !is_fp8(dtype))
    return fail(PKV_ERR_INVALID, "dtype %d is not a pkv_dtype", dtype);
  return PKV_OK;
}

// Types of queries and outputs: f32, f16, bf16.
int check_value_dtype(int dtype, const char* what) {
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(is_fp8(dtype) ? PKV_ERR_UNSUPPORTED : PKV_ERR_INVALID,
                "%s dtype %d: f32, f16 or bf16 expected", what, dtype);
  return PKV_OK;
}

bool finite_positive(float x) { return x > 0.f && x <= 3.4028234663852886e38f; }

int check_desc(const pkv_cache_desc* d) {
  if (!d) return fail(PKV_ERR_INVALID, "desc is NULL");
  if (d->num_pages <= 0) return fail(PKV_ERR_INVALID, "num_pages %d <= 0", d->num_pages);
  if (d->page_size <= 0) return fail(PKV_ERR_INVALID, "page_size %d <= 0", d->page_size);
  if (d->num_kv_heads <= 0) return fail(PKV_ERR_INVALID, "num_kv_heads %d <= 0", d->num_kv_heads);
  if (d->head_dim <= 0) return fail(PKV_ERR_INVALID, "head_dim %d <= 0", d->head_dim);
  if (int rc = check_dtype(d->dtype)) return rc;
  if (d->page_size != pkv::kPageSize)
    return fail(PKV_ERR_UNSUPPORTED, "page_size %d: only %d is built", d->page_size,
                pkv::kPageSize);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", d->head_dim);
  return PKV_OK;
}

// G = 16 is decoded on the matrix cores only.
int check_decode_group(const pkv_cache_desc* d, int q_dtype, int group) {
  if (group == 16 && !pkv::decode_mfma_supported(d->dtype, q_dtype, d->head_dim, 16))
    return fail(PKV_ERR_UNSUPPORTED,
                "16 query heads per KV head: decode is built for head_dim 128 with f16 or bf16 "
                "queries only");
  return PKV_OK;
}

int check_heads(const pkv_cache_desc* d, int32_t num_q_heads, int* group) {
  if (num_q_heads <= 0) return fail(PKV_ERR_INVALID, "num_q_heads %d <= 0", num_q_heads);
  if (num_q_heads % d->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, d->num_kv_heads);
  const int g = num_q_heads / d->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
    return fail(PKV_ERR_UNSUPPORTED,
                "query heads per KV head %d: only 1, 2, 4, 8, 16 are built", g);
  *group = g;
  return PKV_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ---- PKV_CHECK: device-table checks for debugging.  With the environment
// variable PKV_CHECK set (to anything but "" or "0", read at every call), a
// call that reads device tables first copies them to the host on its stream
// (which synchronises the stream), checks the preconditions the kernels
// otherwise only report as NaN rows, and returns PKV_ERR_INVALID with a
// "PKV_CHECK: ..." message instead of launching when one is broken.

bool check_mode() {
  const char* e = std::getenv("PKV_CHECK");
  return e && *e && std::strcmp(e, "0") != 0;
}

int fetch_i32(const int32_t* dev, int64_t n, std::vector<int32_t>* out, hipStream_t s) {
  out->assign((size_t)(n > 0 ? n : 0), 0);
  if (n <= 0) return PKV_OK;
  hipError_t e = hipMemcpyAsync(out->data(), dev, (size_t)n * sizeof(int32_t),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "PKV_CHECK copy: %s", hipGetErrorString(e));
  return PKV_OK;
}

// Page ids of logical pages [first, last) of table row b.
int check_pages(const pkv_cache_desc* d, const std::vector<int32_t>& bt, int32_t stride,
                int32_t b, int64_t first, int64_t last, const char* what) {
  for (int64_t i = first; i < last; ++i) {
    const int32_t pg = bt[(size_t)((int64_t)b * stride + i)];
    if (pg < 0 || pg >= d->num_pages)
      return fail(PKV_ERR_INVALID, "PKV_CHECK: %s block_table[%d][%lld] = %d outside [0, %d)",
                  what, b, (long long)i, pg, d->num_pages);
  }
  return PKV_OK;
}

// Decode: lengths within [0, max_len] and the pages the kernel reads valid
// (with a window, only the sink's pages and the window's).
int debug_check_decode(const pkv_cache_desc* d, const int32_t* block_table, int32_t stride,
                       const int32_t* lens, int32_t batch, int32_t max_len, int32_t window,
                       int32_t sink, hipStream_t s) {
  std::vector<int32_t> bt, ln;
  if (int rc = fetch_i32(lens, batch, &ln, s)) return rc;
  if (int rc = fetch_i32(block_table, (int64_t)batch * stride, &bt, s)) return rc;
  const int P = d->page_size;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = ln[(size_t)b];
    if (L < 0 || L > max_len)
      return fail(PKV_ERR_INVALID, "PKV_CHECK: decode context_lens[%d] = %lld outside [0, %d]",
                  b, (long long)L, max_len);
    const int64_t pages = (L + P - 1) / P;
    if (window > 0 && L > window) {
      const int64_t sink_pages = ((int64_t)(sink < L ? sink : L) + P - 1) / P;
      if (int rc = check_pages(d, bt, stride, b, 0, sink_pages, "decode")) return rc;
      if (int rc = check_pages(d, bt, stride, b, (L - window) / P, pages, "decode")) return rc;
    } else if (int rc = check_pages(d, bt, stride, b, 0, pages, "decode")) {
      return rc;
    }
  }
  return PKV_OK;
}

// Chunked prefill over sequences [0, batch): q_indptr non-decreasing from >= 0
// and ending <= total_rows, chunk lengths <= max_q_len and <= kv_lens <=
// max_kv_len, the pages of every kv_len valid.  With num_decode > 0 the first
// num_decode sequences must be one-row chunks at rows 0 .. num_decode-1.
int debug_check_prefill(const pkv_cache_desc* d, const int32_t* q_indptr,
                        const int32_t* block_table, int32_t stride, const int32_t* kv_lens,
                        int32_t batch, int32_t total_rows, int32_t max_q_len,
                        int32_t max_kv_len, int32_t num_decode, hipStream_t s) {
  std::vector<int32_t> ip, bt, ln;
  if (int rc = fetch_i32(q_indptr, (int64_t)batch + 1, &ip, s)) return rc;
  if (int rc = fetch_i32(kv_lens, batch, &ln, s)) return rc;
  if (int rc = fetch_i32(block_table, (int64_t)batch * stride, &bt, s)) return rc;
  const int P = d->page_size;
  if (ip[0] < 0) return fail(PKV_ERR_INVALID, "PKV_CHECK: q_indptr[0] = %d < 0", ip[0]);
  if (ip[(size_t)batch] > total_rows)
    return fail(PKV_ERR_INVALID, "PKV_CHECK: q_indptr[%d] = %d > total_q_rows %d", batch,
                ip[(size_t)batch], total_rows);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t C = (int64_t)ip[(size_t)b + 1] - ip[(size_t)b];
    const int64_t L = ln[(size_t)b];
    if (b < num_decode && (ip[(size_t)b] != b || C != 1))
      return fail(PKV_ERR_INVALID,
                  "PKV_CHECK: decode row %d: q_indptr[%d..%d] = %d..%d, want %d..%d", b, b,
                  b + 1, ip[(size_t)b], ip[(size_t)b + 1], b, b + 1);
    if (b >= num_decode && (C < 0 || C > max_q_len))
      return fail(PKV_ERR_INVALID, "PKV_CHECK: chunk %d has %lld rows, outside [0, %d]", b,
                  (long long)C, max_q_len);
    if (L < C || L > max_kv_len)
      return fail(PKV_ERR_INVALID, "PKV_CHECK: kv_lens[%d] = %lld outside [%lld, %d]", b,
                  (long long)L, (long long)C, max_kv_len);
    if (int rc = check_pages(d, bt, stride, b, 0, (L + P - 1) / P, "prefill")) return rc;
  }
  return PKV_OK;
}

// Append: slots below num_pages * page_size, each used once (negative: skip).
int debug_check_slots(const pkv_cache_desc* d, const int32_t* slots, int32_t n, hipStream_t s) {
  std::vector<int32_t> sl;
  if (int rc = fetch_i32(slots, n, &sl, s)) return rc;
  const int64_t total = (int64_t)d->num_pages * d->page_size;
  std::unordered_set<int32_t> seen;
  seen.reserve((size_t)n * 2);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t v = sl[(size_t)i];
    if (v < 0) continue;
    if (v >= total)
      return fail(PKV_ERR_INVALID, "PKV_CHECK: slot[%d] = %d >= num_pages * page_size = %lld",
                  i, v, (long long)total);
    if (!seen.insert(v).second)
      return fail(PKV_ERR_INVALID, "PKV_CHECK: slot %d repeats (index %d)", v, i);
  }
  return PKV_OK;
}

// Decode split plan.  Auto rule: aim for about 512 workgroups (two per CU
// on a 256-CU device, one round of residency) for the vector decode kernel,
// 256 (one per CU) for the matrix-core kernel, whose workgroups each keep more
// bytes in flight; never less than 16 pages (256 keys) per split, and no
// split at all for contexts of at most 32 pages.
struct Plan {
  int32_t n_split;
  int32_t pages_per_split;
  size_t o_bytes;      // partial outputs, rounded up to 256
  size_t ws_bytes;     // o_bytes + lse bytes
};

constexpr int64_t kTargetWorkgroups = 512;
constexpr int64_t kTargetWorkgroupsMfma = 256;
constexpr int32_t kXcdSplitTiles = 64;    // prefill: query tiles per (b, kv head)
constexpr int32_t kMinSplitPages = 16;
// Contexts of at most this many pages are not split: the merge launch costs
// more than the shorter workgroups save (the tiny batch, 4 x 8 units of up to
// 32 pages: 13.9 us in one launch against 16.5 us split in two plus the merge).
constexpr int64_t kNoSplitPages = 32;
// Splits for batches of unequal lengths (pkv_decode_split_for_lens): small
// enough that about 1024 workgroups (four per CU) carry the batch, so that the
// hardware balances the uneven tails, and at least 32 pages each.
constexpr int64_t kUnevenWorkgroups = 1024;
constexpr int64_t kUnevenMinPages = 32;

int make_plan(const pkv_cache_desc* d, int32_t batch, int32_t num_q_heads,
              int32_t max_context_len, int32_t split_tokens, int q_dtype, Plan* plan) {
  const int P = d->page_size;
  const int64_t max_pages = ((int64_t)max_context_len + P - 1) / P;
  int64_t pps;
  if (split_tokens > 0) {
    if (split_tokens % P != 0)
      return fail(PKV_ERR_INVALID, "split_tokens %d is not a multiple of page_size %d",
                  split_tokens, P);
    pps = split_tokens / P;
  } else if (split_tokens == 0) {
    const int64_t units = (int64_t)batch * d->num_kv_heads;
    const int group = d->num_kv_heads > 0 ? num_q_heads / d->num_kv_heads : 1;
    const int64_t target = pkv::decode_mfma_supported(d->dtype, q_dtype, d->head_dim, group)
                               ? kTargetWorkgroupsMfma
                               : kTargetWorkgroups;
    int64_t want = units > 0 ? (target + units - 1) / units : 1;
    const int64_t cap = (max_pages + kMinSplitPages - 1) / kMinSplitPages;
    if (want > cap) want = cap;
    if (max_pages <= kNoSplitPages) want = 1;
    if (want < 1) want = 1;
    pps = (max_pages + want - 1) / want;
    if (pps < 1) pps = 1;
  } else {
    return fail(PKV_ERR_INVALID, "split_tokens %d < 0", split_tokens);
  }
  int64_t n = max_pages > 0 ? (max_pages + pps - 1) / pps : 1;
  if (n < 1) n = 1;
  if (n > (1 << 20) || pps > (1 << 30)) return fail(PKV_ERR_INVALID, "split plan out of range");
  plan->n_split = (int32_t)n;
  plan->pages_per_split = (int32_t)pps;
  const size_t rows = (size_t)batch * num_q_heads;
  const size_t ob = rows * (size_t)n * d->head_dim * sizeof(float);
  plan->o_bytes = (ob + 255) & ~(size_t)255;
  plan->ws_bytes = plan->o_bytes + rows * (size_t)n * sizeof(float);
  return PKV_OK;
}

struct DecodeCommon {
  int group;
  Plan plan;
  pkv_decode_opts opts;   // resolved (defaults filled in)
};

// Options with their defaults, checked against the cache descriptor.
int resolve_opts(const pkv_cache_desc* desc, const pkv_decode_opts* in, pkv_decode_opts* out) {
  if (in) {
    *out = *in;
  } else {
    out->q_dtype = desc->dtype;
    out->k_scale = 1.f;
    out->v_scale = 1.f;
    out->window = 0;
    out->sink = 0;
  }
  if (is_fp8(desc->dtype)) {
    if (out->q_dtype != PKV_F16 && out->q_dtype != PKV_BF16)
      return fail(in ? PKV_ERR_UNSUPPORTED : PKV_ERR_INVALID,
                  "fp8 caches need pkv_decode_opts with q_dtype f16 or bf16 (got %d)",
                  out->q_dtype);
    if (desc->head_dim != 128)
      return fail(PKV_ERR_UNSUPPORTED, "fp8 caches are built for head_dim 128 (got %d)",
                  desc->head_dim);
    if (!finite_positive(out->k_scale) || !finite_positive(out->v_scale))
      return fail(PKV_ERR_INVALID, "k_scale and v_scale must be finite and > 0");
  } else {
    if (out->q_dtype != desc->dtype)
      return fail(PKV_ERR_INVALID, "q_dtype %d differs from the cache dtype %d", out->q_dtype,
                  desc->dtype);
    if (out->k_scale != 1.f || out->v_scale != 1.f)
      return fail(PKV_ERR_INVALID, "k_scale / v_scale apply to fp8 caches only (must be 1)");
  }
  if (out->window < 0 || out->sink < 0)
    return fail(PKV_ERR_INVALID, "window %d and sink %d must be >= 0", out->window, out->sink);
  return PKV_OK;
}

// Upper bound on the keys a sequence of at most max_len keys exposes to the
// split plan: with a window, only its pages and the sink's are visited.
int32_t plan_len(int32_t max_len, const pkv_decode_opts& o, int P) {
  if (o.window <= 0) return max_len;
  const int64_t pages = ((int64_t)o.sink + P - 1) / P + ((int64_t)o.window + P - 1) / P + 1;
  const int64_t bound = pages * P;
  return bound < max_len ? (int32_t)bound : max_len;
}

int check_decode(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                 const void* q, int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                 int32_t stride, const int32_t* context_lens, int32_t max_context_len,
                 float scale, int32_t split_tokens, const pkv_decode_opts* opts,
                 DecodeCommon* dc) {
  if (int rc = check_desc(desc)) return rc;
  if (int rc = resolve_opts(desc, opts, &dc->opts)) return rc;
  if (int rc = check_heads(desc, num_q_heads, &dc->group)) return rc;
  if (int rc = check_decode_group(desc, dc->opts.q_dtype, dc->group)) return rc;
  if (batch < 0) return fail(PKV_ERR_INVALID, "batch %d < 0", batch);
  if (stride <= 0) return fail(PKV_ERR_INVALID, "block_table_stride %d <= 0", stride);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)stride * desc->page_size)
    return fail(PKV_ERR_INVALID, "max_context_len %d outside [0, stride * page_size = %lld]",
                max_context_len, (long long)stride * desc->page_size);
  if (!(scale == scale)) return fail(PKV_ERR_INVALID, "scale is NaN");
  if (batch > 0) {
    if (!k_cache || !v_cache || !q || !block_table || !context_lens)
      return fail(PKV_ERR_INVALID, "NULL input pointer");
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q))
      return fail(PKV_ERR_INVALID, "k_cache, v_cache and q must be 16-byte aligned");
  }
  if (int rc = make_plan(desc, batch, num_q_heads,
                         plan_len(max_context_len, dc->opts, desc->page_size), split_tokens,
                         dc->opts.q_dtype, &dc->plan))
    return rc;
  // the split-major grid pads the units to a multiple of 8 (pkv::decode_grid)
  const int64_t units = (int64_t)batch * desc->num_kv_heads;
  const int64_t blocks = (units + 7) / 8 * 8 * dc->plan.n_split;
  if (blocks > 0x7fffffff) return fail(PKV_ERR_INVALID, "grid too large (%lld)", (long long)blocks);
  return PKV_OK;
}

pkv::DecodeArgs decode_args(const pkv_cache_desc* desc, const void* k_cache,
                            const void* v_cache, const void* q, int32_t num_q_heads,
                            const int32_t* block_table, int32_t stride,
                            const int32_t* context_lens, float scale, const DecodeCommon& dc,
                            int32_t batch) {
  const Plan& plan = dc.plan;
  pkv::DecodeArgs a{};
  a.n_units = batch * desc->num_kv_heads;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.q = q;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.num_pages = desc->num_pages;
  a.stride = stride;
  a.num_kv_heads = desc->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.pages_per_split = plan.pages_per_split;
  a.n_split = plan.n_split;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634 * (double)dc.opts.k_scale);
  a.v_scale = dc.opts.v_scale;
  a.window = dc.opts.window;
  a.sink = dc.opts.sink;
  a.part_stride = plan.n_split;
  a.part_offset = 0;
  a.k_quant = dc.opts.k_scale;
  a.v_quant = dc.opts.v_scale;
  return a;
}

// The newest-token rows of the decode-with-append calls: both or neither
// (plain decode), 16-byte aligned when the batch is not empty.
int check_new_rows(int32_t batch, const void* k_new, const void* v_new, bool append) {
  if (!append || batch == 0) return PKV_OK;
  if (!k_new || !v_new) return fail(PKV_ERR_INVALID, "k_new / v_new is NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
  return PKV_OK;
}

// The decode kernel for these types and shapes: matrix cores for grouped
// 16-bit queries (G >= 4, head_dim 128), the vector kernel otherwise.
hipError_t launch_any_decode(const pkv_cache_desc* desc, int q_dtype, int group, int batch,
                             const pkv::DecodeArgs& a, hipStream_t s) {
  if (pkv::decode_mfma_supported(desc->dtype, q_dtype, desc->head_dim, group))
    return pkv::launch_decode_mfma(desc->dtype, q_dtype, group, batch, a, s);
  return pkv::launch_decode(desc->dtype, q_dtype, desc->head_dim, group, batch, a, s);
}

int decode_impl(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                const void* q, int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                int32_t block_table_stride, const int32_t* context_lens, int32_t max_context_len,
                float scale, int32_t split_tokens, const pkv_decode_opts* opts, void* out,
                float* lse_out, void* workspace, size_t workspace_bytes, void* stream,
                const void* k_new = nullptr, const void* v_new = nullptr, bool append = false) {
  DecodeCommon dc;
  if (int rc = check_decode(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                            block_table_stride, context_lens, max_context_len, scale,
                            split_tokens, opts, &dc))
    return rc;
  if (int rc = check_new_rows(batch, k_new, v_new, append)) return rc;
  if (batch == 0) return ok();
  if (!out) return fail(PKV_ERR_INVALID, "out is NULL");
  if (check_mode())
    if (int rc = debug_check_decode(desc, block_table, block_table_stride, context_lens, batch,
                                    max_context_len, dc.opts.window, dc.opts.sink,
                                    (hipStream_t)stream))
      return rc;
  pkv::DecodeArgs a = decode_args(desc, k_cache, v_cache, q, num_q_heads, block_table,
                                  block_table_stride, context_lens, scale, dc, batch);
  a.k_new = append ? k_new : nullptr;
  a.v_new = append ? v_new : nullptr;
  hipStream_t s = (hipStream_t)stream;
  const int qdt = dc.opts.q_dtype;
  if (dc.plan.n_split == 1) {
    a.direct = 1;
    a.out = out;
    a.lse_out = lse_out;
    return hip_status(
        launch_any_decode(desc, qdt, dc.group, batch, a, s),
        "decode launch");
  }
  if (!workspace || workspace_bytes < dc.plan.ws_bytes)
    return fail(PKV_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes,
                dc.plan.ws_bytes);
  if (!aligned16(workspace)) return fail(PKV_ERR_INVALID, "workspace must be 16-byte aligned");
  a.direct = 0;
  a.o_part = (float*)workspace;
  a.lse_part = (float*)((char*)workspace + dc.plan.o_bytes);
  if (int rc = hip_status(
          launch_any_decode(desc, qdt, dc.group, batch, a, s),
          "decode launch"))
    return rc;
  return hip_status(pkv::launch_merge(qdt, desc->head_dim, a.o_part, a.lse_part,
                                      batch * num_q_heads, dc.plan.n_split, out, lse_out, s),
                    "merge launch");
}

int partials_impl(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                  const void* q, int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                  int32_t block_table_stride, const int32_t* context_lens,
                  int32_t max_context_len, float scale, int32_t split_tokens,
                  const pkv_decode_opts* opts, void* workspace, size_t workspace_bytes,
                  void* stream, const void* k_new = nullptr, const void* v_new = nullptr,
                  bool append = false) {
  DecodeCommon dc;
  if (int rc = check_decode(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                            block_table_stride, context_lens, max_context_len, scale,
                            split_tokens, opts, &dc))
    return rc;
  if (int rc = check_new_rows(batch, k_new, v_new, append)) return rc;
  if (batch == 0) return ok();
  if (!workspace || workspace_bytes < dc.plan.ws_bytes)
    return fail(PKV_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes,
                dc.plan.ws_bytes);
  if (!aligned16(workspace)) return fail(PKV_ERR_INVALID, "workspace must be 16-byte aligned");
  if (check_mode())
    if (int rc = debug_check_decode(desc, block_table, block_table_stride, context_lens, batch,
                                    max_context_len, dc.opts.window, dc.opts.sink,
                                    (hipStream_t)stream))
      return rc;
  pkv::DecodeArgs a = decode_args(desc, k_cache, v_cache, q, num_q_heads, block_table,
                                  block_table_stride, context_lens, scale, dc, batch);
  a.k_new = append ? k_new : nullptr;
  a.v_new = append ? v_new : nullptr;
  a.direct = 0;
  a.o_part = (float*)workspace;
  a.lse_part = (float*)((char*)workspace + dc.plan.o_bytes);
  return hip_status(launch_any_decode(desc, dc.opts.q_dtype, dc.group, batch, a,
                                     (hipStream_t)stream),
                    "decode launch");
}

int plan_impl(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
              int32_t max_context_len, int32_t split_tokens, const pkv_decode_opts* opts,
              int32_t* n_split, size_t* workspace_bytes) {
  if (int rc = check_desc(desc)) return rc;
  pkv_decode_opts o;
  if (int rc = resolve_opts(desc, opts, &o)) return rc;
  int group = 0;
  if (int rc = check_heads(desc, num_q_heads, &group)) return rc;
  if (int rc = check_decode_group(desc, o.q_dtype, group)) return rc;
  if (batch < 0) return fail(PKV_ERR_INVALID, "batch %d < 0", batch);
  if (max_context_len < 0) return fail(PKV_ERR_INVALID, "max_context_len %d < 0", max_context_len);
  if (!n_split || !workspace_bytes) return fail(PKV_ERR_INVALID, "NULL output pointer");
  Plan plan;
  if (int rc = make_plan(desc, batch, num_q_heads,
                         plan_len(max_context_len, o, desc->page_size), split_tokens, o.q_dtype,
                         &plan))
    return rc;
  *n_split = plan.n_split;
  *workspace_bytes = plan.n_split > 1 ? plan.ws_bytes : 0;
  return ok();
}

}  // namespace

extern "C" {

int pkv_version(void) { return PKV_VERSION; }

const char* pkv_last_error(void) { return g_err.c_str(); }

int pkv_kv_append(const pkv_cache_desc* desc, void* k_cache, void* v_cache, const void* k_new,
                  const void* v_new, const int32_t* slot_mapping, int32_t n_tokens,
                  void* stream) {
  if (int rc = check_desc(desc)) return rc;
  if (n_tokens < 0) return fail(PKV_ERR_INVALID, "n_tokens %d < 0", n_tokens);
  if (n_tokens == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
    return fail(PKV_ERR_INVALID, "NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_ERR_INVALID, "cache and new-token buffers must be 16-byte aligned");
  if (check_mode())
    if (int rc = debug_check_slots(desc, slot_mapping, n_tokens, (hipStream_t)stream)) return rc;
  return hip_status(pkv::launch_kv_append(desc->dtype, desc->head_dim, desc->num_kv_heads,
                                          desc->num_pages, k_cache, v_cache, k_new, v_new,
                                          slot_mapping, n_tokens, (hipStream_t)stream),
                    "kv_append launch");
}

int pkv_gather_kv(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                  const int32_t* table_row, int32_t len, void* k_out, void* v_out,
                  void* stream) {
  if (int rc = check_desc(desc)) return rc;
  if (len < 0) return fail(PKV_ERR_INVALID, "len %d < 0", len);
  if (len == 0) return ok();
  if (!k_cache || !v_cache || !table_row || !k_out || !v_out)
    return fail(PKV_ERR_INVALID, "NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_out) || !aligned16(v_out))
    return fail(PKV_ERR_INVALID, "buffers must be 16-byte aligned");
  if (check_mode()) {
    std::vector<int32_t> row;
    const int64_t pages = ((int64_t)len + desc->page_size - 1) / desc->page_size;
    if (int rc = fetch_i32(table_row, pages, &row, (hipStream_t)stream)) return rc;
    if (int rc = check_pages(desc, row, (int32_t)pages, 0, 0, pages, "gather")) return rc;
  }
  return hip_status(pkv::launch_gather(desc->dtype, desc->head_dim, desc->num_kv_heads,
                                       desc->num_pages, k_cache, v_cache, table_row, len, k_out,
                                       v_out, (hipStream_t)stream),
                    "gather launch");
}

int pkv_decode_plan(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                    int32_t max_context_len, int32_t split_tokens, int32_t* n_split,
                    size_t* workspace_bytes) {
  return plan_impl(desc, batch, num_q_heads, max_context_len, split_tokens, nullptr, n_split,
                   workspace_bytes);
}

int pkv_decode_plan_ex(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                       int32_t max_context_len, int32_t split_tokens,
                       const pkv_decode_opts* opts, int32_t* n_split, size_t* workspace_bytes) {
  return plan_impl(desc, batch, num_q_heads, max_context_len, split_tokens, opts, n_split,
                   workspace_bytes);
}

int pkv_decode_split_for_lens(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                              const int32_t* lens_host, const pkv_decode_opts* opts,
                              int32_t* split_tokens) {
  if (int rc = check_desc(desc)) return rc;
  pkv_decode_opts o;
  if (int rc = resolve_opts(desc, opts, &o)) return rc;
  int group = 0;
  if (int rc = check_heads(desc, num_q_heads, &group)) return rc;
  if (int rc = check_decode_group(desc, o.q_dtype, group)) return rc;
  if (batch < 0) return fail(PKV_ERR_INVALID, "batch %d < 0", batch);
  if (!split_tokens || (batch > 0 && !lens_host)) return fail(PKV_ERR_INVALID, "NULL pointer");
  const int P = desc->page_size;
  // pages the decode visits (and the split plan counts) for each sequence
  int64_t total = 0, lo = -1, hi = -1;
  int32_t max_len = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = lens_host[b];
    if (L < 0) return fail(PKV_ERR_INVALID, "lens[%d] = %lld < 0", b, (long long)L);
    if (L > max_len) max_len = (int32_t)L;
    const int64_t pages = (L + P - 1) / P;
    int64_t v = pages;
    if (o.window > 0 && L > o.window) {
      const int64_t sink_pages = ((o.sink < L ? (int64_t)o.sink : L) + P - 1) / P;
      const int64_t first = (L - o.window) / P;
      v = sink_pages + (pages - (first > sink_pages ? first : sink_pages));
    }
    total += v;
    lo = (lo < 0 || v < lo) ? v : lo;
    hi = v > hi ? v : hi;
  }
  int64_t pps;
  if (lo == hi) {
    // equal sequences divide evenly: the automatic split
    Plan plan;
    if (int rc = make_plan(desc, batch, num_q_heads, plan_len(max_len, o, P), 0, o.q_dtype,
                           &plan))
      return rc;
    pps = plan.pages_per_split;
  } else {
    // about kUnevenWorkgroups equal splits over the pages the batch visits;
    // the split-major grid hands the first splits (the longest work) out
    // first and spreads every round over the XCDs
    pps = (total * desc->num_kv_heads + kUnevenWorkgroups - 1) / kUnevenWorkgroups;
    if (pps < kUnevenMinPages) pps = kUnevenMinPages;
  }
  if (pps * P > 0x7fffffff) return fail(PKV_ERR_INVALID, "split out of range");
  *split_tokens = (int32_t)(pps * P);
  return ok();
}

int pkv_paged_attn_decode(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                          const void* q, int32_t batch, int32_t num_q_heads,
                          const int32_t* block_table, int32_t block_table_stride,
                          const int32_t* context_lens, int32_t max_context_len, float scale,
                          int32_t split_tokens, void* out, float* lse_out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_impl(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                     block_table_stride, context_lens, max_context_len, scale, split_tokens,
                     nullptr, out, lse_out, workspace, workspace_bytes, stream);
}

int pkv_paged_attn_decode_ex(const pkv_cache_desc* desc, const void* k_cache,
                             const void* v_cache, const void* q, int32_t batch,
                             int32_t num_q_heads, const int32_t* block_table,
                             int32_t block_table_stride, const int32_t* context_lens,
                             int32_t max_context_len, float scale, int32_t split_tokens,
                             const pkv_decode_opts* opts, void* out, float* lse_out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                     block_table_stride, context_lens, max_context_len, scale, split_tokens,
                     opts, out, lse_out, workspace, workspace_bytes, stream);
}

int pkv_paged_attn_decode_partials(const pkv_cache_desc* desc, const void* k_cache,
                                   const void* v_cache, const void* q, int32_t batch,
                                   int32_t num_q_heads, const int32_t* block_table,
                                   int32_t block_table_stride, const int32_t* context_lens,
                                   int32_t max_context_len, float scale, int32_t split_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return partials_impl(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                       block_table_stride, context_lens, max_context_len, scale, split_tokens,
                       nullptr, workspace, workspace_bytes, stream);
}

int pkv_paged_attn_decode_partials_ex(const pkv_cache_desc* desc, const void* k_cache,
                                      const void* v_cache, const void* q, int32_t batch,
                                      int32_t num_q_heads, const int32_t* block_table,
                                      int32_t block_table_stride, const int32_t* context_lens,
                                      int32_t max_context_len, float scale,
                                      int32_t split_tokens, const pkv_decode_opts* opts,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return partials_impl(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                       block_table_stride, context_lens, max_context_len, scale, split_tokens,
                       opts, workspace, workspace_bytes, stream);
}

int pkv_paged_attn_decode_append(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                                 const void* k_new, const void* v_new, const void* q,
                                 int32_t batch, int32_t num_q_heads, const int32_t* block_table,
                                 int32_t block_table_stride, const int32_t* context_lens,
                                 int32_t max_context_len, float scale, int32_t split_tokens,
                                 const pkv_decode_opts* opts, void* out, float* lse_out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                     block_table_stride, context_lens, max_context_len, scale, split_tokens, opts,
                     out, lse_out, workspace, workspace_bytes, stream, k_new, v_new, true);
}

int pkv_paged_attn_decode_append_partials(
    const pkv_cache_desc* desc, void* k_cache, void* v_cache, const void* k_new,
    const void* v_new, const void* q, int32_t batch, int32_t num_q_heads,
    const int32_t* block_table, int32_t block_table_stride, const int32_t* context_lens,
    int32_t max_context_len, float scale, int32_t split_tokens, const pkv_decode_opts* opts,
    void* workspace, size_t workspace_bytes, void* stream) {
  return partials_impl(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                       block_table_stride, context_lens, max_context_len, scale, split_tokens,
                       opts, workspace, workspace_bytes, stream, k_new, v_new, true);
}

// ---- the decode step without a caller workspace (pkv_paged_attn_decode_append_noalloc)
//
// Its split-KV partials go to a file-scope device array, one copy per GPU,
// held for the life of the process.  In host code `scratch` names a host-side
// stand-in, not the device array: its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is passed to kernels.
namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_HIP, "no current HIP device for the scratch array (device %d)", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

size_t pkv_noalloc_scratch_bytes(void) { return kScratchBytes; }

int pkv_paged_attn_decode_append_noalloc(const pkv_cache_desc* desc, void* k_cache,
                                         void* v_cache, const void* k_new, const void* v_new,
                                         const void* q, int32_t batch, int32_t num_q_heads,
                                         const int32_t* block_table, int32_t block_table_stride,
                                         const int32_t* context_lens, int32_t max_context_len,
                                         float scale, int32_t split_tokens,
                                         const pkv_decode_opts* opts, void* out, float* lse_out,
                                         void* stream) {
  DecodeCommon dc;
  if (int rc = check_decode(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                            block_table_stride, context_lens, max_context_len, scale,
                            split_tokens, opts, &dc))
    return rc;
  if (dc.plan.n_split > 1 && dc.plan.ws_bytes > kScratchBytes)
    return fail(PKV_ERR_WORKSPACE,
                "the split plan needs %zu bytes of partials, over the %zu-byte static scratch "
                "(fewer splits: a larger split_tokens)",
                dc.plan.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  if (batch > 0 && dc.plan.n_split > 1)
    if (int rc = scratch_address(&ws)) return rc;
  return decode_impl(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                     block_table_stride, context_lens, max_context_len, scale, split_tokens,
                     opts, out, lse_out, ws, ws ? kScratchBytes : 0, stream, k_new, v_new, true);
}

int pkv_kv_append_quant(const pkv_cache_desc* desc, void* k_cache, void* v_cache,
                        const void* k_new, const void* v_new, int32_t src_dtype, float k_scale,
                        float v_scale, const int32_t* slot_mapping, int32_t n_tokens,
                        void* stream) {
  if (int rc = check_desc(desc)) return rc;
  if (!is_fp8(desc->dtype))
    return fail(PKV_ERR_INVALID, "kv_append_quant writes fp8 caches (dtype %d)", desc->dtype);
  if (int rc = check_value_dtype(src_dtype, "source")) return rc;
  if (!finite_positive(k_scale) || !finite_positive(v_scale))
    return fail(PKV_ERR_INVALID, "k_scale and v_scale must be finite and > 0");
  if (n_tokens < 0) return fail(PKV_ERR_INVALID, "n_tokens %d < 0", n_tokens);
  if (n_tokens == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
    return fail(PKV_ERR_INVALID, "NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_ERR_INVALID, "cache and new-token buffers must be 16-byte aligned");
  if (check_mode())
    if (int rc = debug_check_slots(desc, slot_mapping, n_tokens, (hipStream_t)stream)) return rc;
  return hip_status(pkv::launch_kv_append_quant(desc->dtype, src_dtype, desc->head_dim,
                                                desc->num_kv_heads, desc->num_pages, k_cache,
                                                v_cache, k_new, v_new, k_scale, v_scale,
                                                slot_mapping, n_tokens, (hipStream_t)stream),
                    "kv_append_quant launch");
}

int pkv_merge_states(const float* o_parts, const float* lse_parts, int32_t rows,
                     int32_t n_parts, int32_t head_dim, int32_t out_dtype, void* out,
                     float* lse_out, void* stream) {
  if (rows < 0) return fail(PKV_ERR_INVALID, "rows %d < 0", rows);
  if (n_parts <= 0) return fail(PKV_ERR_INVALID, "n_parts %d <= 0", n_parts);
  if (head_dim <= 0) return fail(PKV_ERR_INVALID, "head_dim %d <= 0", head_dim);
  if (int rc = check_value_dtype(out_dtype, "out")) return rc;
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", head_dim);
  if (rows == 0) return ok();
  if (!o_parts || !lse_parts || !out) return fail(PKV_ERR_INVALID, "NULL pointer");
  if (!aligned16(o_parts)) return fail(PKV_ERR_INVALID, "o_parts must be 16-byte aligned");
  return hip_status(pkv::launch_merge(out_dtype, head_dim, o_parts, lse_parts, rows, n_parts,
                                      out, lse_out, (hipStream_t)stream),
                    "merge launch");
}

namespace {

// Checks and launch of the chunked-prefill kernel for sequences
// [0, batch) of the given (already offset) tables.  opts (nullable): the
// query type and fp8 pool scales; window and sink must be 0.
int prefill_checks(const pkv_cache_desc* desc, int32_t num_q_heads, int32_t batch,
                   int32_t total_q_rows, int32_t max_q_len, int32_t block_table_stride,
                   int32_t max_kv_len, float scale, const pkv_decode_opts* opts,
                   pkv_decode_opts* o, int* group) {
  if (int rc = check_desc(desc)) return rc;
  if (int rc = resolve_opts(desc, opts, o)) return rc;
  if (int rc = check_heads(desc, num_q_heads, group)) return rc;
  if (desc->dtype != PKV_F16 && desc->dtype != PKV_BF16 && !is_fp8(desc->dtype))
    return fail(PKV_ERR_UNSUPPORTED,
                "prefill runs on the matrix cores: f16, bf16 or fp8 pools only");
  if (desc->head_dim != 128 && !(desc->head_dim == 64 && !is_fp8(desc->dtype)))
    return fail(PKV_ERR_UNSUPPORTED,
                "prefill is built for head_dim 128, and 64 with 16-bit pools (got %d)",
                desc->head_dim);
  if (o->window != 0 || o->sink != 0)
    return fail(PKV_ERR_INVALID, "window and sink apply to decode only (got %d, %d)", o->window,
                o->sink);
  if (batch < 0) return fail(PKV_ERR_INVALID, "batch %d < 0", batch);
  if (total_q_rows < 0) return fail(PKV_ERR_INVALID, "total_q_rows %d < 0", total_q_rows);
  if (max_q_len < 0) return fail(PKV_ERR_INVALID, "max_q_len %d < 0", max_q_len);
  if (block_table_stride <= 0)
    return fail(PKV_ERR_INVALID, "block_table_stride %d <= 0", block_table_stride);
  if (max_kv_len < 0 || (int64_t)max_kv_len > (int64_t)block_table_stride * desc->page_size)
    return fail(PKV_ERR_INVALID, "max_kv_len %d outside [0, stride * page_size]", max_kv_len);
  if (max_q_len > max_kv_len)
    return fail(PKV_ERR_INVALID, "max_q_len %d > max_kv_len %d", max_q_len, max_kv_len);
  if (!(scale == scale)) return fail(PKV_ERR_INVALID, "scale is NaN");
  return PKV_OK;
}

int prefill_launch(const pkv_cache_desc* desc, int group, const pkv_decode_opts& o,
                   const void* k_cache, const void* v_cache, const void* q,
                   const int32_t* q_indptr, int32_t batch, int32_t num_q_heads,
                   int32_t total_q_rows, int32_t max_q_len, const int32_t* block_table,
                   int32_t block_table_stride, const int32_t* kv_lens, float scale, void* out,
                   float* lse_out, hipStream_t stream) {
  pkv::PrefillArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.q = q;
  a.q_indptr = q_indptr;
  a.block_table = block_table;
  a.kv_lens = kv_lens;
  a.num_pages = desc->num_pages;
  a.stride = block_table_stride;
  a.num_kv_heads = desc->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.batch = batch;
  a.max_q_len = max_q_len;
  a.total_q = total_q_rows;
  const int rows = pkv::prefill_rows_per_tile(group);
  a.m_tiles = (max_q_len + rows - 1) / rows;
  // Spread each (sequence, KV head)'s query tiles over the XCDs once there
  // are enough of them (>= 8 per XCD) to keep sharing the K/V stream in L2.
  a.xcd_split = a.m_tiles >= kXcdSplitTiles ? 1 : 0;
  a.m_tiles_x = (a.m_tiles + 7) / 8;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634 * (double)o.k_scale);
  a.v_scale = o.v_scale;
  a.out = out;
  a.lse_out = lse_out;
  const int64_t blocks = (int64_t)batch * desc->num_kv_heads *
                         (a.xcd_split ? 8 * (int64_t)a.m_tiles_x : (int64_t)a.m_tiles);
  if (blocks > 0x7fffffff) return fail(PKV_ERR_INVALID, "grid too large");
  return hip_status(
      pkv::launch_prefill(desc->dtype, o.q_dtype, desc->head_dim, group, a, stream),
      "prefill launch");
}

int prefill_impl(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                 const void* q, const int32_t* q_indptr, int32_t batch, int32_t num_q_heads,
                 int32_t total_q_rows, int32_t max_q_len, const int32_t* block_table,
                 int32_t block_table_stride, const int32_t* kv_lens, int32_t max_kv_len,
                 float scale, const pkv_decode_opts* opts, void* out, float* lse_out,
                 void* stream) {
  int group = 0;
  pkv_decode_opts o;
  if (int rc = prefill_checks(desc, num_q_heads, batch, total_q_rows, max_q_len,
                              block_table_stride, max_kv_len, scale, opts, &o, &group))
    return rc;
  if (batch == 0 || max_q_len == 0 || total_q_rows == 0) return ok();
  if (!k_cache || !v_cache || !q || !q_indptr || !block_table || !kv_lens || !out)
    return fail(PKV_ERR_INVALID, "NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(out))
    return fail(PKV_ERR_INVALID, "k_cache, v_cache, q and out must be 16-byte aligned");
  if (check_mode())
    if (int rc = debug_check_prefill(desc, q_indptr, block_table, block_table_stride, kv_lens,
                                     batch, total_q_rows, max_q_len, max_kv_len, 0,
                                     (hipStream_t)stream))
      return rc;
  return prefill_launch(desc, group, o, k_cache, v_cache, q, q_indptr, batch, num_q_heads,
                        total_q_rows, max_q_len, block_table, block_table_stride, kv_lens,
                        scale, out, lse_out, (hipStream_t)stream);
}

int mixed_impl(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
               const void* q, const int32_t* q_indptr, int32_t batch, int32_t num_decode,
               int32_t num_q_heads, int32_t total_q_rows, int32_t max_q_len,
               const int32_t* block_table, int32_t block_table_stride, const int32_t* kv_lens,
               int32_t max_kv_len, float scale, int32_t split_tokens,
               const pkv_decode_opts* opts, void* out, float* lse_out, void* workspace,
               size_t workspace_bytes, void* stream) {
  int group = 0;
  pkv_decode_opts o;
  if (int rc = prefill_checks(desc, num_q_heads, batch, total_q_rows, max_q_len,
                              block_table_stride, max_kv_len, scale, opts, &o, &group))
    return rc;
  if (num_decode < 0 || num_decode > batch || num_decode > total_q_rows)
    return fail(PKV_ERR_INVALID, "num_decode %d outside [0, min(batch %d, total_q_rows %d)]",
                num_decode, batch, total_q_rows);
  if (batch == 0 || total_q_rows == 0) return ok();
  if (!k_cache || !v_cache || !q || !q_indptr || !block_table || !kv_lens || !out)
    return fail(PKV_ERR_INVALID, "NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(out))
    return fail(PKV_ERR_INVALID, "k_cache, v_cache, q and out must be 16-byte aligned");
  const int32_t n_chunk = batch - num_decode;
  if (n_chunk > 0 && max_q_len == 0)
    return fail(PKV_ERR_INVALID, "max_q_len 0 with %d chunk sequences", n_chunk);
  if (check_mode())
    if (int rc = debug_check_prefill(desc, q_indptr, block_table, block_table_stride, kv_lens,
                                     batch, total_q_rows, max_q_len, max_kv_len, num_decode,
                                     (hipStream_t)stream))
      return rc;
  if (num_decode > 0) {
    // decode rows: q rows and out rows 0 .. num_decode-1, i.e. [num_decode][H_q][D]
    if (int rc = decode_impl(desc, k_cache, v_cache, q, num_decode, num_q_heads, block_table,
                             block_table_stride, kv_lens, max_kv_len, scale, split_tokens, opts,
                             out, lse_out, workspace, workspace_bytes, stream))
      return rc;
  }
  if (n_chunk == 0) return ok();
  return prefill_launch(desc, group, o, k_cache, v_cache, q, q_indptr + num_decode, n_chunk,
                        num_q_heads, total_q_rows, max_q_len,
                        block_table + (int64_t)num_decode * block_table_stride,
                        block_table_stride, kv_lens + num_decode, scale, out, lse_out,
                        (hipStream_t)stream);
}

}  // namespace

int pkv_paged_attn_prefill_chunk(const pkv_cache_desc* desc, const void* k_cache,
                                 const void* v_cache, const void* q, const int32_t* q_indptr,
                                 int32_t batch, int32_t num_q_heads, int32_t total_q_rows,
                                 int32_t max_q_len, const int32_t* block_table,
                                 int32_t block_table_stride, const int32_t* kv_lens,
                                 int32_t max_kv_len, float scale, void* out, float* lse_out,
                                 void* stream) {
  return prefill_impl(desc, k_cache, v_cache, q, q_indptr, batch, num_q_heads, total_q_rows,
                      max_q_len, block_table, block_table_stride, kv_lens, max_kv_len, scale,
                      nullptr, out, lse_out, stream);
}

int pkv_paged_attn_prefill_chunk_ex(const pkv_cache_desc* desc, const void* k_cache,
                                    const void* v_cache, const void* q,
                                    const int32_t* q_indptr, int32_t batch,
                                    int32_t num_q_heads, int32_t total_q_rows,
                                    int32_t max_q_len, const int32_t* block_table,
                                    int32_t block_table_stride, const int32_t* kv_lens,
                                    int32_t max_kv_len, float scale,
                                    const pkv_decode_opts* opts, void* out, float* lse_out,
                                    void* stream) {
  return prefill_impl(desc, k_cache, v_cache, q, q_indptr, batch, num_q_heads, total_q_rows,
                      max_q_len, block_table, block_table_stride, kv_lens, max_kv_len, scale,
                      opts, out, lse_out, stream);
}

int pkv_paged_attn_mixed(const pkv_cache_desc* desc, const void* k_cache, const void* v_cache,
                         const void* q, const int32_t* q_indptr, int32_t batch,
                         int32_t num_decode, int32_t num_q_heads, int32_t total_q_rows,
                         int32_t max_q_len, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* kv_lens, int32_t max_kv_len,
                         float scale, int32_t split_tokens, void* out, float* lse_out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return mixed_impl(desc, k_cache, v_cache, q, q_indptr, batch, num_decode, num_q_heads,
                    total_q_rows, max_q_len, block_table, block_table_stride, kv_lens,
                    max_kv_len, scale, split_tokens, nullptr, out, lse_out, workspace,
                    workspace_bytes, stream);
}

int pkv_paged_attn_mixed_ex(const pkv_cache_desc* desc, const void* k_cache,
                            const void* v_cache, const void* q, const int32_t* q_indptr,
                            int32_t batch, int32_t num_decode, int32_t num_q_heads,
                            int32_t total_q_rows, int32_t max_q_len,
                            const int32_t* block_table, int32_t block_table_stride,
                            const int32_t* kv_lens, int32_t max_kv_len, float scale,
                            int32_t split_tokens, const pkv_decode_opts* opts, void* out,
                            float* lse_out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return mixed_impl(desc, k_cache, v_cache, q, q_indptr, batch, num_decode, num_q_heads,
                    total_q_rows, max_q_len, block_table, block_table_stride, kv_lens,
                    max_kv_len, scale, split_tokens, opts, out, lse_out, workspace,
                    workspace_bytes, stream);
}

namespace {

// Shared-prefix (cascade) decode: the plan of its three launches.
struct CascadePlan {
  int group;
  pkv_decode_opts opts;
  Plan suffix;            // split-KV decode over each sequence's own pages
  int32_t n_prefix;       // key splits of the shared pages (0: no shared pages)
  int32_t split_tiles;    // 64-key tiles per split
  int32_t m_tiles;        // query-row tiles of the batch
  int32_t n_parts;        // n_prefix + suffix.n_split partials per row
  size_t o_bytes;         // partial outputs, rounded up to 256
  size_t ws_bytes;
};

constexpr int64_t kPrefixWorkgroups = 256;   // one per CU: one round of residency
constexpr int64_t kPrefixMinTiles = 4;       // 256 keys per split at least

int cascade_plan(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                 int32_t prefix_len, int32_t max_suffix_len, int32_t split_tokens,
                 const pkv_decode_opts* opts, CascadePlan* cp) {
  if (int rc = check_desc(desc)) return rc;
  if (int rc = resolve_opts(desc, opts, &cp->opts)) return rc;
  if (int rc = check_heads(desc, num_q_heads, &cp->group)) return rc;
  if (int rc = check_decode_group(desc, cp->opts.q_dtype, cp->group)) return rc;
  if (desc->dtype != PKV_F16 && desc->dtype != PKV_BF16 && !is_fp8(desc->dtype))
    return fail(PKV_ERR_UNSUPPORTED,
                "the shared pages run on the matrix cores: f16, bf16 or fp8 pools only");
  if (desc->head_dim != 128 && !(desc->head_dim == 64 && !is_fp8(desc->dtype)))
    return fail(PKV_ERR_UNSUPPORTED,
                "shared-prefix decode is built for head_dim 128, and 64 with 16-bit pools "
                "(got %d)", desc->head_dim);
  if (cp->opts.window != 0 || cp->opts.sink != 0)
    return fail(PKV_ERR_INVALID, "window and sink do not apply to the shared-prefix decode");
  if (batch < 0) return fail(PKV_ERR_INVALID, "batch %d < 0", batch);
  if (prefix_len < 0 || prefix_len % desc->page_size != 0)
    return fail(PKV_ERR_INVALID, "prefix_len %d: whole shared pages (a multiple of %d) expected",
                prefix_len, desc->page_size);
  if (max_suffix_len < 0) return fail(PKV_ERR_INVALID, "max_suffix_len %d < 0", max_suffix_len);
  if (int rc = make_plan(desc, batch, num_q_heads, max_suffix_len, split_tokens,
                         cp->opts.q_dtype, &cp->suffix))
    return rc;
  const int rows_per_tile = pkv::prefill_rows_per_tile(cp->group);
  cp->m_tiles = (batch + rows_per_tile - 1) / rows_per_tile;
  cp->n_prefix = 0;
  cp->split_tiles = 0;
  if (prefix_len > 0 && batch > 0) {
    const int64_t tiles = (prefix_len + 63) / 64;
    const int64_t units = (int64_t)desc->num_kv_heads * cp->m_tiles;
    int64_t want = (kPrefixWorkgroups + units - 1) / units;
    const int64_t cap = tiles / kPrefixMinTiles > 0 ? tiles / kPrefixMinTiles : 1;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    const int64_t st = (tiles + want - 1) / want;
    cp->split_tiles = (int32_t)st;
    cp->n_prefix = (int32_t)((tiles + st - 1) / st);
  }
  cp->n_parts = cp->n_prefix + cp->suffix.n_split;
  const size_t rows = (size_t)batch * num_q_heads;
  const size_t ob = rows * (size_t)cp->n_parts * desc->head_dim * sizeof(float);
  cp->o_bytes = (ob + 255) & ~(size_t)255;
  cp->ws_bytes = cp->o_bytes + rows * (size_t)cp->n_parts * sizeof(float);
  const int64_t blocks = (int64_t)desc->num_kv_heads * cp->m_tiles * cp->n_prefix;
  if (blocks > 0x7fffffff) return fail(PKV_ERR_INVALID, "grid too large");
  return PKV_OK;
}

}  // namespace

int pkv_decode_shared_prefix_plan(const pkv_cache_desc* desc, int32_t batch, int32_t num_q_heads,
                                  int32_t prefix_len, int32_t max_suffix_len,
                                  int32_t split_tokens, const pkv_decode_opts* opts,
                                  int32_t* n_parts, size_t* workspace_bytes) {
  CascadePlan cp;
  if (int rc = cascade_plan(desc, batch, num_q_heads, prefix_len, max_suffix_len, split_tokens,
                            opts, &cp))
    return rc;
  if (!n_parts || !workspace_bytes) return fail(PKV_ERR_INVALID, "NULL output pointer");
  *n_parts = cp.n_parts;
  *workspace_bytes = cp.ws_bytes;
  return ok();
}

int pkv_paged_attn_decode_shared_prefix(
    const pkv_cache_desc* desc, const void* k_cache, const void* v_cache, const void* q,
    int32_t batch, int32_t num_q_heads, const int32_t* prefix_table, int32_t prefix_len,
    const int32_t* block_table, int32_t block_table_stride, const int32_t* suffix_lens,
    int32_t max_suffix_len, float scale, int32_t split_tokens, const pkv_decode_opts* opts,
    void* out, float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  CascadePlan cp;
  if (int rc = cascade_plan(desc, batch, num_q_heads, prefix_len, max_suffix_len, split_tokens,
                            opts, &cp))
    return rc;
  // the own-pages part is a split-KV decode: its argument checks
  DecodeCommon dc;
  if (int rc = check_decode(desc, k_cache, v_cache, q, batch, num_q_heads, block_table,
                            block_table_stride, suffix_lens, max_suffix_len, scale,
                            split_tokens, opts, &dc))
    return rc;
  if (batch == 0) return ok();
  if (!out) return fail(PKV_ERR_INVALID, "out is NULL");
  if (prefix_len > 0 && !prefix_table) return fail(PKV_ERR_INVALID, "prefix_table is NULL");
  if (!aligned16(out)) return fail(PKV_ERR_INVALID, "out must be 16-byte aligned");
  if (!workspace || workspace_bytes < cp.ws_bytes)
    return fail(PKV_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, cp.ws_bytes);
  if (!aligned16(workspace)) return fail(PKV_ERR_INVALID, "workspace must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int32_t prefix_pages = prefix_len / desc->page_size;
  if (check_mode()) {
    if (int rc = debug_check_decode(desc, block_table, block_table_stride, suffix_lens, batch,
                                    max_suffix_len, 0, 0, s))
      return rc;
    std::vector<int32_t> pt;
    if (int rc = fetch_i32(prefix_table, prefix_pages, &pt, s)) return rc;
    if (int rc = check_pages(desc, pt, prefix_pages, 0, 0, prefix_pages, "prefix")) return rc;
  }
  float* o_part = (float*)workspace;
  float* lse_part = (float*)((char*)workspace + cp.o_bytes);
  const pkv_decode_opts& o = cp.opts;
  if (cp.n_prefix > 0) {
    // the shared pages: every sequence's query rows against them, split over keys
    pkv::PrefillArgs a{};
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.q = q;
    a.block_table = prefix_table;
    a.num_pages = desc->num_pages;
    a.stride = prefix_pages;
    a.num_kv_heads = desc->num_kv_heads;
    a.num_q_heads = num_q_heads;
    a.batch = 1;
    a.max_q_len = batch;
    a.total_q = batch;
    a.m_tiles = cp.m_tiles;
    a.xcd_split = 0;
    a.m_tiles_x = (cp.m_tiles + 7) / 8;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634 * (double)o.k_scale);
    a.v_scale = o.v_scale;
    a.kv_len0 = prefix_len;
    a.n_ksplit = cp.n_prefix;
    a.split_tiles = cp.split_tiles;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.part_stride = cp.n_parts;
    if (int rc = hip_status(pkv::launch_prefill(desc->dtype, o.q_dtype, desc->head_dim,
                                                cp.group, a, s),
                            "shared-prefix launch"))
      return rc;
  }
  // each sequence's own pages: split-KV partials after the shared ones
  pkv::DecodeArgs a = decode_args(desc, k_cache, v_cache, q, num_q_heads, block_table,
                                  block_table_stride, suffix_lens, scale, dc, batch);
  a.direct = 0;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.part_stride = cp.n_parts;
  a.part_offset = cp.n_prefix;
  if (int rc = hip_status(launch_any_decode(desc, o.q_dtype, dc.group, batch, a, s),
                          "decode launch"))
    return rc;
  return hip_status(pkv::launch_merge(o.q_dtype, desc->head_dim, o_part, lse_part,
                                      batch * num_q_heads, cp.n_parts, out, lse_out, s),
                    "merge launch");
}

int pkv_probe_read(const void* buf, size_t bytes, const int32_t* block_order,
                   int32_t block_bytes, int32_t grid, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(PKV_ERR_INVALID, "NULL pointer");
  if (!aligned16(buf)) return fail(PKV_ERR_INVALID, "buf must be 16-byte aligned");
  if (bytes == 0 || bytes % 16 != 0) return fail(PKV_ERR_INVALID, "bytes must be a positive multiple of 16");
  if (grid <= 0) return fail(PKV_ERR_INVALID, "grid %d <= 0", grid);
  if (block_order) {
    if (block_bytes <= 0 || block_bytes % 4096 != 0)
      return fail(PKV_ERR_INVALID, "block_bytes %d is not a positive multiple of 4096",
                  block_bytes);
    if (bytes % (size_t)block_bytes != 0 || bytes / 4096 > 0x7fffffff)
      return fail(PKV_ERR_INVALID, "bytes is not a whole number of blocks (or over 8 TiB)");
  }
  return hip_status(pkv::launch_read_probe(buf, bytes, block_order, block_bytes, 0x9e3779b9u,
                                           sink, grid, (hipStream_t)stream),
                    "read probe launch");
}

int pkv_probe_mfma(const void* operands, int32_t iters, int32_t vector_work, int32_t grid,
                   uint32_t* sink, int64_t* clocks, void* stream) {
  if (!operands || !sink || !clocks) return fail(PKV_ERR_INVALID, "NULL pointer");
  if (!aligned16(operands)) return fail(PKV_ERR_INVALID, "operands must be 16-byte aligned");
  if (iters <= 0 || grid <= 0) return fail(PKV_ERR_INVALID, "iters and grid must be > 0");
  if (vector_work != 0 && vector_work != 1)
    return fail(PKV_ERR_INVALID, "vector_work must be 0 or 1");
  return hip_status(pkv::launch_mfma_probe(operands, iters, vector_work, grid, 0x9e3779b9u,
                                           sink, clocks, (hipStream_t)stream),
                    "mfma probe launch");
}

int pkv_probe_prefill_loop(const void* operands, int32_t iters, int32_t vector_work,
                           int32_t grid, uint32_t* sink, int64_t* clocks, void* stream) {
  if (!operands || !sink || !clocks) return fail(PKV_ERR_INVALID, "NULL pointer");
  if (!aligned16(operands)) return fail(PKV_ERR_INVALID, "operands must be 16-byte aligned");
  if (iters <= 0 || grid <= 0) return fail(PKV_ERR_INVALID, "iters and grid must be > 0");
  if (vector_work != 0 && vector_work != 1)
    return fail(PKV_ERR_INVALID, "vector_work must be 0 or 1");
  return hip_status(pkv::launch_prefill_loop_probe(operands, iters, vector_work, grid,
                                                   0x9e3779b9u, sink, clocks,
                                                   (hipStream_t)stream),
                    "prefill loop probe launch");
}

int pkv_validate_tables(const pkv_cache_desc* desc, const int32_t* block_table_host,
                        int32_t stride, const int32_t* lens_host, int32_t batch,
                        const int32_t* slots_host, int32_t n_slots) {
  if (int rc = check_desc(desc)) return rc;
  if (batch < 0 || n_slots < 0) return fail(PKV_ERR_INVALID, "negative batch or n_slots");
  if (batch > 0 && (!block_table_host || !lens_host || stride <= 0))
    return fail(PKV_ERR_INVALID, "NULL table or stride <= 0");
  const int P = desc->page_size;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = lens_host[b];
    if (L < 0 || L > (int64_t)stride * P)
      return fail(PKV_ERR_INVALID, "lens[%d] = %lld outside [0, %lld]", b, (long long)L,
                  (long long)stride * P);
    const int64_t np = (L + P - 1) / P;
    for (int64_t i = 0; i < np; ++i) {
      const int32_t pg = block_table_host[(int64_t)b * stride + i];
      if (pg < 0 || pg >= desc->num_pages)
        return fail(PKV_ERR_INVALID, "block_table[%d][%lld] = %d outside [0, %d)", b,
                    (long long)i, pg, desc->num_pages);
    }
  }
  if (n_slots > 0) {
    if (!slots_host) return fail(PKV_ERR_INVALID, "slots is NULL");
    const int64_t total = (int64_t)desc->num_pages * P;
    std::unordered_set<int32_t> seen;
    seen.reserve((size_t)n_slots * 2);
    for (int32_t i = 0; i < n_slots; ++i) {
      const int32_t s = slots_host[i];
      if (s < 0) continue;
      if (s >= total)
        return fail(PKV_ERR_INVALID, "slot[%d] = %d >= num_pages * page_size = %lld", i, s,
                    (long long)total);
      if (!seen.insert(s).second) return fail(PKV_ERR_INVALID, "slot %d repeats (index %d)", s, i);
    }
  }
  return ok();
}

}  // extern "C"
