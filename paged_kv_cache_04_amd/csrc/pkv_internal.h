// Internal interface between the C-ABI host layer (pkv_host.cpp) and the
// kernel launchers (*.hip).  Not installed; the public ABI is include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kPageSize = 16;          // tokens per page (the only size built)
constexpr int kDecodeWaves = 4;        // waves per decode workgroup

struct DecodeArgs {
  const void* k_cache;
  const void* v_cache;
  const void* q;                // [B][H_q][D]
  const int32_t* block_table;   // [B][stride]
  const int32_t* context_lens;  // [B]
  int64_t num_pages;
  int32_t stride;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t pages_per_split;
  int32_t n_split;
  float scale_log2;             // scale * log2(e) (times k_scale for fp8 caches)
  float v_scale;                // multiplies the output (fp8 caches; 1 otherwise)
  int32_t window;               // > 0: keys t >= L - window and t < sink only
  int32_t sink;
  int32_t direct;               // 1: final output to out/lse_out; 0: partials
  void* out;                    // [B][H_q][D] (direct)
  float* lse_out;               // [B][H_q] or null (direct)
  float* o_part;                // [B*H_q][part_stride][D] (partials), split ks at part
  float* lse_part;              // [B*H_q][part_stride]    part_offset + ks
  int32_t part_stride;          // parts per row (n_split unless other parts share the rows)
  int32_t part_offset;
  // Newest-token append (null: none): row b of k_new / v_new [B][H_kv][D]
  // (q's type) goes to position context_lens[b] - 1 before it is attended;
  // fp8 caches quantize it by the pool scales k_quant / v_quant.
  const void* k_new;
  const void* v_new;
  float k_quant;
  float v_quant;
  int32_t n_units;              // batch * H_kv
};

// Grid of a decode launch.  Work units are (sequence b, KV head g), unit =
// b * H_kv + g, each cut into n_split splits.  The grid is split-major: all
// first splits, then all second splits, and so on, each round covering the
// units padded to a multiple of 8 and rotated by its split index.
// Workgroups reach the 8 XCDs round-robin (workgroup i to XCD i % 8), so a
// unit's splits land on different XCDs and every XCD gets a share of each
// round; the hardware hands out the longest work (the first splits, full
// length unless the sequence is short) before the sequences' remainders.
// (A unit-major grid put the only split of every short sequence on the same
// few XCDs whenever n_split was even.)
inline int64_t decode_grid(const DecodeArgs& a) {
  return ((int64_t)a.n_units + 7) / 8 * 8 * a.n_split;
}

// The (split ks, unit) of decode workgroup `bid`; false for a padding
// workgroup, which has no work.
__device__ __forceinline__ bool decode_item(int bid, const DecodeArgs& a, int* ks, int* unit) {
  const int up = (a.n_units + 7) / 8 * 8;
  const int k = bid / up, r = bid % up;
  *ks = k;
  *unit = (r - k % up + up) % up;
  return *unit < a.n_units;
}

struct PrefillArgs {
  const void* k_cache;
  const void* v_cache;
  const void* q;                // packed [sum C][H_q][D]
  const int32_t* q_indptr;      // [B+1]
  const int32_t* block_table;
  const int32_t* kv_lens;
  int64_t num_pages;
  int32_t stride;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t batch;
  int32_t max_q_len;
  int64_t total_q;              // rows of q / out
  int32_t m_tiles;              // query-row tiles per (b, kv head)
  int32_t xcd_split;            // 1: tile ranges spread over the 8 XCDs (see prefill.hip)
  int32_t m_tiles_x;            // ceil(m_tiles / 8): tiles per XCD and (b, kv head)
  float scale_log2;             // softmax scale * log2(e) (* k_scale for fp8 pools)
  float v_scale;                // fp8 pools: V element = v_scale * code; 1 otherwise
  void* out;
  float* lse_out;
  // Shared-prefix form, chosen by o_part != null (all zero / null for a
  // chunked prefill): one sequence (batch 1; q_indptr and kv_lens unused) of
  // total_q query rows over kv_len0 keys, every row seeing every key, the
  // keys cut into n_ksplit splits of split_tiles 64-key tiles; fp32 partials
  // [row][part_stride][D] (row = query row * H_q + head) in o_part and
  // lse_part [row][part_stride], at part ks of each row, instead of out.
  int32_t kv_len0;
  int32_t n_ksplit;
  int32_t split_tiles;
  float* o_part;
  float* lse_part;
  int32_t part_stride;
};

// Each launcher validates nothing: the host layer has done it.
hipError_t launch_kv_append(int dtype, int head_dim, int num_kv_heads, int64_t num_pages,
                            void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* slots, int32_t n_tokens, hipStream_t stream);

hipError_t launch_gather(int dtype, int head_dim, int num_kv_heads, int64_t num_pages,
                         const void* k_cache, const void* v_cache, const int32_t* table_row,
                         int32_t len, void* k_out, void* v_out, hipStream_t stream);

// kv_dtype: element type of the pools; q_dtype: of q and out (equal unless
// the pools are fp8).
hipError_t launch_decode(int kv_dtype, int q_dtype, int head_dim, int group, int batch,
                         const DecodeArgs& a, hipStream_t stream);

// Decode on the matrix cores (16-bit queries, head_dim 128, G = 4, 8 or 16
// with any 16-bit or fp8 pool); same arguments and results as launch_decode,
// which builds G <= 8 only.
bool decode_mfma_supported(int kv_dtype, int q_dtype, int head_dim, int group);
hipError_t launch_decode_mfma(int kv_dtype, int q_dtype, int group, int batch,
                              const DecodeArgs& a, hipStream_t stream);

// fp8 quantizing append from src_dtype (f32, f16, bf16) new tokens.
hipError_t launch_kv_append_quant(int fp8_dtype, int src_dtype, int head_dim, int num_kv_heads,
                                  int64_t num_pages, void* k_cache, void* v_cache,
                                  const void* k_new, const void* v_new, float k_scale,
                                  float v_scale, const int32_t* slots, int32_t n_tokens,
                                  hipStream_t stream);

hipError_t launch_merge(int out_dtype, int head_dim, const float* o_parts,
                        const float* lse_parts, int32_t rows, int32_t n_parts, void* out,
                        float* lse_out, hipStream_t stream);

// kv_dtype: element type of the pools (f16, bf16, or fp8 with q_dtype f16 /
// bf16); q_dtype: of q and out.
hipError_t launch_prefill(int kv_dtype, int q_dtype, int head_dim, int group,
                          const PrefillArgs& a, hipStream_t stream);

// Measurement probes (probe.hip).
hipError_t launch_read_probe(const void* buf, size_t bytes, const int32_t* order,
                             int32_t block_bytes, uint32_t never, uint32_t* sink, int grid,
                             hipStream_t stream);
hipError_t launch_mfma_probe(const void* ops, int32_t iters, int32_t vec, int grid,
                             uint32_t never, uint32_t* sink, int64_t* clocks,
                             hipStream_t stream);
hipError_t launch_prefill_loop_probe(const void* ops, int32_t iters, int32_t vec, int grid,
                                     uint32_t never, uint32_t* sink, int64_t* clocks,
                                     hipStream_t stream);

// Rows of query positions one prefill workgroup covers (per KV head group).
int prefill_rows_per_tile(int group);

}  // namespace pkv
