// The newest token's K/V, written by the decode launch that attends it.
//
// A decode step first stores each sequence's new token at the end of its
// context (page 2, section 5.2: the page that receives it is allocated ahead,
// and the K/V vectors are stored in place), then attends keys 0 .. L-1. The
// position is L - 1, so its page is the last one the sequence visits, and
// exactly one decode workgroup per (sequence, KV head) reads that page: the
// one whose split ends there. That workgroup writes the row itself before it
// starts loading; a separate append launch is not needed.
#pragma once

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// Row b, KV head g of a.k_new / a.v_new into slot (page of position L - 1,
// L - 1 mod P): a bitwise copy when the cache holds q's type, else each
// element divided by the pool scale in IEEE fp32 and rounded to the fp8 code
// (as the quantizing append does).  A page id outside the pool writes nothing
// (the decode itself flags the row).  Every thread of the workgroup calls it;
// the caller waits for the stores and synchronises the workgroup before any
// load of the page.
template <typename QT, typename CT, int D>
__device__ __forceinline__ void append_newest(const DecodeArgs& a, int b, int g, int L, int tid,
                                              int nthreads) {
  const int t = L - 1;
  const int32_t pid = a.block_table[(int64_t)b * a.stride + t / kPageSize];
  if (pid < 0 || pid >= a.num_pages) return;
  constexpr int RB = D * CT::bytes;   // bytes per cache row
  constexpr int NV = RB / 16;         // 16-byte vectors per cache row
  const int64_t dst = (((int64_t)pid * a.num_kv_heads + g) * kPageSize + t % kPageSize) * RB;
  const int64_t src = ((int64_t)b * a.num_kv_heads + g) * D * QT::bytes;
  for (int i = tid; i < 2 * NV; i += nthreads) {
    const int which = i >= NV;        // 0: K, 1: V
    const int vec = i - which * NV;
    char* cache = (char*)(which ? a.v_cache : a.k_cache);
    const char* row = (const char*)(which ? a.v_new : a.k_new) + src;
    if constexpr (!CT::is_fp8) {
      store16(cache + dst + 16 * vec, load16(row + 16 * vec));
    } else {
      constexpr int SB = QT::bytes;   // source bytes per element: 16 elements = SB vectors
      u32x4 in[4];
#pragma unroll
      for (int j = 0; j < SB; ++j) in[j] = load16(row + 16 * (SB * vec + j));
      const float scale = which ? a.v_quant : a.k_quant;
      u32x4 out;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = __fdiv_rn(src_elem<QT>(in, 4 * q + e), scale);
        out.w[q] = fp8_pack4<CT::is_e4m3>(y);
      }
      store16(cache + dst + 16 * vec, out);
    }
  }
}

}  // namespace pkv
