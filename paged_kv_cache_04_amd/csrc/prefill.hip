// Chunked prefill over a paged KV cache on the matrix cores (MFMA).
//
// What is computed: for each sequence b with C_b new query rows at the end of
// kv_len_b tokens (history plus the chunk, whose K/V were appended first),
// chunk row i sits at position kv_len_b - C_b + i and attends to keys
// 0 .. that position (page 4, section 3.1, chunked prefill; bottom-right
// causal alignment).  out = softmax(q K^T * scale) V per query head (page 2,
// section 2.1), accumulated tile by tile with an online softmax (page 2,
// section 2.2).  Keys are reached through the block table (page 3, section
// 3.2).
//
// Work decomposition.  A workgroup (4 wavefronts) owns 128 query rows of one
// (sequence, KV head): 128 / G chunk positions times the G query heads that
// share the KV head (page 4, section 2.2, GQA), so the G heads reuse every
// K/V tile.  Wave w owns rows 32w .. 32w+31.  Keys go in tiles of 64 (four
// pages), double-buffered in LDS: while the waves compute on one buffer, the
// next tile's pages are loaded into registers and then written to the other.
//
// Per tile and wave, on 32x32x16 MFMAs with fp32 accumulation:
//   S^T (64 keys x 32 rows) = K (from LDS) x Q^T (registers); the scores of a
//       query row sit in one lane (16 per 32-key block, the other half of the
//       block in lane + 32), so the row max is an in-lane max and one
//       exchange.
//   online softmax in base 2 (log2 e folded into the scale), rescaling the
//       accumulators only when some row's running max grew (wave vote).
//   O^T (128 x 32) += V^T (from LDS) x P^T: the probabilities are converted in
//       place to bf16/f16; the 32x32 output layout of S^T is already the
//       operand layout P^T needs, given that the V^T operand takes its keys
//       in the same order.  V is written to LDS transposed (key pairs packed
//       with v_perm), K as rows; rows are padded against bank conflicts.
// Keys past the causal limit or the sequence end are selected out of S; K and
// V slots past the sequence end are zero-filled in LDS, so stale or NaN slots
// in a partly filled last page never leak into the products.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int P = kPageSize;
constexpr int D = 128;          // head_dim of the MFMA kernel
constexpr int BK = 64;          // keys per tile (4 pages)
constexpr int NWP = 4;          // waves per workgroup
constexpr int ROWS = 128;       // query rows per workgroup
constexpr int KLD = D + 8;      // K tile row stride in elements (272 bytes)
constexpr int VLD = BK + 4;     // V^T tile row stride in elements (136 bytes)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename TT>
struct Mfma;

template <>
struct Mfma<TBF16> {
  static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                   0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return (uint32_t)TBF16::from_float(lo) | ((uint32_t)TBF16::from_float(hi) << 16);
  }
  static constexpr float POFF = 0.f;
};

template <>
struct Mfma<TF16> {
  static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return (uint32_t)TF16::from_float(lo) | ((uint32_t)TF16::from_float(hi) << 16);
  }
  // f16 probabilities are carried as p * 2^15 so small weights keep precision
  static constexpr float POFF = 15.f;
};

// Registers holding one tile's K and V loads before they go to LDS.
struct TileRegs {
  u32x4 k[4];   // K: thread t holds token t/16 of each of the 4 pages, vector t%16
  u32x4 v[4];   // V: two (key pair, 8-element column) tasks, two rows each
};

template <typename TT, int G>
__global__ __launch_bounds__(NWP * 64, 2) void prefill_kernel(PrefillArgs a) {
  using M = Mfma<TT>;
  constexpr int NPOS = ROWS / G;  // chunk positions per workgroup
  __shared__ __align__(16) uint16_t k_lds[2][BK * KLD];
  __shared__ __align__(16) uint16_t v_lds[2][D * VLD];
  __shared__ int bad_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int half = lane >> 5;     // which 32-lane half
  const int n = lane & 31;        // this lane's query row within the wave

  const int nbg = a.batch * a.num_kv_heads;
  const int bg = blockIdx.x % nbg;
  const int mt = blockIdx.x / nbg;
  const int b = bg / a.num_kv_heads;
  const int g = bg % a.num_kv_heads;

  // sequence geometry, with broken preconditions clamped and flagged
  const int q0 = a.q_indptr[b];
  int C = a.q_indptr[b + 1] - q0;
  int kvl = a.kv_lens[b];
  bool bad = false;
  if (C < 0 || C > a.max_q_len || kvl < C || kvl > a.stride * P || q0 < 0) {
    bad = true;
    C = max(0, min(C, a.max_q_len));
    kvl = max(C, min(kvl, a.stride * P));
  }
  const int pos0 = mt * NPOS;
  if (pos0 >= C) return;  // this tile of positions is past the chunk
  const int npos = min(NPOS, C - pos0);
  const int hist = kvl - C;
  const int n_keys = hist + pos0 + npos;            // keys seen by the last row here
  const int n_tiles = (n_keys + BK - 1) / BK;
  const int seq_pages = (kvl + P - 1) / P;
  const int32_t* bt_row = a.block_table + (int64_t)b * a.stride;

  // this lane's query row
  const int row = 32 * w + n;
  const int pos = pos0 + row / G;
  const int head = g * G + row % G;
  const int64_t qrow = (int64_t)q0 + pos;
  const bool row_ok = (row / G) < npos && qrow >= 0 && qrow < a.total_q;
  const int apos = hist + pos;                       // last key this row sees

  // Q^T operand: 8 k-steps of 16 head dims; lane holds 8 consecutive dims
  u32x4_t qreg[8];
  {
    const bool neg = a.scale_log2 < 0.f;  // fold the sign of the scale into q
    const char* qp = (const char*)a.q + ((qrow * a.num_q_heads + head) * D) * 2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 x;
      if (row_ok) x = load16(qp + (16 * ks + 8 * half) * 2);
      else x.w[0] = x.w[1] = x.w[2] = x.w[3] = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) qreg[ks][e] = neg ? (x.w[e] ^ 0x80008000u) : x.w[e];
    }
  }
  const float c = fabsf(a.scale_log2);

  if (tid == 0) bad_flag = bad ? 1 : 0;

  // ---- staging: global pages -> registers -> LDS
  const int64_t head_block = (int64_t)P * D * 2;
  bool my_bad = false;
  auto page_of = [&](int pi) -> int64_t {  // physical page of logical page pi (or -1)
    if (pi >= seq_pages) return -1;
    int pid = bt_row[pi];
    if (pid < 0 || pid >= a.num_pages) {
      my_bad = true;
      return -1;
    }
    return pid;
  };
  auto load_tile = [&](TileRegs& r, int it) {
    const int pg0 = it * (BK / P);
    int64_t pids[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pids[j] = page_of(pg0 + j);   // uniform: scalar loads
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // K: page j, token tid/16, vector tid%16
      const int tok = tid >> 4, vec = tid & 15;
      const int key = it * BK + j * P + tok;
      if (pids[j] >= 0 && key < kvl) {
        r.k[j] = load16((const char*)a.k_cache + (pids[j] * a.num_kv_heads + g) * head_block +
                        (tok * D + vec * 8) * 2);
      } else {
        r.k[j].w[0] = r.k[j].w[1] = r.k[j].w[2] = r.k[j].w[3] = 0u;
      }
    }
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {  // V: keys 2kp, 2kp+1; 8 columns from 8*dv
      const int task = tid + 256 * j2;
      const int kp = task & 31, dv = task >> 5;
      const int key = 2 * kp;                      // within the tile
      const int pj = key / P;
      const int64_t pid = pj == 0 ? pids[0] : pj == 1 ? pids[1] : pj == 2 ? pids[2] : pids[3];
      const int tok = key % P;
      const char* src = (const char*)a.v_cache +
                        (pid < 0 ? 0 : (pid * a.num_kv_heads + g)) * head_block +
                        (tok * D + dv * 8) * 2;
      const int kabs = it * BK + key;
      u32x4 z;
      z.w[0] = z.w[1] = z.w[2] = z.w[3] = 0u;
      r.v[2 * j2] = (pid >= 0 && kabs < kvl) ? load16(src) : z;
      r.v[2 * j2 + 1] = (pid >= 0 && kabs + 1 < kvl) ? load16(src + D * 2) : z;
    }
  };
  auto store_tile = [&](const TileRegs& r, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = j * P + (tid >> 4);
      store16(&k_lds[buf][key * KLD + (tid & 15) * 8], r.k[j]);
    }
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const int task = tid + 256 * j2;
      const int kp = task & 31, dv = task >> 5;
      uint32_t* vt = reinterpret_cast<uint32_t*>(&v_lds[buf][0]);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t x0 = r.v[2 * j2].w[e2], x1 = r.v[2 * j2 + 1].w[e2];
        // column d = 8dv + 2e2 (low halves) and d + 1 (high halves): (key 2kp, key 2kp+1)
        const uint32_t lo = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
        const int d = 8 * dv + 2 * e2;
        vt[(d * VLD) / 2 + kp] = lo;
        vt[((d + 1) * VLD) / 2 + kp] = hi;
      }
    }
  };

  // ---- accumulators
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = -INFINITY;  // running max of the raw (unscaled) scores of this row
  float l_run = 0.f;        // running sum of exp2(c * s - c * m_run) over this lane's keys

  TileRegs tr;
  load_tile(tr, 0);
  store_tile(tr, 0);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < n_tiles;
    if (more) load_tile(tr, it + 1);

    // S^T = K Q^T for two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    const uint16_t* kt = k_lds[buf];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4_t av =
            *reinterpret_cast<const u32x4_t*>(kt + (32 * kb + n) * KLD + 16 * ks + 8 * half);
        s[kb] = M::run(av, qreg[ks], s[kb]);
      }
    }

    // keys past this row's position (or the sequence end) are selected out
    const int t0 = it * BK;
    const bool masked = t0 + BK - 1 > hist + pos0;
    auto visible = [&](int kb, int i) {
      const int t = t0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
      return t <= apos && t < kvl;
    };
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = visible(kb, i) ? s[kb][i] : -INFINITY;
    }

    // running max (raw units; c >= 0)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run) != 0) {
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m_run = m_new;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * c - M::POFF;

    // probabilities -> packed B operands of the PV MFMA (k-step ks = keys 16ks..16ks+15)
    u32x4_t pk[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = exp2_fast(fmaf(s[kb][8 * sub + e], c, -mc));
          p[e] = (masked && !visible(kb, 8 * sub + e)) ? 0.f : pe;
          l_run += p[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[2 * kb + sub][e] = M::pack(p[2 * e], p[2 * e + 1]);
      }

    // O^T += V^T P^T
    const uint16_t* vt = v_lds[buf];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int koff = 16 * ks + 4 * half;  // keys koff..koff+3 and koff+8..koff+11
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* rowp = vt + (32 * db + n) * VLD + koff;
        const uint2 lo = *reinterpret_cast<const uint2*>(rowp);
        const uint2 hi = *reinterpret_cast<const uint2*>(rowp + 8);
        u32x4_t av;
        av[0] = lo.x;
        av[1] = lo.y;
        av[2] = hi.x;
        av[3] = hi.y;
        o[db] = M::run(av, pk[ks], o[db]);
      }
    }

    if (more) store_tile(tr, buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  if (my_bad) bad_flag = 1;
  __syncthreads();
  const float l_tot = l_run + xor_f(l_run, 32);
  if (!row_ok) return;
  const bool poison = bad_flag != 0;
  const float inv = 1.f / l_tot;
  char* op = (char*)a.out + ((qrow * a.num_q_heads + head) * D) * 2;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * db + 8 * j + 4 * half;
      float v0 = o[db][4 * j + 0] * inv, v1 = o[db][4 * j + 1] * inv;
      float v2 = o[db][4 * j + 2] * inv, v3 = o[db][4 * j + 3] * inv;
      if (poison) v0 = v1 = v2 = v3 = __builtin_nanf("");
      uint2 st;
      st.x = M::pack(v0, v1);
      st.y = M::pack(v2, v3);
      *reinterpret_cast<uint2*>(op + d * 2) = st;
    }
  if (a.lse_out && half == 0) {
    float lse = (m_run * c + log2_fast(l_tot) - M::POFF) * kLn2;
    if (m_run == -INFINITY) lse = -INFINITY;
    a.lse_out[qrow * a.num_q_heads + head] = poison ? __builtin_nanf("") : lse;
  }
}

template <typename TT>
hipError_t launch_t(int group, const PrefillArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.batch * a.num_kv_heads * a.m_tiles;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(NWP * 64);
  switch (group) {
    case 1: hipLaunchKernelGGL((prefill_kernel<TT, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<TT, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<TT, 4>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<TT, 8>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int prefill_rows_per_tile(int group) { return ROWS / group; }

hipError_t launch_prefill(int dtype, int head_dim, int group, const PrefillArgs& a,
                          hipStream_t stream) {
  if (head_dim != D) return hipErrorInvalidValue;
  switch (dtype) {
    case 1: return launch_t<TF16>(group, a, stream);
    case 2: return launch_t<TBF16>(group, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
