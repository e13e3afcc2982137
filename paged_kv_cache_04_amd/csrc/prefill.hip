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
// pages) through two LDS buffers: while the waves compute on one, direct
// global-to-LDS loads (no registers) fill the other with the next tile.
//
// LDS layout: K and V tiles are stored as they sit in the pages, one 256-byte
// row per key, with the sixteen 16-byte chunks of row r permuted by
// chunk ^ swz(r) so that the operand reads below hit distinct banks.
//
// Per tile and wave, on 32x32x16 MFMAs with fp32 accumulation:
//   S^T (64 keys x 32 rows) = K x Q^T: K rows are read as 16-byte chunks, Q^T
//       stays in registers.  The scores of a query row sit in one lane (16 per
//       32-key block, the other 16 in lane + 32): the row max is an in-lane
//       max and one exchange.
//   online softmax in base 2 (log2 e folded into the scale); the reference
//       max of a row moves only when a score exceeds it by more than 8 (in
//       log2 units), so the accumulators are rescaled rarely (wave vote).
//   O^T (128 x 32) += V^T x P^T: the probabilities are converted in place to
//       bf16/f16 (the S^T output layout is the P^T operand layout), and the
//       V^T operand comes from transposing LDS reads (ds_read_b64_tr_b16) of
//       the row-major V tile, with keys taken in the order P^T holds them.
// Keys past the causal limit or the sequence end are selected out of S; V
// rows past the sequence end are zeroed in LDS before use, so stale or NaN
// slots in a partly filled last page never reach the products.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int P = kPageSize;
constexpr int D = 128;           // head_dim of the MFMA kernel
constexpr int BK = 64;           // keys per tile (4 pages)
constexpr int NWP = 4;           // waves per workgroup
constexpr int ROWS = 128;        // query rows per workgroup
constexpr int ROWB = D * 2;      // bytes per key row (256)
constexpr int TILEB = BK * ROWB; // bytes per K or V tile (16 KiB)
constexpr float kLazyLog2 = 8.f; // rescale when a row max grows by > 2^8

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint8_t __attribute__((address_space(3))) lds_u8;

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

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
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));  // RNE
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
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));  // RNE
  }
  // f16 probabilities are carried as p * 2^7 (p <= 2^8, so <= 2^15 < 65504)
  // so that small weights keep their precision
  static constexpr float POFF = 7.f;
};

// Chunk permutation of key row r (physical chunk = logical chunk ^ swz(r)),
// for 64 LDS banks (256 bytes per cycle).  It is a bijection on r % 16, so
// the K operand reads of 16 consecutive rows at one logical chunk hit all 16
// chunk positions; and it puts r % 4 into chunk bits 2-3 and r / 4 % 4 into
// bits 0-1, so the transposing V reads of 32 lanes (4 keys x two adjacent
// 32-byte chunk pairs) cover 8 distinct chunk pairs.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Direct global-to-LDS copy through a buffer descriptor: lane i's 16 bytes
// at byte offset voff of the buffer go to lds_base + 16 * i.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, lds_u8* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)lds_base,
                                           16, voff, 0, 0, 0);
}
// Descriptor of one 4-KiB (page, head) block: base address, no stride, range
// 4096 bytes, 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const char* base) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, P * D * 2, 0x00020000);
}

// Transposing LDS read: in each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte chunks addressed by lanes 4k + i / 4, k = 0..3.
__device__ __forceinline__ uint2 read_tr(const lds_u8* p) {
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4_t __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(uint2, r);
}

template <typename TT, int G>
__global__ __launch_bounds__(NWP * 64, 2) void prefill_kernel(PrefillArgs a) {
  using M = Mfma<TT>;
  constexpr int NPOS = ROWS / G;  // chunk positions per workgroup
  __shared__ __align__(1024) uint8_t k_lds0[TILEB];
  __shared__ __align__(1024) uint8_t k_lds1[TILEB];
  __shared__ __align__(1024) uint8_t v_lds0[TILEB];
  __shared__ __align__(1024) uint8_t v_lds1[TILEB];
  __shared__ int bad_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int half = lane >> 5;     // which 32-lane half
  const int n = lane & 31;        // this lane's query row within the wave

  // Workgroups are handed to the 8 XCDs round-robin (workgroup i to XCD
  // i % 8), and each XCD has its own L2.  Default order: (b, kv head) fastest,
  // so when there are at least 8 such pairs each XCD keeps whole pairs and all
  // their query tiles share the K/V stream in its L2.  With xcd_split, XCD x
  // takes the x-th eighth of the query tiles of every pair instead: every XCD
  // gets the same share of long and short sequences, and the tiles of one
  // pair on one XCD still read the same keys together.
  const int nbg = a.batch * a.num_kv_heads;
  int bg, mt;
  if (a.xcd_split) {
    const int x = blockIdx.x % 8, j = blockIdx.x / 8;
    bg = j % nbg;
    mt = x * a.m_tiles_x + j / nbg;
    if (mt >= a.m_tiles) return;     // padding of the last XCD's range
  } else {
    bg = blockIdx.x % nbg;
    mt = blockIdx.x / nbg;
  }
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
  // scale in log2 units; kept >= 1e-30 so that a masked score (-inf) times it
  // stays -inf (a zero scale would give NaN; 1e-30 changes no result)
  const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);

  if (tid == 0) bad_flag = bad ? 1 : 0;

  // ---- staging: wave w copies page w of the tile (key rows 16w .. 16w+15)
  // of K and V as four 1-KiB LDS chunks of four rows; lane i of a chunk fills
  // row 4j + i/16, physical chunk i%16 with logical chunk (i%16) ^ swz(row).
  // The page, its descriptor and the LDS destination are the same for the
  // whole wave (scalar registers); each lane adds a fixed offset.  The page id
  // of the next tile is loaded one tile ahead.
  const int64_t head_block = (int64_t)P * D * 2;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t dma_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * j + (lane >> 4);               // key row within the page
    dma_off[j] = (uint32_t)(r * ROWB + (((lane & 15) ^ swz(r)) * 16));
  }
  bool my_bad = false;
  int pid_next = 0;
  auto fetch_pid = [&](int it) {
    const int pi = it * (BK / P) + wu;
    pid_next = (it < n_tiles && pi < seq_pages) ? bt_row[pi] : 0;
  };
  auto issue_tile = [&](int it, lds_u8* kdst, lds_u8* vdst) {
    const int pi = it * (BK / P) + wu;
    int pid = __builtin_amdgcn_readfirstlane(pid_next);
    fetch_pid(it + 1);
    if (pi < seq_pages && (pid < 0 || pid >= a.num_pages)) my_bad = true;
    if (pid < 0 || pid >= a.num_pages) pid = 0;   // always a readable page
    const int64_t base = ((int64_t)pid * a.num_kv_heads + g) * head_block;
    const __amdgpu_buffer_rsrc_t kr = page_rsrc((const char*)a.k_cache + base);
    const __amdgpu_buffer_rsrc_t vr = page_rsrc((const char*)a.v_cache + base);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dma16(kr, dma_off[j], kdst + (16 * wu + 4 * j) * ROWB);
      dma16(vr, dma_off[j], vdst + (16 * wu + 4 * j) * ROWB);
    }
  };
  // V rows of keys past the sequence end become zero (edge tiles only)
  auto zero_tail = [&](int it, uint8_t* vdst) {
    const int first = kvl - it * BK;   // first row to clear
    for (int idx = tid; idx < BK * (ROWB / 16); idx += NWP * 64) {
      const int r = idx / (ROWB / 16);
      if (r >= first)
        *reinterpret_cast<uint4*>(vdst + r * ROWB + (idx % (ROWB / 16)) * 16) =
            make_uint4(0u, 0u, 0u, 0u);
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

  // Online-softmax update for one tile: running max, rescale, probabilities
  // packed as the B operands of the PV MFMA (k-step ks = keys 16ks..16ks+15).
  auto softmax_tile = [&](f32x16_t (&s)[2], u32x4_t (&pk)[4]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    const bool grow = (m_run == -INFINITY) ? (mx > -INFINITY) : ((mx - m_run) * c > kLazyLog2);
    if (__ballot(grow) != 0) {
      __asm__ volatile("");   // keep this a branch: the rescale is rare
      mx = fmaxf(mx, xor_f(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m_run = m_new;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * c - M::POFF;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = exp2_fast(fmaf(s[kb][8 * sub + e], c, -mc));   // masked: exp2(-inf) = 0
          l_run += p[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[2 * kb + sub][e] = M::pack(p[2 * e], p[2 * e + 1]);
      }
  };

  // Per-lane LDS byte offsets, the same for every tile: the K operand of
  // k-step ks (row n, logical chunk 2ks + half) and the V^T operand reads of
  // head-dim block db for key slots 0..3 (a) and 4..7 (b) at k-step 0.
  int k_off[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) k_off[ks] = n * ROWB + (((2 * ks + half) ^ swz(n)) * 16);
  const int q16 = lane >> 4, li = lane & 15;
  const int kk = li >> 2, jj = li & 3;
  const int key_a0 = 4 * (q16 >> 1) + kk;      // key of slots 0..3 at k-step 0
  int va_off[4], vb_off[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int dcol = 32 * db + 16 * (q16 & 1) + 4 * jj;   // first of 4 head dims
    const int lc = dcol >> 3, sub8 = (dcol & 7) * 2;      // chunk, byte in chunk
    va_off[db] = key_a0 * ROWB + ((lc ^ swz(key_a0)) * 16) + sub8;
    vb_off[db] = (key_a0 + 8) * ROWB + ((lc ^ swz(key_a0 + 8)) * 16) + sub8;
  }

  // One tile from LDS buffers (kt, vt); MASKED tiles are the few that reach
  // past some row's causal limit or the sequence end.
  auto compute_tile = [&](int it, const lds_u8* kt, const lds_u8* vt, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    // S^T = K Q^T for two 32-key blocks
    f32x16_t s[2];
    const f32x16_t zero16 = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4_t av = *reinterpret_cast<const u32x4_t __attribute__((address_space(3)))*>(
            kt + kb * 32 * ROWB + k_off[ks]);
        s[kb] = M::run(av, qreg[ks], ks == 0 ? zero16 : s[kb]);
      }
    }
    // keys past this row's position (or the sequence end) are selected out:
    // score i of block kb is key t0 + 32kb + 8(i/4) + 4half + i%4
    const int t0 = it * BK;
    if constexpr (MASKED) {
      const int thr = min(apos, kvl - 1) - t0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3) <= thr) ? s[kb][i] : -INFINITY;
    }
    u32x4_t pk[4];
    softmax_tile(s, pk);

    // O^T += V^T P^T.  The 16-lane group q16 = lane / 16 covers head dims
    // 32db + 16 (q16 & 1) .. +15 with key half h = q16 >> 1; source lane
    // 4k + j of the group points at key (16ks + 4h + k) (+8 for slots 4..7),
    // dims +4j .. +4j+3, so result lane i holds dim +i for keys k = 0..3.
    // The swizzle of key 16ks + x equals that of key x, so k-step ks only
    // adds 16 rows to the k-step 0 offsets.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint2 lo = read_tr(vt + ks * 16 * ROWB + va_off[db]);
        const uint2 hi = read_tr(vt + ks * 16 * ROWB + vb_off[db]);
        u32x4_t av;
        av[0] = lo.x;
        av[1] = lo.y;
        av[2] = hi.x;
        av[3] = hi.y;
        o[db] = M::run(av, pk[ks], o[db]);
      }
    }
  };

  lds_u8* kb0 = (lds_u8*)k_lds0;
  lds_u8* kb1 = (lds_u8*)k_lds1;
  lds_u8* vb0 = (lds_u8*)v_lds0;
  lds_u8* vb1 = (lds_u8*)v_lds1;

  // Tile it computes from buffer it % 2 while tile it + 1 loads into the
  // other one.  Tiles [0, n_full) lie wholly below every row's causal limit
  // (and inside the sequence); only the rest need the mask and the tail fill.
  auto run_tile = [&](int it, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const bool odd = (it & 1) != 0;
    if (MASKED && it * BK + BK > kvl) {
      zero_tail(it, odd ? v_lds1 : v_lds0);
      __syncthreads();
    }
    if (it + 1 < n_tiles) issue_tile(it + 1, odd ? kb0 : kb1, odd ? vb0 : vb1);
    compute_tile(it, odd ? kb1 : kb0, odd ? vb1 : vb0, masked_tag);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  const int n_full = min(n_tiles, (hist + pos0 + 1) / BK);

  fetch_pid(0);
  issue_tile(0, kb0, vb0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Unmasked tiles in pairs, so that each half names its LDS buffers at
  // compile time (which lets the compiler see that the reads of one buffer
  // never wait for the copy into the other).
  int it = 0;
  for (; it + 1 < n_full; it += 2) {
    issue_tile(it + 1, kb1, vb1);
    compute_tile(it, kb0, vb0, BoolTag<false>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 2 < n_tiles) issue_tile(it + 2, kb0, vb0);
    compute_tile(it + 1, kb1, vb1, BoolTag<false>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (; it < n_full; ++it) run_tile(it, BoolTag<false>{});
  for (; it < n_tiles; ++it) run_tile(it, BoolTag<true>{});

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
  const int64_t blocks = (int64_t)a.batch * a.num_kv_heads *
                         (a.xcd_split ? 8 * (int64_t)a.m_tiles_x : (int64_t)a.m_tiles);
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
