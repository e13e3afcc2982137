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
// head_dim 128, or 64 with 16-bit pools (the tiles then hold 128-byte rows;
// the QK products take half the k-steps and PV half the output blocks).
//
// Work decomposition.  A workgroup (8 wavefronts, one per CU) owns 256 query
// rows of one (sequence, KV head): 256 / G chunk positions times the G query
// heads that share the KV head (page 4, section 2.2, GQA), so the G heads
// reuse every K/V tile.  Wave w owns rows 32w .. 32w+31.  Keys go in tiles of
// 64 (four pages); direct global-to-LDS loads (no registers) bring each K and
// V page into LDS once for all 256 rows, one tile ahead of its use.
//
// LDS layout: K and V tiles are stored as they sit in the pages, one 256-byte
// row per key, with the sixteen 16-byte chunks of row r permuted by
// chunk ^ swz(r) so that the operand reads below hit distinct banks.
//
// Per tile and wave, on 32x32x16 MFMAs with fp32 accumulation:
//   S^T (64 keys x 32 rows) = K x Q^T: K rows are read as 16-byte chunks, Q^T
//       stays in registers.  The scores of a query row sit in one lane (16 per
//       32-key block, the other 16 in lane + 32).
//   online softmax in base 2 (log2 e folded into the scale) against a lazy
//       reference max: the weights exp2(c (s - m)) are formed with the current
//       reference m, which moves to the running max (rescaling the
//       accumulators) only when a weight could exceed 2^8 (its lane's sum
//       does) or no reference is set yet.
//   O^T (128 x 32) += V^T x P^T: the weights are converted in place to
//       bf16/f16 (the S^T output layout is the P^T operand layout), and the
//       V^T operand comes from transposing LDS reads (ds_read_b64_tr_b16) of
//       the row-major V tile, with keys taken in the order P^T holds them.
// The tiles are software-pipelined per wave: the MFMAs that form S of the
// next tile run beside the vector work of this tile's weights.
// Keys past the causal limit or the sequence end are selected out of S; V
// rows past the sequence end are zeroed in LDS before use, so stale or NaN
// slots in a partly filled last page never reach the products.
//
// fp8 pools (OCP E4M3 / E5M2 with one fp32 scale per pool, queries f16 or
// bf16; page 4, section 3.1 prefills in chunks over an e5m2 cache): a page
// block is 2 KiB.  The wave that copies a page brings it into a staging
// buffer of its own and, halfway through the iteration (after its weights,
// before its PV step), waits for its own copies and widens the page exactly to
// the query type into the same swizzled tile the 16-bit pools use (every fp8
// value is exact in f16 and in bf16); from there the tile loop is the same.
// Each element is widened once per workgroup, not once per wave that reads
// it.  The K scale is folded into the softmax scale, the V scale into the
// final normalisation.
//
// Shared-prefix form (the first pass of a cascade decode): the decode queries
// of many sequences that share their first pages (page 2, section 3.2:
// identical prompt prefixes share physical pages) form one "sequence" of
// query rows; every row sees every key of the shared pages (no causal mask),
// the keys are cut into splits so that enough workgroups run, and each split
// writes fp32 partial results (out / l and the log-sum-exp) for the same
// log-sum-exp merge that combines split-KV decode partials.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int P = kPageSize;
constexpr int BK = 64;           // keys per tile (4 pages)
constexpr int NWP = 8;           // waves per workgroup
constexpr int ROWS = 256;        // query rows per workgroup
constexpr int kLazyLog2 = 8;     // weights stay below 2^(8 + POFF)
constexpr int kRankMax = 256;    // longest-first sequence order up to this batch

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
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
// for 64 LDS banks (256 bytes per cycle).
// NCH = 16 (head_dim 128, 256-byte rows): a bijection on r % 16, so the K
// operand reads of 16 consecutive rows at one logical chunk hit all 16 chunk
// positions; and it puts r % 4 into chunk bits 2-3 and r / 4 % 4 into bits
// 0-1, so the transposing V reads of 32 lanes (4 keys x two adjacent 32-byte
// chunk pairs) cover 8 distinct chunk pairs.
// NCH = 8 (head_dim 64, 128-byte rows: rows r and r + 1 share the 64 banks,
// one half each): x = (r / 2) % 8 is mapped by a bijection g, so the 8 rows
// of one parity among 16 consecutive rows hit 8 distinct chunks; g sends x
// and x + 1 (the two keys of one parity among 4 consecutive keys) to
// different chunk pairs, which keeps the transposing V reads apart.
template <int NCH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (NCH == 16) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
  }
}

// Direct global-to-LDS copy through a buffer descriptor: lane i's 16 bytes
// at byte offset voff of the buffer go to lds_base + 16 * i.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, lds_u8* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)lds_base,
                                           16, voff, 0, 0, 0);
}
// Descriptor of one (page, head) block of `bytes` bytes (4 KiB at 16 bits, 2
// KiB in fp8): base address, no stride, 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

// Transposing LDS read: in each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte chunks addressed by lanes 4k + i / 4, k = 0..3.
__device__ __forceinline__ uint2 read_tr(const lds_u8* p) {
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4_t __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(uint2, r);
}

// TT: type of q, out and the tiles' elements; CT: type of the pools (TT, or
// an fp8 type); D: head_dim (128, or 64 for 16-bit pools); PFX: the
// shared-prefix form (one sequence, no causal mask, key splits, fp32
// partials) instead of a chunked prefill.
template <typename TT, typename CT, int D, int G, bool PFX>
__global__ __launch_bounds__(NWP * 64, 1) void prefill_kernel(PrefillArgs a) {
  using M = Mfma<TT>;
  constexpr bool F8 = CT::is_fp8;
  constexpr int ROWB = D * 2;       // bytes per tile row (a key's D elements of TT)
  constexpr int TILEB = BK * ROWB;  // bytes per K or V tile
  constexpr int NCH = ROWB / 16;    // 16-byte chunks per tile row
  constexpr int KS = D / 16;        // QK k-steps (16 head dims each)
  constexpr int QG = KS / 2;        // QK groups of two k-steps
  constexpr int DB = D / 32;        // PV output blocks of 32 head dims
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(!F8 || D == 128, "fp8 pools are built for head_dim 128");
  constexpr int PAGEB = P * D * CT::bytes;  // bytes of one (page, head) block
  constexpr int NPOS = ROWS / G;  // chunk positions per workgroup
  __shared__ __align__(1024) uint8_t k_lds0[TILEB];
  __shared__ __align__(1024) uint8_t k_lds1[TILEB];
  __shared__ __align__(1024) uint8_t v_lds0[TILEB];
  __shared__ __align__(1024) uint8_t v_lds1[TILEB];
  // fp8: one staging page per wave (the page it copies, before widening)
  __shared__ __align__(1024) uint8_t stg[F8 ? NWP * PAGEB : 16];
  __shared__ int bad_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int half = lane >> 5;     // which 32-lane half
  const int n = lane & 31;        // this lane's query row within the wave

  // Workgroups are handed to the 8 XCDs round-robin (workgroup i to XCD
  // i % 8), and each XCD has its own L2.  Default order: (b, kv head) fastest,
  // so when there are at least 8 such pairs each XCD keeps whole pairs and all
  // their query tiles share the K/V stream in its L2.  With xcd_split (long
  // chunks) the query tiles of each pair are dealt round the XCDs, tile mt to
  // XCD (mt + pair) % 8: a pair's tiles on one XCD still read the same keys
  // (all start at key 0), every XCD gets light and heavy causal tiles alike,
  // and the first tile of the pairs -- all a one-row chunk has -- lands on a
  // different XCD for each pair.
  // Longest first: a workgroup of a causal chunk sees more keys the higher its
  // tile, so each mapping hands out the heavy tiles first, and with xcd_split
  // each XCD walks the sequences by decreasing key count (their KV heads
  // interleaved, so that a long sequence's workgroups start together).  When
  // there are more workgroups than CUs, the CU that frees first (lightest
  // work so far) then takes the heaviest of the workgroups still waiting: the
  // two 4093-row chunks of an 8192-token batch (histories 0 and 65536) with
  // the short one first had put its heaviest tiles before the long chunk's
  // heaviest on the same CUs.
  const int nbg = a.batch * a.num_kv_heads;
  int bg, mt, ks = 0;
  if (!PFX && a.xcd_split) {
    const int x = blockIdx.x % 8, j = blockIdx.x / 8;
    const int hk = a.num_kv_heads;
    const int jt = j / hk;
    const int r = jt / a.m_tiles_x;            // rank of the sequence
    const int k = jt % a.m_tiles_x;            // k-th heaviest tile of its pairs here
    // the sequence of rank r by (kv_len descending, index ascending); batches
    // above kRankMax keep their index order
    __shared__ int seq_of_rank;
    if (a.batch <= kRankMax) {
      for (int s = tid; s < a.batch; s += NWP * 64) {
        const int ws = a.kv_lens[s];
        int rk = 0;
        for (int o = 0; o < a.batch; ++o) {
          const int wo = a.kv_lens[o];
          rk += (wo > ws || (wo == ws && o < s)) ? 1 : 0;
        }
        if (rk == r) seq_of_rank = s;
      }
      __syncthreads();
    }
    const int bq = a.batch <= kRankMax ? seq_of_rank : r;
    bg = bq * hk + j % hk;
    mt = 8 * (a.m_tiles_x - 1 - k) + ((x + 8 - (bg & 7)) & 7);
    if (mt >= a.m_tiles) return;     // padding past the last tile
  } else if constexpr (PFX) {        // key split next, so a split's row tiles share L2
    bg = blockIdx.x % nbg;
    const int id = blockIdx.x / nbg;
    ks = id % a.n_ksplit;
    mt = id / a.n_ksplit;
  } else {
    bg = blockIdx.x % nbg;
    mt = a.m_tiles - 1 - blockIdx.x / nbg;
  }
  const int b = bg / a.num_kv_heads;
  const int g = bg % a.num_kv_heads;

  // sequence geometry, with broken preconditions clamped and flagged
  const int q0 = PFX ? 0 : a.q_indptr[b];
  int C = PFX ? (int)a.total_q : a.q_indptr[b + 1] - q0;
  int kvl = PFX ? a.kv_len0 : a.kv_lens[b];
  const int kv_min = PFX ? 0 : C;   // causal rows are the last C keys
  bool bad = false;
  if (C < 0 || C > a.max_q_len || kvl < kv_min || kvl > a.stride * P || q0 < 0) {
    bad = true;
    C = max(0, min(C, a.max_q_len));
    kvl = max(kv_min, min(kvl, a.stride * P));
  }
  const int pos0 = mt * NPOS;
  if (pos0 >= C) return;  // this tile of positions is past the chunk
  const int npos = min(NPOS, C - pos0);
  const int hist = kvl - C;
  // keys seen by the last row here; the tiles of this key split
  const int n_keys = PFX ? kvl : hist + pos0 + npos;
  const int tile0 = PFX ? ks * a.split_tiles : 0;
  const int tiles_all = (n_keys + BK - 1) / BK;
  const int n_tiles = PFX ? max(0, min(tiles_all, tile0 + a.split_tiles) - tile0) : tiles_all;
  const int seq_pages = (kvl + P - 1) / P;
  const int32_t* bt_row = a.block_table + (int64_t)b * a.stride;

  // this lane's query row
  const int row = 32 * w + n;
  const int pos = pos0 + row / G;
  const int head = g * G + row % G;
  const int64_t qrow = (int64_t)q0 + pos;
  const bool row_ok = (row / G) < npos && qrow >= 0 && qrow < a.total_q;
  const int apos = PFX ? kvl - 1 : hist + pos;   // last key this row sees

  if (PFX && n_tiles == 0) {   // an empty key split: o = 0, lse = -inf
    if (row_ok) {
      const int64_t prow = (qrow * a.num_q_heads + head) * a.part_stride + ks;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float z = bad ? __builtin_nanf("") : 0.f;
          *reinterpret_cast<float4*>(a.o_part + prow * D + 32 * db + 8 * j + 4 * half) =
              make_float4(z, z, z, z);
        }
      if (half == 0) a.lse_part[prow] = bad ? __builtin_nanf("") : -INFINITY;
    }
    return;
  }

  // Q^T operand: 8 k-steps of 16 head dims; lane holds 8 consecutive dims
  u32x4_t qreg[KS];
  {
    const bool neg = a.scale_log2 < 0.f;  // fold the sign of the scale into q
    const char* qp = (const char*)a.q + ((qrow * a.num_q_heads + head) * D) * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
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

  // ---- staging: waves 0-3 copy the K and the V pages of a tile, wave w
  // page w of each (key rows 16w .. +15), as four 1-KiB LDS
  // chunks of four rows; lane i of a chunk fills row 4j + i/16, physical
  // chunk i%16 with logical chunk (i%16) ^ swz(row).  The page, its
  // descriptor and the LDS destination are the same for the whole wave
  // (scalar registers); each lane adds a fixed offset.  fp8: the page goes
  // unpermuted into the wave's staging buffer as two 1-KiB chunks, and
  // widen_page() fills the tile rows.
  const int64_t head_block = (int64_t)PAGEB;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int wp = wu & 3;          // page of the tile this wave copies
  // Waves 0-3 copy the tile's pages, K and V (wave w: page w of the tile);
  // waves 4-7 copy nothing.  The two waves on a SIMD (w and w + 4) share its
  // issue slots and the older one (w) gets ahead, so the younger one ends
  // each tile; with the copies split between them (w: K, w + 4: V), w waited
  // ~1100 of a tile's ~3500 cycles at the barrier while w + 4 finished its
  // copies and its products.  All copies on w took ~450 cycles off the tile.
  const bool kwave = wu < 4;
  constexpr int NDMA = PAGEB / 1024;             // 1-KiB copies per page (16-bit pools)
  constexpr int RPC = 1024 / ROWB;               // tile rows per 1-KiB copy
  uint32_t dma_off[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int r = RPC * j + lane / NCH;          // key row within the page
    dma_off[j] = (uint32_t)(r * ROWB + (((lane % NCH) ^ swz<NCH>(r)) * 16));
  }
  bool my_bad = false;
  // block-table entry of this wave's page of tile t (0 past the sequence)
  auto load_pid = [&](int t) -> int {
    const int pi = (tile0 + t) * (BK / P) + wp;
    return (t < n_tiles && pi < seq_pages) ? bt_row[pi] : 0;
  };
  // wave-uniform page id, flagged and replaced by page 0 when out of range
  auto check_pid = [&](int t, int loaded) -> int {
    const int pid = __builtin_amdgcn_readfirstlane(loaded);
    const int pi = (tile0 + t) * (BK / P) + wp;
    const bool out = pid < 0 || pid >= a.num_pages;
    if (pi < seq_pages && out) my_bad = true;
    return out ? 0 : pid;
  };
  // fp8: a copying wave stages its K page in slot wp and its V page in slot
  // wp + 4 of stg (a constant offset from the K slot, folded into the LDS
  // instructions)
  lds_u8* stg_k = (lds_u8*)(stg + (F8 ? wp * PAGEB : 0));
  constexpr int STG_V = F8 ? 4 * PAGEB : 0;
  auto copy_page = [&](const void* pool, int pid, lds_u8* dst, lds_u8* staging) {
    const __amdgpu_buffer_rsrc_t r =
        page_rsrc((const char*)pool + ((int64_t)pid * a.num_kv_heads + g) * head_block, PAGEB);
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < PAGEB / 1024; ++j) dma16(r, (uint32_t)(j * 1024 + 16 * lane), staging + j * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < NDMA; ++j) dma16(r, dma_off[j], dst + (16 * wp + RPC * j) * ROWB);
    }
  };
  // fp8: widen the staged page (after this wave's own copy has landed) into
  // rows 16wp .. 16wp+15 of tile dst: lane i takes the 8-element chunks
  // i, i+64, i+128, i+192 of the page (row = chunk / 16, logical chunk =
  // chunk % 16) and stores each at its swizzled place.
  auto widen_page = [&](lds_u8* dst, const lds_u8* staging) {
    if constexpr (F8) {
#pragma unroll 1
      for (int i = 0; i < P * NCH / 64; ++i) {
        const int ch = lane + 64 * i, r = ch / NCH, lc = ch % NCH;
        const u32x2_t x = *reinterpret_cast<const u32x2_t __attribute__((address_space(3)))*>(
            staging + r * (D * CT::bytes) + lc * 8);
        u32x4_t y;
        y[0] = CT::template cvt2<TT, false>(x[0]);
        y[1] = CT::template cvt2<TT, true>(x[0]);
        y[2] = CT::template cvt2<TT, false>(x[1]);
        y[3] = CT::template cvt2<TT, true>(x[1]);
        *reinterpret_cast<u32x4_t __attribute__((address_space(3)))*>(
            dst + (16 * wp + r) * ROWB + ((lc ^ swz<NCH>(r)) * 16)) = y;
      }
    }
  };
  // V rows of keys past the sequence end become zero (edge tiles only)
  auto zero_tail = [&](int it, uint8_t* vdst) {
    const int first = kvl - (tile0 + it) * BK;   // first row to clear
    for (int idx = tid; idx < BK * (ROWB / 16); idx += NWP * 64) {
      const int r = idx / (ROWB / 16);
      if (r >= first)
        *reinterpret_cast<uint4*>(vdst + r * ROWB + (idx % (ROWB / 16)) * 16) =
            make_uint4(0u, 0u, 0u, 0u);
    }
  };

  // ---- accumulators
  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  // reference max of this row (raw scores): the running max at its last
  // update; the accumulators hold weights exp2(c * (s - m_run)) * 2^POFF
  float m_run = -INFINITY;
  float l_run = 0.f;        // sum of this lane's weights (keys of its half)

  // Per-lane LDS byte offsets, the same for every tile: the K operand of
  // k-step ks (row n, logical chunk 2ks + half) and the V^T operand reads of
  // head-dim block db for key slots 0..3 (a) and 4..7 (b) at k-step 0.
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = n * ROWB + (((2 * ks + half) ^ swz<NCH>(n)) * 16);
  const int q16 = lane >> 4, li = lane & 15;
  const int kk = li >> 2, jj = li & 3;
  const int key_a0 = 4 * (q16 >> 1) + kk;      // key of slots 0..3 at k-step 0
  int va_off[DB], vb_off[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int dcol = 32 * db + 16 * (q16 & 1) + 4 * jj;   // first of 4 head dims
    const int lc = dcol >> 3, sub8 = (dcol & 7) * 2;      // chunk, byte in chunk
    va_off[db] = key_a0 * ROWB + ((lc ^ swz<NCH>(key_a0)) * 16) + sub8;
    vb_off[db] = (key_a0 + 8) * ROWB + ((lc ^ swz<NCH>(key_a0 + 8)) * 16) + sub8;
  }

  // S^T = K Q^T of one tile, two 32-key blocks: score i of block kb is key
  // t0 + 32kb + 8(i/4) + 4half + i%4 of this lane's row.  Group g covers the
  // k-steps 2g, 2g+1 of both blocks (four MFMAs).
  typedef u32x4_t KOps[4];
  auto k_read = [&](const lds_u8* kt, int g, KOps& ka) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
      ka[x] = *reinterpret_cast<const u32x4_t __attribute__((address_space(3)))*>(
          kt + (x & 1) * 32 * ROWB + k_off[2 * g + (x >> 1)]);
  };
  auto s_group = [&](int g, const KOps& ka, f32x16_t (&s)[2]) {
    const f32x16_t zero16 = {};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int ks = 2 * g + (x >> 1), kb = x & 1;
      s[kb] = M::run(ka[x], qreg[ks], ks == 0 ? zero16 : s[kb]);
    }
  };
  auto s_tile = [&](const lds_u8* kt, f32x16_t (&s)[2]) {
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      KOps ka;
      k_read(kt, g, ka);
      s_group(g, ka, s);
    }
  };
  // keys past this row's position (or the sequence end) are selected out
  auto mask_tile = [&](int it, f32x16_t (&s)[2]) {
    const int thr = min(apos, kvl - 1) - (tile0 + it) * BK - 4 * half;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        s[kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3) <= thr) ? s[kb][i] : -INFINITY;
  };
  // Weights of keys 16ks .. 16ks+15 against the reference max (mc = m_run *
  // c - POFF), packed as the B operand of PV k-step ks; their fp32 sum goes
  // into ls.
  auto weights = [&](const f32x16_t (&s)[2], int ks, float mc, u32x4_t& pk, float& ls) {
    const int kb = ks >> 1, sub = ks & 1;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2_fast(fmaf(s[kb][8 * sub + e], c, -mc));   // masked: exp2(-inf) = 0
      ls += p[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = M::pack(p[2 * e], p[2 * e + 1]);
  };
  // O^T += V^T P^T for k-step ks.  The 16-lane group q16 = lane / 16 covers
  // head dims 32db + 16 (q16 & 1) .. +15 with key half h = q16 >> 1; source
  // lane 4k + j of the group points at key (16ks + 4h + k) (+8 for slots
  // 4..7), dims +4j .. +4j+3, so result lane i holds dim +i for keys k = 0..3.
  // The swizzle of key 16ks + x equals that of key x, so k-step ks only adds
  // 16 rows to the k-step 0 offsets.
  typedef u32x4_t VOps[DB];
  auto v_read = [&](const lds_u8* vt, int ks, VOps& va) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint2 lo = read_tr(vt + ks * 16 * ROWB + va_off[db]);
      const uint2 hi = read_tr(vt + ks * 16 * ROWB + vb_off[db]);
      va[db][0] = lo.x;
      va[db][1] = lo.y;
      va[db][2] = hi.x;
      va[db][3] = hi.y;
    }
  };
  auto pv_step = [&](const VOps& va, const u32x4_t& pk) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = M::run(va[db], pk, o[db]);
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  // ---- software pipeline over key tiles.  Iteration j holds S(j) in
  // registers, K(j+1) and V(j) in LDS, and:
  //   copies (waves 0-3) V(j+1) into the other V buffer and K(j+2) into the
  //   buffer K(j) used; every wave finished with both buffers before the
  //   last barrier;
  //   computes S(j+1) on the matrix cores while the vector units form the
  //   weights of S(j) against the current reference (the stream is fenced
  //   into regions of four MFMAs, each with its K operand reads and the
  //   weights of one 16-key step, which bounds the registers in flight);
  //   checks the weights (rare fix-up, below);
  //   O += P(j) V(j);
  //   waits for its copies and meets the other waves.
  // Tiles [0, n_full) lie wholly below every row's causal limit (and inside
  // the sequence); only the rest need the mask and the V tail fill.  S(j+1)
  // is formed even for the last tile (from a buffer that no copy targets;
  // the result is unused) so that the stream has no branch.  The LDS
  // buffers are named at compile time in each instance (even / odd j), which
  // lets the compiler see that reads of one buffer never wait for the copy
  // into another.
  const float wmax = __builtin_ldexpf(1.f, kLazyLog2 + (int)M::POFF);
  int pid_f = 0;      // block-table entry of the page this wave copies next
  int pid_v = 0;      // checked page id of the V page this wave copies next
  auto iteration = [&](int j, lds_u8* kd, const lds_u8* kc, uint8_t* vc_raw, lds_u8* vd,
                       f32x16_t (&s_cur)[2], f32x16_t (&s_nxt)[2], auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const lds_u8* vc = (const lds_u8*)vc_raw;
    // V(j+1), from the id checked when K(j+1) was copied, and K(j+2); both
    // land before this iteration's closing barrier
    if (kwave) {
      if (j + 1 < n_tiles) copy_page(a.v_cache, pid_v, vd, stg_k + STG_V);
      if (j + 2 < n_tiles) {
        pid_v = check_pid(j + 2, pid_f);
        copy_page(a.k_cache, pid_v, kd, stg_k);
      }
      pid_f = load_pid(j + 3);
    }
    if constexpr (MASKED) mask_tile(j, s_cur);
    fence();

    // S(j+1) beside the weights of S(j)
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * c - M::POFF;
    u32x4_t pk[4];
    float ls = 0.f;
    KOps ka;
    // head_dim 64 has two QK groups: they go with every second weights step
    constexpr int QSTEP = 4 / QG;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g % QSTEP == 0) k_read(kc, g / QSTEP, ka);
      weights(s_cur, g, mc, pk[g], ls);
      if (g % QSTEP == 0) s_group(g / QSTEP, ka, s_nxt);
      fence();
    }
    // A weight above 2^(8+POFF) shows in its lane's sum; so does a reference
    // not set yet.  Then the reference moves to the running max (the wave
    // votes; rare: scores seldom grow by more than 8 in log2 units), the
    // accumulators are rescaled and the weights recomputed.  A NaN sum does
    // not vote, so NaN reaches the output.
    if (__ballot(ls > wmax || m_run == -INFINITY) != 0) {
      __asm__ volatile("");   // keep this a branch: it is rare
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_cur[kb][i]);
      mx = fmaxf(mx, xor_f(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m_run = m_new;
      const float mc2 = (m_run == -INFINITY) ? 0.f : m_run * c - M::POFF;
      ls = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) weights(s_cur, g, mc2, pk[g], ls);
    }
    fence();
    // fp8: widen the pages this wave copied above, once its copies have
    // landed.  Their destinations (K(j), read in iteration j-1, and V(j-1),
    // read in that iteration's PV) are free since the last barrier and read
    // only after the next one; widening here overlaps the other waves' PV.
    if constexpr (F8) {
      if (kwave && j + 1 < n_tiles) {
        __builtin_amdgcn_s_waitcnt(0);
        widen_page(vd, stg_k + STG_V);
        if (j + 2 < n_tiles) widen_page(kd, stg_k);
      }
    }
    if (MASKED && (tile0 + j) * BK + BK > kvl) {
      zero_tail(j, vc_raw);
      __syncthreads();
    }
    VOps v0, v1;
    v_read(vc, 0, v0);
    v_read(vc, 1, v1);
    pv_step(v0, pk[0]);
    fence();
    v_read(vc, 2, v0);
    pv_step(v1, pk[1]);
    fence();
    v_read(vc, 3, v1);
    pv_step(v0, pk[2]);
    fence();
    pv_step(v1, pk[3]);
    l_run += ls;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  lds_u8* kb0 = (lds_u8*)k_lds0;
  lds_u8* kb1 = (lds_u8*)k_lds1;
  lds_u8* vb0 = (lds_u8*)v_lds0;
  lds_u8* vb1 = (lds_u8*)v_lds1;
  f32x16_t s0[2], s1[2];

  // prologue: K(0), V(0), K(1) in; S(0)
  {
    const int pid0 = check_pid(0, load_pid(0));
    if (kwave) {
      copy_page(a.k_cache, pid0, kb0, stg_k);
      copy_page(a.v_cache, pid0, vb0, stg_k + STG_V);
      if constexpr (F8) {
        __builtin_amdgcn_s_waitcnt(0);
        widen_page(kb0, stg_k);
        widen_page(vb0, stg_k + STG_V);
      }
      if (n_tiles > 1) {
        pid_v = check_pid(1, load_pid(1));
        copy_page(a.k_cache, pid_v, kb1, stg_k);
        if constexpr (F8) {
          __builtin_amdgcn_s_waitcnt(0);
          widen_page(kb1, stg_k);
        }
      }
      pid_f = load_pid(2);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    s_tile(kb0, s0);
    __syncthreads();   // every wave has read K(0): its buffer takes K(2)
  }
  // tiles wholly below every row's limit and inside the sequence
  const int n_full = PFX ? max(0, min(n_tiles, kvl / BK - tile0))
                         : min(n_tiles, (hist + pos0 + 1) / BK);
  int j = 0;
  for (; j + 1 < n_full; j += 2) {
    iteration(j, kb0, kb1, v_lds0, vb1, s0, s1, BoolTag<false>{});
    iteration(j + 1, kb1, kb0, v_lds1, vb0, s1, s0, BoolTag<false>{});
  }
  if (j < n_full) {
    iteration(j, kb0, kb1, v_lds0, vb1, s0, s1, BoolTag<false>{});
    ++j;
  }
  if (j < n_tiles && (j & 1)) {
    iteration(j, kb1, kb0, v_lds1, vb0, s1, s0, BoolTag<true>{});
    ++j;
  }
  for (; j < n_tiles; j += 2) {
    iteration(j, kb0, kb1, v_lds0, vb1, s0, s1, BoolTag<true>{});
    if (j + 1 < n_tiles) iteration(j + 1, kb1, kb0, v_lds1, vb0, s1, s0, BoolTag<true>{});
  }

  // ---- epilogue
  if (my_bad) bad_flag = 1;
  __syncthreads();
  const float l_tot = l_run + xor_f(l_run, 32);
  if (!row_ok) return;
  const bool poison = bad_flag != 0;
  const float inv = a.v_scale / l_tot;   // v_scale: 1 for 16-bit pools
  if constexpr (PFX) {   // fp32 partials of key split ks
    const int64_t prow = (qrow * a.num_q_heads + head) * a.part_stride + ks;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float4 v = make_float4(o[db][4 * j] * inv, o[db][4 * j + 1] * inv,
                               o[db][4 * j + 2] * inv, o[db][4 * j + 3] * inv);
        if (poison) v = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                    __builtin_nanf(""));
        *reinterpret_cast<float4*>(a.o_part + prow * D + 32 * db + 8 * j + 4 * half) = v;
      }
    if (half == 0) {
      float lse = (m_run * c + log2_fast(l_tot) - M::POFF) * kLn2;
      if (m_run == -INFINITY) lse = -INFINITY;
      a.lse_part[prow] = poison ? __builtin_nanf("") : lse;
    }
    return;
  }
  char* op = (char*)a.out + ((qrow * a.num_q_heads + head) * D) * 2;
#pragma unroll
  for (int db = 0; db < DB; ++db)
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

template <typename TT, typename CT, int D, bool PFX>
hipError_t launch_g(int group, const dim3 grid, const PrefillArgs& a, hipStream_t stream) {
  const dim3 block(NWP * 64);
  switch (group) {
    case 1: hipLaunchKernelGGL((prefill_kernel<TT, CT, D, 1, PFX>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<TT, CT, D, 2, PFX>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<TT, CT, D, 4, PFX>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<TT, CT, D, 8, PFX>), grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL((prefill_kernel<TT, CT, D, 16, PFX>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TT, typename CT, int D>
hipError_t launch_t(int group, const PrefillArgs& a, hipStream_t stream) {
  const bool pfx = a.o_part != nullptr;
  const int64_t blocks = (int64_t)a.batch * a.num_kv_heads *
                         (a.xcd_split ? 8 * (int64_t)a.m_tiles_x : (int64_t)a.m_tiles) *
                         (pfx ? a.n_ksplit : 1);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  return pfx ? launch_g<TT, CT, D, true>(group, grid, a, stream)
             : launch_g<TT, CT, D, false>(group, grid, a, stream);
}

template <typename TT>
hipError_t launch_q(int kv_dtype, int head_dim, int group, const PrefillArgs& a,
                    hipStream_t stream) {
  switch (kv_dtype) {
    case 1:
    case 2:
      if (head_dim == 64) return launch_t<TT, TT, 64>(group, a, stream);
      if (head_dim == 128) return launch_t<TT, TT, 128>(group, a, stream);
      return hipErrorInvalidValue;
    case 3:
      return head_dim == 128 ? launch_t<TT, TFP8E4M3, 128>(group, a, stream)
                             : hipErrorInvalidValue;
    case 4:
      return head_dim == 128 ? launch_t<TT, TFP8E5M2, 128>(group, a, stream)
                             : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int prefill_rows_per_tile(int group) { return ROWS / group; }

hipError_t launch_prefill(int kv_dtype, int q_dtype, int head_dim, int group,
                          const PrefillArgs& a, hipStream_t stream) {
  if (kv_dtype != 3 && kv_dtype != 4 && kv_dtype != q_dtype) return hipErrorInvalidValue;
  switch (q_dtype) {
    case 1: return launch_q<TF16>(kv_dtype, head_dim, group, a, stream);
    case 2: return launch_q<TBF16>(kv_dtype, head_dim, group, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
