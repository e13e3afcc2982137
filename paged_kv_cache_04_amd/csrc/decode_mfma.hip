// Paged decode attention on the matrix cores, for grouped queries (G = 4, 8
// and 16).
//
// Same operation and work decomposition as the vector decode kernel: out =
// softmax(q K^T * scale) V for each query head over keys 0 .. len-1 of its
// sequence, reached through the block table (page 2, section 2.1; page 3,
// section 3.2), one workgroup per (sequence, KV head, split) with the G query
// heads of that KV head (page 4, section 2.2), an online softmax per head
// (page 2, section 2.2), split partials merged by log-sum-exp.
//
// With G query heads per KV head the decode is a small matrix product per
// page: S^T (16 keys x G heads) = K Q^T and O^T (D x G) += V^T P^T.  On the
// vector units that is 16 G D multiply-adds per page (256 packed dot products
// per lane at G = 8); on the matrix cores it is a handful of 16x16x32 MFMAs
// with the heads as the N dimension (padded to 16 below G = 16).  A wave takes two pages
// per step (32 keys, the K dimension of one MFMA) so that:
//
//   S^T:  per page, 4 MFMAs (K-dim 128 = 4 x 32) of K (16 keys x 32 dims,
//         straight from HBM into registers) and Q^T (32 dims x 16 heads, held
//         in registers).  The dimension order inside each MFMA is permuted so
//         that a lane's K operand is 16 contiguous bytes of its key row; Q^T
//         uses the same order.  The loads themselves read whole 128-byte
//         lines (8 rows per instruction, two lanes' groups per line), and a
//         select plus a swap of the two 8-lane halves of each 16-lane row
//         rebuild the operand: a load shaped as the operand would read a
//         64-byte half of 16 lines, twice the L2 requests per byte.
//         Output: lane (n = l % 16, q = l / 16) holds the scores of head n
//         for keys 4q .. 4q+3 of the page.
//   P^T:  the scores of both pages, exponentiated, are exactly the B operand
//         of the PV MFMA (keys 4q..4q+3 of page A, then of page B), packed to
//         f16/bf16 in place.
//   O^T:  8 MFMAs (D = 8 blocks of 16 dims); the V^T operand is read from LDS
//         with transposing reads (ds_read_b64_tr_b16 for 16-bit pools, 4 keys
//         of one dimension per read and page; ds_read_b64_tr_b8 for fp8 pools,
//         8 keys of one dimension per read, widened exactly to f16/bf16).  V
//         pages reach LDS by direct buffer loads (no registers), into
//         per-wave buffers whose 32-byte (16-bit) or 16-byte (fp8) chunks are
//         XOR-swizzled by row so that the transposing reads are free of bank
//         conflicts.
//
// Each lane's O^T accumulators belong to a single head, so the online-softmax
// rescale is a lane-local multiply.  The reference max of a head moves only
// when a score exceeds it by more than 8 (log2 units; wave vote); every
// probability then stays <= 2^8, and f16 probabilities carry 2^7 (<= 2^15).
// Keys past the sequence end or hidden by a window are selected out of S; their
// V rows still enter the MFMA, multiplied by an exact zero probability, so they
// are zeroed in LDS first (a NaN or infinity there would survive 0 * V).  Only
// pages that hold such keys need it: the last page of a sequence and the pages
// a window cuts.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_append.h"

namespace pkv {

namespace {

constexpr int P = kPageSize;
constexpr int NW = kDecodeWaves;
constexpr int D = 128;

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint8_t __attribute__((address_space(3))) lds_u8;

template <int N>
struct IntTag {
  static constexpr int value = N;
};

template <typename QT>
struct Mf;

template <>
struct Mf<TF16> {
  static __device__ __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
  }
  static constexpr float POFF = 7.f;   // p carried as p * 2^7 (<= 2^15)
};

template <>
struct Mf<TBF16> {
  static __device__ __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf162_t));
  }
  static constexpr float POFF = 0.f;
};

template <typename QT, typename CT>
struct MCfg {
  static constexpr bool FP8 = CT::is_fp8;
  static constexpr int ROW = D * CT::bytes;    // bytes per key row of one head (256 / 128)
  static constexpr int PAGEB = P * ROW;        // bytes per (page, head) block (4096 / 2048)
  static constexpr int KL = FP8 ? 2 : 4;       // 16-byte K loads per lane and page
  static constexpr int VD = PAGEB / 1024;      // 1-KiB direct loads per V page (4 / 2)
  static constexpr int NB = FP8 ? 3 : 2;       // steps (page pairs) in flight per wave
  // non-temporal (streaming) hints, as measured on the 128K decode: 16-bit
  // pools are fastest with both K loads and V copies streaming (~3% over
  // neither); fp8 pools with only the V copies streaming (both streaming, or
  // neither, is 10-15% slower there)
  static constexpr bool K_NT = !FP8;
  static constexpr bool V_NT = true;
  static constexpr int OPS = 2 * (KL + VD);    // memory instructions per step
  static_assert(NB * OPS <= 63, "vmcnt range");
};

// V page swizzle: 16-bit pools permute the eight 32-byte groups of a 256-byte
// row by row % 8; fp8 pools permute the eight 16-byte chunks of a 128-byte row
// by (row / 2) % 8.  Both keep the transposing reads of one instruction on
// distinct banks.  Returns the byte offset of (row, logical byte b) in LDS.
template <bool FP8>
__device__ __forceinline__ int vswz(int row, int b) {
  if constexpr (FP8)
    return row * 128 + ((((b >> 4) ^ (row >> 1)) & 7) << 4) + (b & 15);
  else
    return row * 256 + ((((b >> 5) ^ row) & 7) << 5) + (b & 31);
}

template <typename QT, typename CT, int G, bool WIN>
__global__ __launch_bounds__(NW * 64, 2) void decode_mfma_kernel(DecodeArgs a) {
  using C = MCfg<QT, CT>;
  using M = Mf<QT>;
  constexpr int PAGEB = C::PAGEB;
  // per-slot V buffers, one object per slot so that the compiler sees that a
  // read of one slot never depends on the copies into the others; the first
  // also holds the cross-wave reduction of the accumulators at the end
  constexpr int VB0 = NW * 2 * PAGEB > NW * G * D * 4 ? NW * 2 * PAGEB : NW * G * D * 4;
  __shared__ __align__(1024) uint8_t vb0[VB0];
  __shared__ __align__(1024) uint8_t vb1[NW * 2 * PAGEB];
  __shared__ __align__(1024) uint8_t vb2[C::NB > 2 ? NW * 2 * PAGEB : 16];
  __shared__ int pid_lds[NW][64];
  __shared__ float red_m[NW][16];
  __shared__ float red_l[NW][16];
  __shared__ int bad_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;       // head column (S^T, P^T, O^T) / key row (K operand)
  const int q = lane >> 4;       // 16-lane group
  int ks, unit;
  if (!decode_item(blockIdx.x, a, &ks, &unit)) return;   // padding workgroup
  const int g = unit % a.num_kv_heads;
  const int b = unit / a.num_kv_heads;
  const int hq0 = g * G;

  int L = a.context_lens[b];
  bool len_bad = (L < 0) || (L > a.stride * P);
  L = max(0, min(L, a.stride * P));
  const int n_pages = (L + P - 1) / P;
  int lo = 0, sink_n = 0;
  if (WIN && a.window > 0) {
    lo = max(0, L - a.window);
    sink_n = min(a.sink, L);
  }
  const int sp = WIN && lo > 0 ? (sink_n + P - 1) / P : 0;
  const int wp = WIN ? max(sp, lo / P) : 0;
  const int gap = wp - sp;
  int n_vp = n_pages - gap;
  const int cover = a.n_split * a.pages_per_split;
  if (n_vp > cover) {
    len_bad = true;
    n_vp = cover;
  }
  const int p0 = ks * a.pages_per_split;
  const int p1 = min(n_vp, p0 + a.pages_per_split);
  auto lpage = [&](int v) {
    if constexpr (WIN) return v < sp ? v : v + gap;
    return v;
  };

  if (p0 >= p1) {  // empty split: no keys, o = 0 and lse = -inf
    for (int idx = tid; idx < G * D; idx += NW * 64) {
      const int h = idx / D, d = idx % D;
      const int64_t row = (int64_t)b * a.num_q_heads + hq0 + h;
      const float o = len_bad ? __builtin_nanf("") : 0.f;
      const float lse = len_bad ? __builtin_nanf("") : -INFINITY;
      if (a.direct) {
        store_elem<QT>(a.out, row * D + d, o);
        if (d == 0 && a.lse_out) a.lse_out[row] = lse;
      } else {
        a.o_part[(row * a.part_stride + a.part_offset + ks) * D + d] = o;
        if (d == 0) a.lse_part[row * a.part_stride + a.part_offset + ks] = lse;
      }
    }
    return;
  }
  if (tid == 0) bad_flag = 0;
  // the split that ends at the last visited page holds position L - 1: store
  // the newest token there first (all of this workgroup's loads come after)
  if (a.k_new != nullptr && !len_bad && L > 0 && p1 == n_vp) {
    append_newest<QT, CT, D>(a, b, g, L, tid, NW * 64);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Q^T operand: lane (head n, group q), MFMA j holds the 8 dims the K
  // operand of the same MFMA uses (16-bit: 32j + 8q ..; fp8: 64(j/2) + 16q +
  // 8(j%2) ..); heads past G are zero.
  u32x4_t qb[4];
  {
    const bool hv = n < G;
    const char* qp = (const char*)a.q + (((int64_t)b * a.num_q_heads + hq0 + (hv ? n : 0)) * D) * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = C::FP8 ? 64 * (j >> 1) + 16 * q + 8 * (j & 1) : 32 * j + 8 * q;
      const u32x4 x = load16(qp + d0 * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) qb[j][e] = hv ? x.w[e] : 0u;
    }
  }

  f32x4_t o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // reference max of head n (log2 units), same in its 4 lanes
  float mref = 0.f;         // m_run - POFF, or 0 before the first key
  float l_lane = 0.f;       // sum of this lane's probabilities (times 2^POFF)

  const int32_t* bt_row = a.block_table + (int64_t)b * a.stride;
  const int n_local = p1 - p0;
  // wave w takes page pairs (2w + 8s, 2w + 8s + 1) of the split, s = 0, 1, ...
  const int my_steps = n_local > 2 * w ? (n_local - 2 * w + 7) / 8 : 0;
  const int64_t head_block = (int64_t)PAGEB;
  bool wave_bad = false;

  u32x4_t kr[C::NB][2][C::KL];

  // Loads of step s into register slot / LDS slot SLOT: K rows of both pages
  // into registers, V pages into this wave's LDS buffer of the slot.
  auto issue = [&](int s, auto slot_tag) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_tag)::value;
    if ((s & 31) == 0) {  // page ids of steps s .. s+31, staged in LDS
      const int v = p0 + 8 * (s + (lane >> 1)) + 2 * w + (lane & 1);
      const int id = v < p1 ? bt_row[lpage(v)] : 0;
      wave_lds_sync();
      pid_lds[w][lane] = id;
      wave_lds_sync();
    }
    uint8_t* vb = SLOT == 0 ? vb0 : (SLOT == 1 ? vb1 : vb2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = p0 + 8 * s + 2 * w + h;
      int pid = __builtin_amdgcn_readfirstlane(pid_lds[w][(2 * s + h) & 63]);
      if (v < p1 && (pid < 0 || pid >= a.num_pages)) wave_bad = true;
      if (v >= p1 || pid < 0 || pid >= a.num_pages) pid = 0;   // a readable page
      const int64_t blk = ((int64_t)pid * a.num_kv_heads + g) * head_block;
      const char* kbase = (const char*)a.k_cache + blk;
      // K rows: loads 2L and 2L + 1 read the 128-byte line L of rows 0 .. 7
      // and 8 .. 15, whole: lane (n, q) of load 2L + x reads row 8x + n % 8,
      // bytes 128L + 64((n / 8) ^ x) + 16q .. +15 (k_operand rebuilds the
      // MFMA layout from the pair)
#pragma unroll
      for (int j = 0; j < C::KL; ++j) {
        const int x = j & 1;
        const int off = ((n & 7) + 8 * x) * C::ROW + 128 * (j >> 1) + 64 * ((n >> 3) ^ x) + 16 * q;
        kr[SLOT][h][j] =
            __builtin_bit_cast(u32x4_t, C::K_NT ? load16_stream(kbase + off) : load16(kbase + off));
      }
      // V page: 1-KiB direct copies; lane i fills LDS bytes 16i .. 16i+15 of
      // the copy, i.e. physical row r / chunk c, holding logical chunk c ^ swz
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const char*)a.v_cache + blk), (short)0, PAGEB, 0x00020000);
      lds_u8* dst = (lds_u8*)(vb + (w * 2 + h) * PAGEB);
#pragma unroll
      for (int c = 0; c < C::VD; ++c) {
        const int pos = c * 1024 + 16 * lane;            // physical byte in the page
        int src;
        if constexpr (C::FP8) {
          const int row = pos >> 7, pc = (pos >> 4) & 7;
          src = row * 128 + (((pc ^ (row >> 1)) & 7) << 4);
        } else {
          const int row = pos >> 8, pg = (pos >> 5) & 7, half = (pos >> 4) & 1;
          src = row * 256 + (((pg ^ row) & 7) << 5) + (half << 4);
        }
        lds_u8* to = dst + c * 1024;
        // the cache policy is an immediate: one literal per form
        if constexpr (C::V_NT)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (void __attribute__((address_space(3)))*)to,
                                                   16, (uint32_t)src, 0, 0, 2);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (void __attribute__((address_space(3)))*)to,
                                                   16, (uint32_t)src, 0, 0, 0);
      }
    }
  };

  // K operand of row n, bytes 64j + 16q .. +15 of the row, from the load
  // pair (X, Y) of line j / 2: the first half of a line sits in X for rows
  // 0 .. 7 and in Y for rows 8 .. 15, each in its own lane; the second half
  // sits in the lane n ^ 8 of X (rows 0 .. 7) or Y (rows 8 .. 15)
  auto k_operand = [&](u32x4_t xr, u32x4_t yr, int j) __attribute__((always_inline)) {
    u32x4_t r;
    const bool lo = n < 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (j & 1) {
        const uint32_t xs = (uint32_t)__builtin_amdgcn_mov_dpp((int)xr[e], kDppRowRor8, 0xF, 0xF, true);
        const uint32_t ys = (uint32_t)__builtin_amdgcn_mov_dpp((int)yr[e], kDppRowRor8, 0xF, 0xF, true);
        r[e] = lo ? xs : ys;
      } else {
        r[e] = lo ? xr[e] : yr[e];
      }
    }
    return r;
  };

  auto vis = [&](int t) {
    if constexpr (WIN) return t < L && (t >= lo || t < sink_n);
    return t < L;
  };

  // Step s from slot SLOT; `later` = steps issued after it (their memory
  // instructions may still be in flight).
  auto compute = [&](int s, int later, auto slot_tag) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_tag)::value;
    // wait for this step's loads (K registers and V copies)
    if (later >= 2) __builtin_amdgcn_s_waitcnt(((2 * C::OPS) & 15) | (((2 * C::OPS) >> 4) << 14) | 0x0F70);
    else if (later == 1) __builtin_amdgcn_s_waitcnt((C::OPS & 15) | ((C::OPS >> 4) << 14) | 0x0F70);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    uint8_t* vb = SLOT == 0 ? vb0 : (SLOT == 1 ? vb1 : vb2);

    int t0[2];
    bool part[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = p0 + 8 * s + 2 * w + h;
      t0[h] = v < p1 ? lpage(v) * P : L;   // a page past the split: every key masked
      part[h] = t0[h] + P > L || (WIN && max(t0[h], sink_n) < min(t0[h] + P, lo));
    }
    // V rows of keys that are not visible (past the end of the sequence, or
    // hidden by a window) enter the MFMA with p = 0: zero them in LDS so that
    // a NaN or infinity stored there cannot turn 0 * V into NaN
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (part[h]) {
        uint8_t* pg = vb + (w * 2 + h) * PAGEB;
#pragma unroll
        for (int it = 0; it < PAGEB / 1024; ++it) {
          const int x = lane + 64 * it;          // 16-byte chunk of the page
          const int row = (x * 16) / C::ROW;     // the swizzle stays inside a row
          if (!vis(t0[h] + row)) *reinterpret_cast<uint4*>(pg + x * 16) = make_uint4(0u, 0u, 0u, 0u);
        }
        wave_lds_sync();
      }
    }

    // S^T for both pages
    f32x4_t sacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sacc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      u32x4_t kop[C::KL];
#pragma unroll
      for (int j = 0; j < C::KL; ++j)
        kop[j] = k_operand(kr[SLOT][h][j & ~1], kr[SLOT][h][j | 1], j);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4_t av;
        if constexpr (C::FP8) {
          const u32x4_t raw = kop[j >> 1];
          const uint32_t w0 = raw[2 * (j & 1)], w1 = raw[2 * (j & 1) + 1];
          av[0] = CT::template cvt2<QT, false>(w0);
          av[1] = CT::template cvt2<QT, true>(w0);
          av[2] = CT::template cvt2<QT, false>(w1);
          av[3] = CT::template cvt2<QT, true>(w1);
        } else {
          av = kop[j];
        }
        sacc[h] = M::run(av, qb[j], sacc[h]);
      }
    }
    // scores of head n, keys t0[h] + 4q + i, in log2 units
    float sc[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = sacc[h][i] * a.scale_log2;
        sc[4 * h + i] = (!part[h] || vis(t0[h] + 4 * q + i)) ? x : -INFINITY;
      }
    float mx = sc[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sc[k]);
    const bool grow = (m_run == -INFINITY) ? (mx > -INFINITY) : (mx - m_run > 8.f);
    if (__ballot(grow) != 0) {
      __asm__ volatile("");   // keep this a branch: the rescale is rare
      float hm = fmaxf(mx, xor_f(mx, 16));
      hm = fmaxf(hm, xor_f(hm, 32));                  // max over the head's 4 lanes
      const float m_new = fmaxf(m_run, hm);
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - m_new);
      l_lane *= alpha;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] *= alpha;
      m_run = m_new;
      mref = (m_run == -INFINITY) ? 0.f : m_run - M::POFF;
    }
    float p[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      p[k] = exp2_fast(sc[k] - mref);                 // masked: exp2(-inf) = 0
      l_lane += p[k];
    }
    u32x4_t pb;
#pragma unroll
    for (int e = 0; e < 4; ++e) pb[e] = M::pack(p[2 * e], p[2 * e + 1]);

    // O^T += V^T P^T, 8 blocks of 16 dims
    const uint8_t* pa = vb + (w * 2 + 0) * PAGEB;
    const uint8_t* pbp = vb + (w * 2 + 1) * PAGEB;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      u32x4_t av;
      if constexpr (C::FP8) {
        // lane 16q + 2k + j addresses key row 4q + k % 4 of page k / 4, dims
        // 16 blk + 8j .. +7; it receives 8 keys of dim 16 blk + n
        const int kk = (lane & 15) >> 1, jj = lane & 1;
        const uint8_t* pg = kk < 4 ? pa : pbp;
        const int row = 4 * q + (kk & 3);
        const i32x2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (i32x2_t __attribute__((address_space(3)))*)(lds_u8*)(pg +
                                                                   vswz<true>(row, 16 * blk + 8 * jj)));
        const uint32_t w0 = (uint32_t)r[0], w1 = (uint32_t)r[1];
        av[0] = CT::template cvt2<QT, false>(w0);
        av[1] = CT::template cvt2<QT, true>(w0);
        av[2] = CT::template cvt2<QT, false>(w1);
        av[3] = CT::template cvt2<QT, true>(w1);
      } else {
        // lane 16q + 4k + j addresses key row 4q + k, dims 16 blk + 4j .. +3;
        // it receives 4 keys of dim 16 blk + n, from each page
        const int kk = (lane & 15) >> 2, jj = lane & 3;
        const int off = vswz<false>(4 * q + kk, 2 * (16 * blk + 4 * jj));
        const i16x4_t ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4_t __attribute__((address_space(3)))*)(lds_u8*)(pa + off));
        const i16x4_t rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4_t __attribute__((address_space(3)))*)(lds_u8*)(pbp + off));
        const uint2 ua = __builtin_bit_cast(uint2, ra), ub = __builtin_bit_cast(uint2, rb);
        av[0] = ua.x;
        av[1] = ua.y;
        av[2] = ub.x;
        av[3] = ub.y;
      }
      o[blk] = M::run(av, pb, o[blk]);
    }
  };

  // Software pipeline over this wave's steps, NB slots deep; step s uses slot
  // s % NB.  The steady-state loop issues exactly one step (NB - 1 ahead)
  // before each compute, so every iteration has the same loads in flight; the
  // last steps drain in a tail without new loads.
  constexpr int NB = C::NB;
  auto prologue = [&](auto u_tag) {
    constexpr int U = decltype(u_tag)::value;
    if (U < my_steps) issue(U, IntTag<U>{});
  };
  prologue(IntTag<0>{});
  if constexpr (NB > 2) prologue(IntTag<1>{});
  int s = 0;
  auto steady = [&](auto u_tag) {
    constexpr int U = decltype(u_tag)::value;
    issue(s + U + NB - 1, IntTag<(U + NB - 1) % NB>{});
    compute(s + U, NB - 1, IntTag<U>{});
  };
  for (; s + 2 * NB - 2 < my_steps; s += NB) {
    steady(IntTag<0>{});
    steady(IntTag<1>{});
    if constexpr (NB > 2) steady(IntTag<2>{});
  }
  auto tail = [&](auto u_tag) {
    constexpr int U = decltype(u_tag)::value;
    if (s + U < my_steps) {
      if (s + U + NB - 1 < my_steps) issue(s + U + NB - 1, IntTag<(U + NB - 1) % NB>{});
      compute(s + U, min(NB - 1, my_steps - 1 - (s + U)), IntTag<U % NB>{});
    }
  };
  tail(IntTag<0>{});
  tail(IntTag<1>{});
  if constexpr (NB > 2) {
    tail(IntTag<2>{});
    tail(IntTag<3>{});
  }

  // ---- combine the 4 waves: per head (m, l) and O^T, through LDS
  const float l_pair = l_lane + xor_f(l_lane, 16);
  const float l_head = l_pair + xor_f(l_pair, 32);   // over the head's 4 lanes
  if (wave_bad) bad_flag = 1;
  __syncthreads();                          // every wave is done with its V buffers
  float* red_o = reinterpret_cast<float*>(vb0);   // [NW][G][D], reuses the V buffers
  if (q == 0) {
    red_m[w][n] = m_run;
    red_l[w][n] = l_head;
  }
  if (n < G) {
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) red_o[(w * G + n) * D + 16 * blk + 4 * q + i] = o[blk][i];
  }
  __syncthreads();

  const bool any_bad = len_bad || bad_flag != 0;
  for (int idx = tid; idx < G * D; idx += NW * 64) {
    const int h = idx / D, d = idx % D;
    float Mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) Mx = fmaxf(Mx, red_m[ww][h]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = red_m[ww][h];
      const float e = (mw == -INFINITY) ? 0.f : exp2_fast(mw - Mx);
      den = fmaf(e, red_l[ww][h], den);
      num = fmaf(e, red_o[(ww * G + h) * D + d], num);
    }
    float out = num / den * a.v_scale;
    float lse = (Mx + log2_fast(den) - M::POFF) * kLn2;
    if (any_bad) {
      out = __builtin_nanf("");
      lse = __builtin_nanf("");
    }
    const int64_t row = (int64_t)b * a.num_q_heads + hq0 + h;
    if (a.direct) {
      store_elem<QT>(a.out, row * D + d, out);
      if (d == 0 && a.lse_out) a.lse_out[row] = lse;
    } else {
      a.o_part[(row * a.part_stride + a.part_offset + ks) * D + d] = out;
      if (d == 0) a.lse_part[row * a.part_stride + a.part_offset + ks] = lse;
    }
  }
}

template <typename QT, typename CT, bool WIN>
hipError_t launch_w(int group, const dim3 grid, const DecodeArgs& a, hipStream_t stream) {
  const dim3 block(NW * 64);
  switch (group) {
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<QT, CT, 4, WIN>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<QT, CT, 8, WIN>), grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<QT, CT, 16, WIN>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename QT, typename CT>
hipError_t launch_c(int group, int batch, const DecodeArgs& a, hipStream_t stream) {
  (void)batch;
  const int64_t blocks = decode_grid(a);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  if (a.window > 0) return launch_w<QT, CT, true>(group, grid, a, stream);
  return launch_w<QT, CT, false>(group, grid, a, stream);
}

template <typename QT>
hipError_t launch_q(int kv_dtype, int group, int batch, const DecodeArgs& a,
                    hipStream_t stream) {
  switch (kv_dtype) {
    case 1:
    case 2: return launch_c<QT, QT>(group, batch, a, stream);
    case 3: return launch_c<QT, TFP8E4M3>(group, batch, a, stream);
    case 4: return launch_c<QT, TFP8E5M2>(group, batch, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Where the matrix cores pay: from 4 query heads per KV head.  At G = 8 the
// vector kernel's 256 packed dot products per page and lane are what limits
// it; at G = 4 it keeps up with memory, but this kernel, with whole-line K
// loads and streaming hints, moves the same bytes 4-5% faster (batch 8 at
// 128K: 626 against 651 us; batch 64 at 0.5-4K: 109 against 115 us).  G = 16
// (a full MFMA N dimension) is built here only; G = 1 and 2 stay on the
// vector kernel, which has no padded heads to carry.
bool decode_mfma_supported(int kv_dtype, int q_dtype, int head_dim, int group) {
  const bool q16 = q_dtype == 1 || q_dtype == 2;
  const bool fp8 = kv_dtype == 3 || kv_dtype == 4;
  if (!q16 || head_dim != D || !(fp8 || kv_dtype == q_dtype)) return false;
  return group == 4 || group == 8 || group == 16;
}

hipError_t launch_decode_mfma(int kv_dtype, int q_dtype, int group, int batch,
                              const DecodeArgs& a, hipStream_t stream) {
  switch (q_dtype) {
    case 1: return launch_q<TF16>(kv_dtype, group, batch, a, stream);
    case 2: return launch_q<TBF16>(kv_dtype, group, batch, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
