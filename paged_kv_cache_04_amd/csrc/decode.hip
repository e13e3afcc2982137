// Paged decode attention: one query token per sequence against its paged K/V,
// GQA, split over the keys (flash-decoding) with a log-sum-exp merge.
//
// What is computed (page 2, section 2.1): out = softmax(q K^T * scale) V for
// each query head, keys 0 .. len-1 of the sequence, where key t lives in page
// block_table[b][t / 16] at offset t % 16 (page 3, section 3.2).  The keys are
// consumed page by page with an online softmax (page 2, section 2.2): a running
// maximum m, a running sum l of exp(s - m) and a running weighted sum of V
// rows, rescaled whenever m grows.  Exponentials are base 2 with log2(e)
// folded into the scale.
//
// Work decomposition.  One workgroup (4 wavefronts) owns one (sequence b, KV
// head g, split k) and all G = H_q / H_kv query heads of that KV head, so each
// K/V page block is read from HBM once per KV head, never once per query head
// (page 4, section 2.2: GQA shares KV heads).  A split is a run of
// pages_per_split logical pages; wave w of the workgroup takes pages
// w, w+4, w+8, ... of the split.  Each wave keeps its own (m, l, acc) state;
// the four are combined through LDS at the end.  Every wave keeps the loads
// of the next pages in flight while it computes the current one (register
// buffers: two for 16-bit pools at G <= 4, which then fit three workgroups
// per CU -- more resident waves hide the start-up of short sequences --, three
// for 16-bit pools at G = 8 and two for f32, at two workgroups per CU; five
// for fp8).  K/V are read once, with streaming (non-temporal) loads.
//
// Per page (16 tokens x D elements, one contiguous 2-8 KiB block per head):
//   K, "row layout": 8 lanes per token, 8 tokens per pass, 2 passes; lane c of
//      a token reads 16-byte vectors c, c+8, ... so each load instruction
//      reads whole 128-byte lines.  q for the G heads sits in registers in the
//      same layout.  Each lane forms G partial dot products (packed dot2 for
//      f16/bf16, fp32 FMA for f32).  A transposed butterfly over the 8 lanes
//      (three DPP exchanges, each halving the values a lane keeps) leaves lane
//      c holding the complete score of head c >> (3 - log2 G), so the softmax
//      work of a page (max vote, exp2, running sum) is done once per
//      (token, head), not once per lane.
//   running max: updated only when some score exceeds it (a wave vote), then
//      reduced over the tokens and broadcast per head with v_readlane.
//   V, "column layout": each lane holds 4 consecutive elements of a token row
//      (8-byte loads for f16/bf16, 16-byte for f32), D / 4 lanes per row and
//      64 / (D / 4) token groups; each lane accumulates G x 4 fp32 outputs.
//      For f16/bf16 the probabilities are rounded to the value type and stored
//      as pairs of tokens in LDS; V elements of the same two tokens are paired
//      with v_perm, and one packed dot2 adds both tokens' contributions.  f16
//      probabilities are carried as p * 2^15 (exact power-of-two scaling; the
//      largest is 2^15 < 65504) so that small weights keep their precision.
//      For f32 the probabilities stay fp32 and PV is plain FMA.
// Tokens past the end of the sequence (the tail of the last page) are
// selected out, never multiplied by zero, so stale or NaN slots never leak.
//
// fp8 caches (OCP E4M3 / E5M2, one scale per pool): K vectors hold 16
// elements, each widened exactly to the query's type (f16 or bf16) with the
// hardware pair conversion right before the packed dot products; V rows of
// two tokens are interleaved byte-wise with v_perm and widened into the same
// token pairs the 16-bit path forms.  The K scale is folded into the softmax
// scale, the V scale into the final normalisation.  Pages carry half the
// bytes, so five pages per wave are kept in flight instead of three.
//
// Sliding window (page 4, section 2.3): with window w > 0 a sequence of L
// keys shows keys t >= L - w and t < sink.  The visited logical pages are
// [0, sp) (the sink) and [wp, n_pages) (the window); splits run over this
// list of visited pages, so hidden pages cost nothing, not even a table
// lookup.  Keys inside a visited page that are hidden are selected out like
// the tail of the last page.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_append.h"

namespace pkv {

namespace {

constexpr int P = kPageSize;
constexpr int NW = kDecodeWaves;

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// QT: type of q and out; CT: type of the cache elements (QT itself, or an
// fp8 type with QT f16 / bf16).
template <typename QT, typename CT, int D, int G>
struct DecodeCfg {
  static constexpr int ES = CT::bytes;       // cache element bytes
  static constexpr int QES = QT::bytes;
  static constexpr bool FP8 = CT::is_fp8;
  static constexpr int VEC = 16 / ES;        // elements per 16-byte K vector
  static constexpr int KL = 8;               // lanes per K row
  static constexpr int KT = 64 / KL;         // tokens per K pass
  static constexpr int KP = P / KT;          // K passes per page
  static constexpr int KV = D / (KL * VEC);  // 16-byte vectors per lane per K row
  static constexpr int QW = VEC * QES / 16;  // 16-byte q vectors per K vector
  static constexpr int VE = 4;               // V elements per lane per token
  static constexpr int VW = VE * ES / 4;     // 32-bit words of one V load (1, 2 or 4)
  static constexpr int DG = D / VE;          // lanes per V row
  static constexpr int TG = 64 / DG;         // V token groups
  static constexpr int VT = P / TG;          // V tokens per lane per page
  static constexpr int HSHIFT = 3 - ilog2(G);  // lane c owns head c >> HSHIFT
  static constexpr bool PACKED = (QES == 2); // packed-pair PV for 16-bit queries
  // f16 probabilities are stored as p * 2^15
  static constexpr float POFF = QT::is_f16 ? 15.f : 0.f;
  // pages in flight per wave: the one being computed plus NB - 1 ahead; OCC:
  // workgroups per CU the registers are sized for
  static constexpr bool OCC3 = !FP8 && ES == 2 && G <= 4;
  static constexpr int NB = FP8 ? 5 : ((ES == 4 || OCC3) ? 2 : 3);
  // f32 at head_dim 128 with G >= 4 holds 16 G registers of q per lane: one
  // workgroup per CU (a wave per SIMD, 512 registers) instead of spilling
  static constexpr bool OCC1 = ES == 4 && D == 128 && G >= 4;
  static constexpr int OCC = OCC3 ? 3 : (OCC1 ? 1 : 2);
  static_assert(KV >= 1 && KV * KL * VEC == D, "head_dim / vector mismatch");
  static_assert(QW >= 1, "q vector layout");
  static_assert(TG >= 1 && VT * TG == P, "V layout mismatch");
  static_assert(!PACKED || VT % 2 == 0, "packed PV pairs tokens");
  static_assert(!FP8 || QES == 2, "fp8 caches take f16 or bf16 queries");
  static_assert(FP8 || ES == QES, "one element type unless the cache is fp8");
  static_assert(G >= 1 && G <= 8 && (G & (G - 1)) == 0, "group size");
};

// Partial dot product of one lane's slice of q and of a K row.
template <typename QT, typename CT, int KV, int QW>
__device__ __forceinline__ float dot_slice(const u32x4 (&q)[KV][QW], const u32x4 (&k)[KV]) {
  float acc = 0.f;
  if constexpr (CT::bytes == 4) {
#pragma unroll
    for (int v = 0; v < KV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(u2f(q[v][0].w[i]), u2f(k[v].w[i]), acc);
  } else if constexpr (CT::is_fp8) {
    // k word i holds elements 4i .. 4i+3; q word j holds elements 2j, 2j+1
#pragma unroll
    for (int v = 0; v < KV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t kw = k[v].w[i];
        acc = QT::dot2(q[v][i / 2].w[(2 * i) % 4], CT::template cvt2<QT, false>(kw), acc);
        acc = QT::dot2(q[v][i / 2].w[(2 * i) % 4 + 1], CT::template cvt2<QT, true>(kw), acc);
      }
  } else {
#pragma unroll
    for (int v = 0; v < KV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = QT::dot2(q[v][0].w[i], k[v].w[i], acc);
  }
  return acc;
}

// One transposed butterfly step over a lane bit: the lane keeps half of its N
// values (the upper half if `hi`), sends the other half to its partner and adds
// what the partner sends.  Afterwards v[0 .. N/2) hold the kept half.
template <int N, int CTRL>
__device__ __forceinline__ void tstep(float (&v)[8], bool hi) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float a = v[i], b = v[i + N / 2];
    const float send = hi ? a : b;
    const float keep = hi ? b : a;
    v[i] = keep + dpp_f<CTRL>(send);
  }
}

// Sum G per-lane partials over the 8 lanes of a token; lane c returns the
// full sum for head c >> (3 - log2 G).
template <int G>
__device__ __forceinline__ float reduce_heads(float (&v)[8], int c) {
  if constexpr (G >= 2) tstep<G, kDppHalfMirror>(v, (c & 4) != 0);
  else v[0] += dpp_f<kDppHalfMirror>(v[0]);
  if constexpr (G >= 4) tstep<G / 2, kDppQuadXor2>(v, (c & 2) != 0);
  else v[0] += dpp_f<kDppQuadXor2>(v[0]);
  if constexpr (G >= 8) tstep<G / 4, kDppQuadXor1>(v, (c & 1) != 0);
  else v[0] += dpp_f<kDppQuadXor1>(v[0]);
  return v[0];
}

// Max / sum over the 8 token groups of the row layout (lane bits 3..5).
__device__ __forceinline__ float max_tokens(float x) {
  x = fmaxf(x, dpp_f<kDppRowRor8>(x));
  x = fmaxf(x, xor_f(x, 16));
  return fmaxf(x, xor_f(x, 32));
}
__device__ __forceinline__ float sum_tokens(float x) {
  x += dpp_f<kDppRowRor8>(x);
  x += xor_f(x, 16);
  return x + xor_f(x, 32);
}

template <typename QT, typename CT, int D, int G>
struct PageRegs {
  using C = DecodeCfg<QT, CT, D, G>;
  u32x4 k[C::KP][C::KV];
  uint32_t v[C::VT][C::VW];
};

// WIN: a sliding window is in force (the visited-page map and the hidden-key
// test are compiled only then).
template <typename QT, typename CT, int D, int G, bool WIN>
__global__ __launch_bounds__(NW * 64, (DecodeCfg<QT, CT, D, G>::OCC)) void decode_kernel(DecodeArgs a) {
  using C = DecodeCfg<QT, CT, D, G>;
  using TT = QT;
  constexpr int ES = C::ES, VEC = C::VEC;
  // probabilities of the current page: packed pairs (16-bit) or floats [t][h]
  constexpr int PWORDS = C::PACKED ? (P / 2) * G : P * G;
  __shared__ uint32_t p_lds[NW][PWORDS];
  __shared__ float red_m[NW][G];
  __shared__ float red_l[NW][G];
  __shared__ float red_acc[NW][G][D];
  __shared__ int bad_flag;
  __shared__ int pid_lds[NW][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  int ks, unit;
  if (!decode_item(blockIdx.x, a, &ks, &unit)) return;   // padding workgroup
  const int g = unit % a.num_kv_heads;
  const int b = unit / a.num_kv_heads;
  const int hq0 = g * G;

  // A length outside [0, stride * P], or more visited pages than the grid
  // covers, breaks a precondition: clamp and poison the row.
  int L = a.context_lens[b];
  bool len_bad = (L < 0) || (L > a.stride * P);
  L = max(0, min(L, a.stride * P));
  const int n_pages = (L + P - 1) / P;
  // visible keys: t >= lo, and t < sink_n (without a window: all of them)
  int lo = 0, sink_n = 0;
  if (WIN && a.window > 0) {
    lo = max(0, L - a.window);
    sink_n = min(a.sink, L);
  }
  // visited pages: logical [0, sp) then [wp, n_pages); virtual page v is
  // logical page v (v < sp) or v + gap
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
        store_elem<TT>(a.out, row * D + d, o);
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

  // row layout: lane = tk * 8 + c
  const int c = lane & (C::KL - 1);
  const int tk = lane / C::KL;
  const int h_own = c >> C::HSHIFT;
  const bool p_writer = (c & ((1 << C::HSHIFT) - 1)) == 0;
  // column layout: lane = tg * DG + dg
  const int dg = lane % C::DG;
  const int tg = lane / C::DG;

  u32x4 qv[G][C::KV][C::QW];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int v = 0; v < C::KV; ++v)
#pragma unroll
      for (int qw = 0; qw < C::QW; ++qw)
        qv[h][v][qw] = load16((const char*)a.q +
                              (((int64_t)b * a.num_q_heads + hq0 + h) * D + v * C::KL * VEC +
                               c * VEC) * C::QES + 16 * qw);

  float m_own = -INFINITY, l_own = 0.f;
  float acc[G][C::VE];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < C::VE; ++e) acc[h][e] = 0.f;

  const int32_t* bt_row = a.block_table + (int64_t)b * a.stride;
  const int my_pages = (p1 - p0 > w) ? (p1 - p0 - w + NW - 1) / NW : 0;
  const int64_t head_block = (int64_t)P * D * ES;  // bytes of one (page, head) block
  bool wave_bad = false;
  uint32_t* pw = p_lds[w];
  __syncthreads();

  // Issue the loads of this wave's i-th page into r.  The wave's page ids are
  // staged in LDS 64 at a time, so a lookup waits only on LDS, never on the
  // K/V loads in flight (those drain only at a refill, once per 64 pages).
  auto issue = [&](PageRegs<QT, CT, D, G>& r, int i) {
    if ((i & 63) == 0) {
      const int idx = i + lane;
      const int v = idx < my_pages ? bt_row[lpage(p0 + w + NW * idx)] : 0;
      wave_lds_sync();
      pid_lds[w][lane] = v;
      wave_lds_sync();
    }
    int pid = __builtin_amdgcn_readfirstlane(pid_lds[w][i & 63]);
    if (pid < 0 || pid >= a.num_pages) {
      wave_bad = true;
      pid = 0;
    }
    const int64_t blk = ((int64_t)pid * a.num_kv_heads + g) * head_block;
    const char* kb = (const char*)a.k_cache + blk;
    const char* vb = (const char*)a.v_cache + blk;
#pragma unroll
    for (int rr = 0; rr < C::KP; ++rr)
#pragma unroll
      for (int v = 0; v < C::KV; ++v)
        r.k[rr][v] = load16_stream(kb + ((tk + C::KT * rr) * D + v * C::KL * VEC + c * VEC) * ES);
#pragma unroll
    for (int j = 0; j < C::VT; ++j) {
      const char* src = vb + ((tg + C::TG * j) * D + dg * C::VE) * ES;
      if constexpr (C::VW == 1) {
        r.v[j][0] = load4_stream(src);
      } else if constexpr (C::VW == 2) {
        const u32x2 x = load8_stream(src);
        r.v[j][0] = x.w[0];
        r.v[j][1] = x.w[1];
      } else {
        const u32x4 x = load16_stream(src);
#pragma unroll
        for (int e = 0; e < 4; ++e) r.v[j][e] = x.w[e];
      }
    }
  };

  // Online-softmax update with the wave's i-th page held in r.
  // key t of a visited page is visible
  auto vis = [&](int t) {
    if constexpr (WIN) return t < L && (t >= lo || t < sink_n);
    return t < L;
  };
  auto compute = [&](const PageRegs<QT, CT, D, G>& r, int i) {
    const int pi = lpage(p0 + w + NW * i);  // logical page index
    const int t0 = pi * P;
    // some key of the page is past the end or hidden by the window
    const bool partial = t0 + P > L || (WIN && max(t0, sink_n) < min(t0 + P, lo));

    float s[C::KP];
#pragma unroll
    for (int rr = 0; rr < C::KP; ++rr) {
      float part[8];
#pragma unroll
      for (int h = 0; h < G; ++h) part[h] = dot_slice<QT, CT, C::KV, C::QW>(qv[h], r.k[rr]);
      const float sc = reduce_heads<G>(part, c) * a.scale_log2;
      const bool valid = !partial || vis(t0 + tk + C::KT * rr);
      s[rr] = valid ? sc : -INFINITY;
    }

    bool need = false;
#pragma unroll
    for (int rr = 0; rr < C::KP; ++rr) need |= s[rr] > m_own;
    if (__ballot(need) != 0) {
      float mx = s[0];
#pragma unroll
      for (int rr = 1; rr < C::KP; ++rr) mx = fmaxf(mx, s[rr]);
      const float mn = fmaxf(m_own, max_tokens(mx));
      const float alpha = exp2_fast(m_own - mn);
      m_own = mn;
      l_own *= alpha;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ah = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(alpha), h << C::HSHIFT));
#pragma unroll
        for (int e = 0; e < C::VE; ++e) acc[h][e] *= ah;
      }
    }

    wave_lds_sync();  // the previous page's probabilities have been read
#pragma unroll
    for (int rr = 0; rr < C::KP; ++rr) {
      const float pf = exp2_fast(s[rr] - m_own + C::POFF);
      l_own += (C::POFF != 0.f) ? pf * (1.f / 32768.f) : pf;
      if (p_writer) {
        const int t = tk + C::KT * rr;
        if constexpr (C::PACKED) {
          const int word = ((t % C::TG) + C::TG * ((t / C::TG) >> 1)) * G + h_own;
          const int half = (t / C::TG) & 1;
          reinterpret_cast<uint16_t*>(pw)[word * 2 + half] = TT::from_float(pf);
        } else {
          reinterpret_cast<float*>(pw)[t * G + h_own] = pf;
        }
      }
    }
    wave_lds_sync();

    if constexpr (C::PACKED) {
#pragma unroll
      for (int pp = 0; pp < C::VT / 2; ++pp) {
        const int ta = tg + C::TG * 2 * pp, tb = ta + C::TG;
        uint32_t wa[C::VW], wb[C::VW];
        const bool va = !partial || vis(t0 + ta), vb_ok = !partial || vis(t0 + tb);
#pragma unroll
        for (int e = 0; e < C::VW; ++e) {
          wa[e] = va ? r.v[2 * pp][e] : 0u;
          wb[e] = vb_ok ? r.v[2 * pp + 1][e] : 0u;
        }
        uint32_t pr[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pr[h] = pw[(tg + C::TG * pp) * G + h];
        if constexpr (C::FP8) {
          // bytes (a0 b0 a1 b1) and (a2 b2 a3 b3), widened to (a_e, b_e) pairs
          const uint32_t x0 = __builtin_amdgcn_perm(wb[0], wa[0], 0x05010400u);
          const uint32_t x1 = __builtin_amdgcn_perm(wb[0], wa[0], 0x07030602u);
          const uint32_t y[4] = {CT::template cvt2<QT, false>(x0),
                                 CT::template cvt2<QT, true>(x0),
                                 CT::template cvt2<QT, false>(x1),
                                 CT::template cvt2<QT, true>(x1)};
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[h][e] = TT::dot2(pr[h], y[e], acc[h][e]);
        } else {
#pragma unroll
          for (int i2 = 0; i2 < C::VW; ++i2) {
            const uint32_t lo2 = __builtin_amdgcn_perm(wb[i2], wa[i2], 0x05040100u);
            const uint32_t hi2 = __builtin_amdgcn_perm(wb[i2], wa[i2], 0x07060302u);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              acc[h][2 * i2] = TT::dot2(pr[h], lo2, acc[h][2 * i2]);
              acc[h][2 * i2 + 1] = TT::dot2(pr[h], hi2, acc[h][2 * i2 + 1]);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::VT; ++j) {
        const int t = tg + C::TG * j;
        const bool valid = !partial || vis(t0 + t);
        const float* pf = reinterpret_cast<const float*>(pw) + t * G;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ph = pf[h];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[h][e] = fmaf(ph, valid ? u2f(r.v[j][e]) : 0.f, acc[h][e]);
        }
      }
    }
  };

  {
    // software pipeline: NB register buffers, loads issued NB - 1 pages ahead
    PageRegs<QT, CT, D, G> rb[C::NB];
#pragma unroll
    for (int j = 0; j < C::NB - 1; ++j)
      if (j < my_pages) issue(rb[j], j);
    for (int i = 0; i < my_pages; i += C::NB) {
#pragma unroll
      for (int u = 0; u < C::NB; ++u) {
        const int ii = i + u;
        if (ii < my_pages) {
          if (ii + C::NB - 1 < my_pages) issue(rb[(u + C::NB - 1) % C::NB], ii + C::NB - 1);
          compute(rb[u], ii);
        }
      }
    }
  }

  // l: the owners of each head sum over the 8 token groups
  l_own = sum_tokens(l_own);
  // acc: sum over the token groups of the column layout
#pragma unroll
  for (int msk = C::DG; msk < 64; msk <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < C::VE; ++e) acc[h][e] += xor_f(acc[h][e], msk);

  if (tk == 0 && p_writer) {
    red_m[w][h_own] = m_own;
    red_l[w][h_own] = l_own;
  }
  if (tg == 0) {
    // undo the f16 probability offset 2^15 (exact) and apply the V scale
    const float unscale = (C::POFF != 0.f ? 1.f / 32768.f : 1.f) * a.v_scale;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < C::VE; ++e) red_acc[w][h][dg * C::VE + e] = acc[h][e] * unscale;
  }
  if (wave_bad) bad_flag = 1;
  __syncthreads();

  const bool any_bad = len_bad || bad_flag != 0;
  for (int idx = tid; idx < G * D; idx += NW * 64) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, red_m[ww][h]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = red_m[ww][h];
      const float e = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
      den = fmaf(e, red_l[ww][h], den);
      num = fmaf(e, red_acc[ww][h][d], num);
    }
    float o = num / den;
    float lse = (M + log2_fast(den)) * kLn2;
    if (any_bad) {
      o = __builtin_nanf("");
      lse = __builtin_nanf("");
    }
    const int64_t row = (int64_t)b * a.num_q_heads + hq0 + h;
    if (a.direct) {
      store_elem<TT>(a.out, row * D + d, o);
      if (d == 0 && a.lse_out) a.lse_out[row] = lse;
    } else {
      a.o_part[(row * a.part_stride + a.part_offset + ks) * D + d] = o;
      if (d == 0) a.lse_part[row * a.part_stride + a.part_offset + ks] = lse;
    }
  }
}

template <typename QT, typename CT, int D, bool WIN>
hipError_t launch_w(int group, const dim3 grid, const DecodeArgs& a, hipStream_t stream) {
  const dim3 block(NW * 64);
  // 16-bit queries at head_dim 128 run G = 4 and 8 on the matrix cores (see
  // decode_mfma_supported): those instances are not built here
  constexpr bool MC = QT::bytes == 2 && D == 128;
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_kernel<QT, CT, D, 1, WIN>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<QT, CT, D, 2, WIN>), grid, block, 0, stream, a); break;
    case 4:
      if constexpr (MC) return hipErrorInvalidValue;
      else hipLaunchKernelGGL((decode_kernel<QT, CT, D, 4, WIN>), grid, block, 0, stream, a);
      break;
    case 8:
      if constexpr (MC) return hipErrorInvalidValue;
      else hipLaunchKernelGGL((decode_kernel<QT, CT, D, 8, WIN>), grid, block, 0, stream, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename QT, typename CT, int D>
hipError_t launch_g(int group, int batch, const DecodeArgs& a, hipStream_t stream) {
  (void)batch;
  const int64_t blocks = decode_grid(a);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  if (a.window > 0) return launch_w<QT, CT, D, true>(group, grid, a, stream);
  return launch_w<QT, CT, D, false>(group, grid, a, stream);
}

template <typename TT>
hipError_t launch_d(int head_dim, int group, int batch, const DecodeArgs& a,
                    hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_g<TT, TT, 64>(group, batch, a, stream);
    case 128: return launch_g<TT, TT, 128>(group, batch, a, stream);
    default: return hipErrorInvalidValue;
  }
}

// fp8 caches: head_dim 128, f16 or bf16 queries
template <typename CT>
hipError_t launch_fp8(int q_dtype, int head_dim, int group, int batch, const DecodeArgs& a,
                      hipStream_t stream) {
  if (head_dim != 128) return hipErrorInvalidValue;
  switch (q_dtype) {
    case 1: return launch_g<TF16, CT, 128>(group, batch, a, stream);
    case 2: return launch_g<TBF16, CT, 128>(group, batch, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(int kv_dtype, int q_dtype, int head_dim, int group, int batch,
                         const DecodeArgs& a, hipStream_t stream) {
  switch (kv_dtype) {
    case 0: return q_dtype == 0 ? launch_d<TF32>(head_dim, group, batch, a, stream)
                                : hipErrorInvalidValue;
    case 1: return q_dtype == 1 ? launch_d<TF16>(head_dim, group, batch, a, stream)
                                : hipErrorInvalidValue;
    case 2: return q_dtype == 2 ? launch_d<TBF16>(head_dim, group, batch, a, stream)
                                : hipErrorInvalidValue;
    case 3: return launch_fp8<TFP8E4M3>(q_dtype, head_dim, group, batch, a, stream);
    case 4: return launch_fp8<TFP8E5M2>(q_dtype, head_dim, group, batch, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
