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
// w, w+4, w+8, ... of the split, keeping four independent page streams in
// flight per workgroup.  Each wave keeps its own (m, l, acc) state; the four
// are combined through LDS at the end.
//
// Per page (16 tokens x D elements, one contiguous 2-8 KiB block per head):
//   K, "row layout": 8 lanes per token, 8 tokens per pass, 2 passes; lane c of
//      a token reads 16-byte vectors c, c+8, ... so each load instruction
//      reads whole 128-byte lines.  q for the G heads sits in registers in the
//      same layout.  Partial dot products (packed dot2 for f16/bf16, fp32 FMA
//      for f32) are summed over the 8 lanes with three DPP adds.
//   softmax: the running max is updated only when some score exceeds it
//      (a wave vote); otherwise the page costs one exp2 per score.
//   V, "column layout": DG = D / vec lanes cover one token row, 64 / DG token
//      groups; each lane accumulates G x vec outputs over its tokens.  The
//      probabilities cross from the row layout to the column layout through
//      a small per-wave LDS buffer.
// Tokens past the end of the sequence (the tail of the last page) are
// selected out, never multiplied by zero, so stale or NaN slots never leak.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int P = kPageSize;
constexpr int NW = kDecodeWaves;

template <typename TT, int D, int G>
struct DecodeCfg {
  static constexpr int ES = TT::bytes;
  static constexpr int VEC = 16 / ES;        // elements per 16-byte vector
  static constexpr int KL = 8;               // lanes per K row
  static constexpr int KT = 64 / KL;         // tokens per K pass
  static constexpr int KP = P / KT;          // K passes per page
  static constexpr int KV = D / (KL * VEC);  // 16-byte vectors per lane per K row
  static constexpr int DG = D / VEC;         // lanes per V row
  static constexpr int TG = 64 / DG;         // V token groups
  static constexpr int VT = P / TG;          // V tokens per lane per page
  static_assert(KV >= 1 && KV * KL * VEC == D, "head_dim / vector mismatch");
  static_assert(TG >= 1 && VT * TG == P, "V layout mismatch");
};

// Partial dot product of one lane's slice of q and of a K row.
template <typename TT, int KV>
__device__ __forceinline__ float dot_slice(const u32x4 (&q)[KV], const u32x4 (&k)[KV]) {
  float acc = 0.f;
  if constexpr (TT::bytes == 4) {
#pragma unroll
    for (int v = 0; v < KV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(u2f(q[v].w[i]), u2f(k[v].w[i]), acc);
  } else {
#pragma unroll
    for (int v = 0; v < KV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = TT::dot2(q[v].w[i], k[v].w[i], acc);
  }
  return acc;
}

// Widen one 16-byte vector of V to floats.
template <typename TT, int VEC>
__device__ __forceinline__ void widen(const u32x4& x, float (&f)[VEC]) {
  if constexpr (TT::bytes == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = u2f(x.w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = TT::lo(x.w[i]);
      f[2 * i + 1] = TT::hi(x.w[i]);
    }
  }
}

template <typename TT, int D, int G>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using C = DecodeCfg<TT, D, G>;
  constexpr int ES = C::ES, VEC = C::VEC;
  __shared__ float p_lds[NW][P][G];
  __shared__ float red_m[NW][G];
  __shared__ float red_l[NW][G];
  __shared__ float red_acc[NW][G][D];
  __shared__ int bad_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  int bid = blockIdx.x;
  const int ks = bid % a.n_split;
  bid /= a.n_split;
  const int g = bid % a.num_kv_heads;
  const int b = bid / a.num_kv_heads;
  const int hq0 = g * G;

  // Pages reachable through the grid and the table row; a length outside
  // [0, that * P] breaks a precondition: clamp it and poison the row.
  const int cover = min(a.n_split * a.pages_per_split, a.stride);
  int L = a.context_lens[b];
  const bool len_bad = (L < 0) || (L > cover * P);
  L = len_bad ? max(0, min(L, cover * P)) : L;
  const int n_pages = (L + P - 1) / P;
  const int p0 = ks * a.pages_per_split;
  const int p1 = min(n_pages, p0 + a.pages_per_split);

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
        a.o_part[(row * a.n_split + ks) * D + d] = o;
        if (d == 0) a.lse_part[row * a.n_split + ks] = lse;
      }
    }
    return;
  }
  if (tid == 0) bad_flag = 0;

  // q slices for the G heads, row layout.
  const int c = lane & (C::KL - 1);
  const int tk = lane / C::KL;
  u32x4 qv[G][C::KV];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int v = 0; v < C::KV; ++v)
      qv[h][v] = load16((const char*)a.q +
                        (((int64_t)b * a.num_q_heads + hq0 + h) * D + v * C::KL * VEC + c * VEC) *
                            ES);

  const int dg = lane % C::DG;
  const int tg = lane / C::DG;

  float m[G], l_lane[G], acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l_lane[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
  }

  const int32_t* bt_row = a.block_table + (int64_t)b * a.stride;
  const int my_pages = (p1 - p0 > w) ? (p1 - p0 - w + NW - 1) / NW : 0;
  const int64_t head_block = (int64_t)P * D * ES;  // bytes of one (page, head) block
  bool wave_bad = false;
  int pid_vec = 0;
  __syncthreads();

  for (int i = 0; i < my_pages; ++i) {
    if ((i & 63) == 0) {  // page ids of the next 64 pages of this wave, one per lane
      const int idx = i + lane;
      pid_vec = idx < my_pages ? bt_row[p0 + w + NW * idx] : 0;
    }
    int pid = __builtin_amdgcn_readlane(pid_vec, i & 63);
    if (pid < 0 || pid >= a.num_pages) {
      wave_bad = true;
      pid = 0;
    }
    const int pi = p0 + w + NW * i;  // logical page index
    const int64_t blk = ((int64_t)pid * a.num_kv_heads + g) * head_block;
    const char* kb = (const char*)a.k_cache + blk;
    const char* vb = (const char*)a.v_cache + blk;

    u32x4 kr[C::KP][C::KV];
#pragma unroll
    for (int r = 0; r < C::KP; ++r)
#pragma unroll
      for (int v = 0; v < C::KV; ++v)
        kr[r][v] = load16(kb + ((tk + C::KT * r) * D + v * C::KL * VEC + c * VEC) * ES);
    u32x4 vr[C::VT];
#pragma unroll
    for (int j = 0; j < C::VT; ++j) vr[j] = load16(vb + ((tg + C::TG * j) * D + dg * VEC) * ES);

    const bool partial = (pi + 1) * P > L;

    // scores (log2 units)
    float s[C::KP][G];
#pragma unroll
    for (int r = 0; r < C::KP; ++r) {
      const bool valid = !partial || (pi * P + tk + C::KT * r < L);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float d = sum8(dot_slice<TT, C::KV>(qv[h], kr[r]));
        s[r][h] = valid ? d * a.scale_log2 : -INFINITY;
      }
    }

    // running max: reduce and rescale only when some score exceeds it
    bool need = false;
#pragma unroll
    for (int r = 0; r < C::KP; ++r)
#pragma unroll
      for (int h = 0; h < G; ++h) need |= s[r][h] > m[h];
    if (__ballot(need) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = s[0][h];
#pragma unroll
        for (int r = 1; r < C::KP; ++r) mx = fmaxf(mx, s[r][h]);
        mx = fmaxf(mx, dpp_f<kDppRowRor8>(mx));
        mx = fmaxf(mx, xor_f(mx, 16));
        mx = fmaxf(mx, xor_f(mx, 32));
        const float mn = fmaxf(m[h], mx);
        const float alpha = exp2_fast(m[h] - mn);
        m[h] = mn;
        l_lane[h] *= alpha;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] *= alpha;
      }
    }

    float p[C::KP][G];
#pragma unroll
    for (int r = 0; r < C::KP; ++r)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        p[r][h] = exp2_fast(s[r][h] - m[h]);
        l_lane[h] += p[r][h];
      }

    // probabilities: row layout -> column layout through LDS
    wave_lds_sync();
    if (c == 0) {
#pragma unroll
      for (int r = 0; r < C::KP; ++r)
#pragma unroll
        for (int h = 0; h < G; ++h) p_lds[w][tk + C::KT * r][h] = p[r][h];
    }
    wave_lds_sync();

#pragma unroll
    for (int j = 0; j < C::VT; ++j) {
      const int t = tg + C::TG * j;
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = p_lds[w][t][h];
      float vf[VEC];
      widen<TT, VEC>(vr[j], vf);
      if (partial && pi * P + t >= L) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(pv[h], vf[e], acc[h][e]);
    }
  }

  // l: sum over the 8 token groups of the row layout
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = l_lane[h];
    x += dpp_f<kDppRowRor8>(x);
    x += xor_f(x, 16);
    x += xor_f(x, 32);
    l_lane[h] = x;
  }
  // acc: sum over the token groups of the column layout
#pragma unroll
  for (int msk = C::DG; msk < 64; msk <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] += xor_f(acc[h][e], msk);

  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      red_m[w][h] = m[h];
      red_l[w][h] = l_lane[h];
    }
  }
  if (tg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) red_acc[w][h][dg * VEC + e] = acc[h][e];
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
      a.o_part[(row * a.n_split + ks) * D + d] = o;
      if (d == 0) a.lse_part[row * a.n_split + ks] = lse;
    }
  }
}

template <typename TT, int D>
hipError_t launch_g(int group, int batch, const DecodeArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)batch * a.num_kv_heads * a.n_split;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(NW * 64);
  switch (group) {
    case 1: hipLaunchKernelGGL((decode_kernel<TT, D, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<TT, D, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<TT, D, 4>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_kernel<TT, D, 8>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TT>
hipError_t launch_d(int head_dim, int group, int batch, const DecodeArgs& a,
                    hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_g<TT, 64>(group, batch, a, stream);
    case 128: return launch_g<TT, 128>(group, batch, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(int dtype, int head_dim, int group, int batch, const DecodeArgs& a,
                         hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_d<TF32>(head_dim, group, batch, a, stream);
    case 1: return launch_d<TF16>(head_dim, group, batch, a, stream);
    case 2: return launch_d<TBF16>(head_dim, group, batch, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
