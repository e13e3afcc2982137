// Measurement aids: the ceilings the kernels' rooflines are read against.
//
// Not part of the attention path.  The bench runs them on the same GPU, in
// the same process, to report measured denominators beside the nominal
// peaks:
//   - a read probe: every byte of a buffer read once with 16-byte streaming
//     loads, either sequentially or as whole blocks in a caller-given order
//     (the decode's pattern: randomly placed 4 KiB (page, head) blocks);
//   - a matrix-core probe: a register-only loop of 32x32x16 bf16 MFMAs on
//     random operands, alone or with the vector work the prefill kernel
//     does per MFMA, timed in shader clocks and in the 100 MHz constant
//     clock so that the clock under that load comes out too;
//   - the prefill kernel's tile loop on its own: the same MFMAs, LDS operand
//     reads and vector work per 64-key tile and wave, without the page
//     copies, barriers, masks or rescaling around them.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint8_t __attribute__((address_space(3))) lds_t;

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;          // 16-byte loads in flight per thread

// Sequential: workgroup w reads 16-byte vectors w * T + i, stepping by the
// whole grid.  The accumulated XOR is stored only if it equals a value the
// caller passes and no data is expected to produce, so the loads cannot be
// dropped and nothing is written in practice.
__global__ __launch_bounds__(kReadThreads) void read_seq_kernel(const uint4* buf, int64_t n_vec,
                                                                uint32_t never,
                                                                uint32_t* sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  for (; i + (kReadUnroll - 1) * stride < n_vec; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = load16_stream(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].w[0] ^ v[u].w[1] ^ v[u].w[2] ^ v[u].w[3];
  }
  for (; i < n_vec; i += stride) {
    const u32x4 v = load16_stream(buf + i);
    acc ^= v.w[0] ^ v.w[1] ^ v.w[2] ^ v.w[3];
  }
  if (acc == never) sink[0] = acc;
}

// Blocks: the buffer is read as whole blocks of block_bytes (a multiple of
// 4 KiB) in the order `order` gives (ids outside [0, n_blocks) are skipped).
// Each 4 KiB piece is one 16-byte vector per thread; workgroup w takes
// pieces w, w + G, ... (pieces of one block are consecutive), kReadUnroll
// pieces in flight.
__global__ __launch_bounds__(kReadThreads) void read_blocks_kernel(const char* buf,
                                                                   const int32_t* order,
                                                                   int32_t n_blocks,
                                                                   int32_t block_bytes,
                                                                   uint32_t never,
                                                                   uint32_t* sink) {
  uint32_t acc = 0;
  const int k = block_bytes / 4096;
  const int n_piece = n_blocks * k;      // < 2^31: the host checks bytes / 4096
  const int stride = gridDim.x;
  for (int p0 = blockIdx.x; p0 < n_piece; p0 += stride * kReadUnroll) {
    // the pieces' block ids first, then all loads back to back (a piece past
    // the end or with an id out of range reads block 0 and is dropped)
    int piece[kReadUnroll];
    bool use[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int p = p0 + u * stride;
      const int id = p < n_piece ? order[p / k] : -1;
      use[u] = id >= 0 && id < n_blocks;
      piece[u] = use[u] ? id * k + p % k : 0;
    }
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = load16_stream(buf + (int64_t)piece[u] * 4096 + threadIdx.x * 16);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      if (use[u]) acc ^= v[u].w[0] ^ v[u].w[1] ^ v[u].w[2] ^ v[u].w[3];
  }
  if (acc == never) sink[0] = acc;
}

// Matrix-core loop: each wave runs `iters` rounds of 4 independent 32x32x16
// bf16 MFMAs on operands loaded from `ops` (256 16-byte vectors).  VEC adds,
// per MFMA, the prefill kernel's vector work per 32 scores and 16 keys:
// a scale-and-shift FMA, an exp2, an add into a running sum and, every
// second MFMA, a bf16 pair conversion.  Wave 0 of workgroup 0 records its
// shader-clock and constant-clock (100 MHz) cycle counts.
template <bool VEC>
__global__ __launch_bounds__(512) void mfma_loop_kernel(const uint4* ops, int32_t iters,
                                                        uint32_t never, uint32_t* sink,
                                                        int64_t* clocks) {
  const int lane = threadIdx.x & 63;
  const uint4 a4 = ops[(threadIdx.x * 7 + 3) & 255];
  const uint4 b4 = ops[(threadIdx.x * 13 + 5) & 255];
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, a4);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, b4);
  f32x16_t acc[4] = {};
  float x[4], sum[4];
  uint32_t pk = 0;
  for (int i = 0; i < 4; ++i) {
    x[i] = -(float)((lane + i) & 15) * 0.0625f;
    sum[i] = 0.f;
  }
  const float c = __builtin_bit_cast(float, a4.x & 0x3f7fffffu) * 0.5f;   // in (0, 1)
  const int64_t t0 = clock64();
  const int64_t r0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m], 0, 0, 0);
      if constexpr (VEC) {
        const float p = __builtin_amdgcn_exp2f(fmaf(x[m], c, -1.f));
        sum[m] += p;
        x[m] = p - 1.f;
        if (m & 1) {
          const f32x2_t v = {x[m - 1], x[m]};
          pk ^= __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
        }
      }
    }
  }
  const int64_t t1 = clock64();
  const int64_t r1 = wall_clock64();
  float s = 0.f;
  for (int m = 0; m < 4; ++m)
    for (int i = 0; i < 16; ++i) s += acc[m][i];
  for (int i = 0; i < 4; ++i) s += sum[i];
  const uint32_t h = __builtin_bit_cast(uint32_t, s) ^ pk;
  if (h == never) sink[0] = h;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = r1 - r0;
  }
}

// The prefill kernel's per-wave work on one 64-key tile at bf16, head_dim
// 128, 32 query rows per wave, two waves per SIMD: K and V tiles in LDS in
// that kernel's layout (256-byte key rows, 16-byte chunk c of row r at
// c ^ swz(r)), filled once from `ops`; Q^T in registers.  Per tile: 16 QK
// MFMAs (two 32-key blocks x 8 k-steps of 16 head dims, K operands read from
// LDS) and, with VEC, the weights of the previous tile's scores beside them
// (an FMA, an exp2 and an add per score, a bf16 pair conversion per two);
// then 16 PV MFMAs (4 k-steps of 16 keys x 4 blocks of 32 head dims) with
// V^T operands from transposing LDS reads.  Without VEC the PV steps take
// fixed B operands and the scores accumulate across tiles, so that no MFMA
// is dead code.  Each iteration runs two tiles.
__device__ __forceinline__ int tile_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <bool VEC>
__global__ __launch_bounds__(512, 1) void prefill_loop_kernel(const uint4* ops, int32_t iters,
                                                              uint32_t never, uint32_t* sink,
                                                              int64_t* clocks) {
  constexpr int ROWB = 256;
  __shared__ __align__(1024) uint8_t kt[64 * ROWB];
  __shared__ __align__(1024) uint8_t vt[64 * ROWB];
  const int t = threadIdx.x, lane = t & 63, n = lane & 31, half = lane >> 5;
  for (int i = t; i < 64 * ROWB / 16; i += 512) {
    reinterpret_cast<uint4*>(kt)[i] = ops[(i * 3 + 1) & 255];
    reinterpret_cast<uint4*>(vt)[i] = ops[(i * 5 + 2) & 255];
  }
  bf16x8_t qr[8], pfix[4];
  for (int i = 0; i < 8; ++i) qr[i] = __builtin_bit_cast(bf16x8_t, ops[(t * 3 + 7 + 17 * i) & 255]);
  for (int i = 0; i < 4; ++i) pfix[i] = __builtin_bit_cast(bf16x8_t, ops[(t * 5 + 1 + 13 * i) & 255]);
  __syncthreads();
  // per-lane LDS byte offsets: K operand of k-step ks; V^T operand of block db
  // (key slots 0..3 and 4..7 at k-step 0; k-step ks adds 16 rows)
  int k_off[8], va_off[4], vb_off[4];
  for (int ks = 0; ks < 8; ++ks) k_off[ks] = n * ROWB + (((2 * ks + half) ^ tile_swz(n)) * 16);
  const int q16 = lane >> 4, li = lane & 15, kk = li >> 2, jj = li & 3;
  const int key0 = 4 * (q16 >> 1) + kk;
  for (int db = 0; db < 4; ++db) {
    const int dcol = 32 * db + 16 * (q16 & 1) + 4 * jj;
    const int lc = dcol >> 3, sub8 = (dcol & 7) * 2;
    va_off[db] = key0 * ROWB + ((lc ^ tile_swz(key0)) * 16) + sub8;
    vb_off[db] = (key0 + 8) * ROWB + ((lc ^ tile_swz(key0 + 8)) * 16) + sub8;
  }
  const lds_t* kl = (const lds_t*)kt;
  const lds_t* vl = (const lds_t*)vt;
  const float c = 0.1f + (t & 7) * 1e-3f;
  const float mc = 0.25f;
  f32x16_t s0[2] = {}, s1[2] = {}, o[4] = {};
  float l = 0.f;
  const f32x16_t zero16 = {};

  auto tile = [&](f32x16_t (&sc)[2], f32x16_t (&sn)[2]) {
    __asm__ volatile("" ::: "memory");   // operands are read from LDS every tile
    bf16x8_t pk[4];
    float ls = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (VEC) {
        const int kb = g >> 1, sub = g & 1;
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][8 * sub + e], c, -mc));
          ls += p[e];
        }
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2_t v = {p[2 * e], p[2 * e + 1]};
          w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
        }
        pk[g] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      } else {
        pk[g] = pfix[g];
      }
      bf16x8_t ka[4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        ka[x] = *reinterpret_cast<const bf16x8_t __attribute__((address_space(3)))*>(
            kl + (x & 1) * 32 * ROWB + k_off[2 * g + (x >> 1)]);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int ks = 2 * g + (x >> 1), kb = x & 1;
        sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x], qr[ks],
                                                         (VEC && ks == 0) ? zero16 : sn[kb], 0,
                                                         0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t va[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4_t __attribute__((address_space(3)))*)(vl + ks * 16 * ROWB + va_off[db]));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4_t __attribute__((address_space(3)))*)(vl + ks * 16 * ROWB + vb_off[db]));
        const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
        va[db] = __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], pk[ks], o[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    l += ls;
  };

  const int64_t t0 = clock64();
  const int64_t r0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
    tile(s0, s1);
    tile(s1, s0);
  }
  const int64_t t1 = clock64();
  const int64_t r1 = wall_clock64();
  float s = l;
  for (int i = 0; i < 16; ++i) {
    s += s0[0][i] + s0[1][i] + s1[0][i] + s1[1][i];
    for (int db = 0; db < 4; ++db) s += o[db][i];
  }
  const uint32_t h = __builtin_bit_cast(uint32_t, s);
  if (h == never) sink[0] = h;
  if (blockIdx.x == 0 && t == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, const int32_t* order,
                             int32_t block_bytes, uint32_t never, uint32_t* sink, int grid,
                             hipStream_t stream) {
  if (order == nullptr) {
    hipLaunchKernelGGL(read_seq_kernel, dim3(grid), dim3(kReadThreads), 0, stream,
                       (const uint4*)buf, (int64_t)(bytes / 16), never, sink);
  } else {
    hipLaunchKernelGGL(read_blocks_kernel, dim3(grid), dim3(kReadThreads), 0, stream,
                       (const char*)buf, order, (int32_t)(bytes / block_bytes), block_bytes,
                       never, sink);
  }
  return hipGetLastError();
}

hipError_t launch_mfma_probe(const void* ops, int32_t iters, int32_t vec, int grid,
                             uint32_t never, uint32_t* sink, int64_t* clocks,
                             hipStream_t stream) {
  if (vec)
    hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(grid), dim3(512), 0, stream,
                       (const uint4*)ops, iters, never, sink, clocks);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(grid), dim3(512), 0, stream,
                       (const uint4*)ops, iters, never, sink, clocks);
  return hipGetLastError();
}

hipError_t launch_prefill_loop_probe(const void* ops, int32_t iters, int32_t vec, int grid,
                                     uint32_t never, uint32_t* sink, int64_t* clocks,
                                     hipStream_t stream) {
  if (vec)
    hipLaunchKernelGGL(prefill_loop_kernel<true>, dim3(grid), dim3(512), 0, stream,
                       (const uint4*)ops, iters, never, sink, clocks);
  else
    hipLaunchKernelGGL(prefill_loop_kernel<false>, dim3(grid), dim3(512), 0, stream,
                       (const uint4*)ops, iters, never, sink, clocks);
  return hipGetLastError();
}

}  // namespace pkv
