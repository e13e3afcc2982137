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
//     clock so that the clock under that load comes out too.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

}  // namespace pkv
