// Measured ceilings of this part: what an HBM read stream and the matrix cores sustain
// here, so that the GEMMs can be reported against the chip as it runs (clock under its
// power limit, real memory latency) next to the specification figures.  The method's
// whole point is speed ("[Feature] support qqq(w4a8) for lmdeploy", "Throughput":
// serving throughput of FP16, W4A16 and W4A8 side by side), and a roofline fraction is
// only as meaningful as its denominator.
//
//  * read_stream_kernel: every 16-byte chunk of a buffer read once (grid-stride, U
//    non-temporal loads in flight per thread, as the decode kernels read their weights),
//    the data folded with xor and one word per wave stored, so no load is dead.  Timed by
//    the caller at the byte counts of the GEMMs' weights.
//  * mfma_loop_kernel: C independent accumulator chains of v_mfma_f32_32x32x16_f16 or
//    v_mfma_i32_32x32x32_i8 per wave, no memory traffic in the loop; the operands come
//    from a caller buffer (constant or random values: the sustained rate depends on the
//    data through the power limit).
#include "kernels.hpp"

namespace w4 {

namespace {

template <int U>
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&buf[i + u * stride]);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = buf[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, kWave);
  if ((threadIdx.x & 63) == 0) sink[(int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = acc;
}

constexpr int kChains = 4;

// KIND 0: fp16 32x32x16 (2 * 32 * 32 * 16 flops per MFMA); 1: int8 32x32x32.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(const u32x4* __restrict__ ops, int64_t nops, int iters,
                                                        float* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 a[kChains], b[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    a[c] = ops[(gid * 2 * kChains + 2 * c) % nops];
    b[c] = ops[(gid * 2 * kChains + 2 * c + 1) % nops];
  }
  float total = 0.0f;
  if constexpr (KIND == 0) {
    float16_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = mfma32(__builtin_bit_cast(half8_t, a[c]), __builtin_bit_cast(half8_t, b[c]), acc[c]);
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) total += acc[c][r];
  } else {
    int16_t_ acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = mfma32_i8(__builtin_bit_cast(int4_t, a[c]), __builtin_bit_cast(int4_t, b[c]), acc[c]);
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) total += (float)acc[c][r];
  }
  out[gid] = total;
}

}  // namespace

hipError_t launch_ceiling_read(const void* buf, int64_t bytes, uint32_t* sink, int blocks, int unroll,
                               hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (unroll == 8)
    hipLaunchKernelGGL(read_stream_kernel<8>, dim3(blocks), dim3(256), 0, stream, (const u32x4*)buf, n16, sink);
  else
    hipLaunchKernelGGL(read_stream_kernel<4>, dim3(blocks), dim3(256), 0, stream, (const u32x4*)buf, n16, sink);
  return hipGetLastError();
}

hipError_t launch_ceiling_mfma(const void* operands, int64_t operand_bytes, int kind, int iters, float* out,
                               int blocks, hipStream_t stream) {
  const int64_t nops = operand_bytes / 16;
  if (kind == 1)
    hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(blocks), dim3(256), 0, stream, (const u32x4*)operands, nops, iters,
                       out);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(blocks), dim3(256), 0, stream, (const u32x4*)operands, nops, iters,
                       out);
  return hipGetLastError();
}

}  // namespace w4
