// Weight quantization and packing kernels (offline-style, one pass over W).
//
//  * awq_pack: asymmetric 4-bit group quantization ("Some fixes for AWQ",
//    neuralmagic/compressed-tensors PR 269, opening comment: the asymmetric rule of
//    AutoAWQ's pseudo-quantize) and packing 8 codes per 32-bit word (packed weight
//    format of the Triton AWQ kernels in "Implement AWQ quantization support for
//    LLaMA", vllm-project/vllm PR 1032: pack_num = 8), each word split by parity
//    (elements 0, 2, 4, 6 in nibbles 0..3, elements 1, 3, 5, 7 in nibbles 4..7: the
//    order the GEMMs expand in one shift and four v_and_or_b32), in the tiled layout.
//    The zero points keep the plain nibble order (element i in nibble i).
//    Per-channel weights (group_size -1: one group over K, a reading of the
//    per-channel variant named on "[Feature] support qqq(w4a8) for lmdeploy") take
//    their row statistics from awq_rowstats first.  Symmetric weights (the W4A16
//    preset beside W4A16_ASYM in the same compressed-tensors thread, read with the
//    W4A8 per-channel constants) use s = fp16(max(max|w| / 7, 1e-5)) and the fixed zero
//    point 8, so code = clamp(rint(w / s) + 8, 0, 15) = clamp(rint(w / s), -8, 7) + 8 is
//    the asymmetric code formula with z = 8.
//  * awq_unpack_dequant: fp16((q - z) * s), the GEMM's dequantization, exported.
//  * w4a8_pack: symmetric int4 weights for the W4A8 GEMM, per-channel or two-level
//    with int8 group scales ("[Feature] support qqq(w4a8) for lmdeploy", section
//    "Benchmark": QQQ per-channel and QQQ-g128 variants), as biased nibbles q + 8 in
//    words split by halves (elements 0..3 in the even nibbles, 4..7 in the odd ones: the
//    order the int8 expansion takes without byte permutations).
//  * w8a8_pack: per-channel symmetric int8 weights for W8A8 (the 8-bit-weight method
//    mentioned on the vLLM AWQ page, and W8A8 as named on the compressed-tensors
//    page; constants as the first level of the two-level W4A8 rule):
//    s = fp16(max(max|w| / 127, 1e-5)), q = clamp(rint(w / s), -127, 127), stored in
//    the tiled int8 layout (tiled8_offset); padding rows hold 0.
//
// Every quantization decision is made in fp32 with IEEE division and
// round-half-to-even (rintf), and there is no a*b+c in these expressions, so the
// codes are bit-reproducible.
#include "kernels.hpp"

namespace w4 {

// Scale and zero point of one group (or row) from its statistics: asymmetric
// s = fp16(max((max - min) / 15, 1e-5)), z = clamp(rint(-min / s), 0, 15); symmetric
// s = fp16(max(max(|min|, |max|) / 7, 1e-5)), z = 8.
__device__ __forceinline__ void group_scale_zero(float mn, float mx, int sym, half_t& s16, float& z) {
  if (sym) {
    s16 = (half_t)fmaxf(fmaxf(-mn, mx) / 7.0f, 1e-5f);
    z = 8.0f;
  } else {
    s16 = (half_t)fmaxf((mx - mn) / 15.0f, 1e-5f);
    z = fminf(fmaxf(rintf(-mn / (float)s16), 0.0f), 15.0f);
  }
}

// Per-channel statistics: one workgroup per 8 rows, one wave per 2 rows; min and max of
// each row over K give its scale (scales[n]) and zero point (the 8 nibbles of
// qzeros[n / 8]).
__global__ __launch_bounds__(256) void awq_rowstats_kernel(const half_t* __restrict__ w, half_t* __restrict__ scales,
                                                            int32_t* __restrict__ qzeros, int N, int K, int sym) {
  __shared__ uint32_t znib[8];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * 8;
  for (int rr = 0; rr < 2; ++rr) {
    const int i = wave * 2 + rr;
    const int n = n0 + i;
    uint32_t zb = 0;
    if (n < N) {
      const half8_t* row = reinterpret_cast<const half8_t*>(w + (int64_t)n * K);
      float mn = INFINITY, mx = -INFINITY;
      for (int j = lane; j < K / 8; j += kWave) {
        const half8_t v = row[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          mn = fminf(mn, (float)v[e]);
          mx = fmaxf(mx, (float)v[e]);
        }
      }
      mn = -wave_max(-mn);
      mx = wave_max(mx);
      half_t s16;
      float z;
      group_scale_zero(mn, mx, sym, s16, z);
      if (lane == 0) scales[n] = s16;
      zb = ((uint32_t)z) << (4 * i);
    }
    if (lane == 0) znib[i] = zb;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= znib[i];
    qzeros[n0 / 8] = (int32_t)word;
  }
}

// One thread per (128-k unit g, row n), n fastest, over npad = N rounded up to 16 rows:
// the 8 threads of a zero-point word are 8 consecutive lanes, and padding rows
// (n >= N) write code 0 so that the whole tiled array is defined.  The unit holds SUB
// groups of 128 / SUB k (group sizes 128, 64, 32).  Per-channel (perchan = 1, SUB = 1):
// scale and zero point come from awq_rowstats and are not rewritten.
template <int SUB>
__global__ __launch_bounds__(256) void awq_pack_kernel(const half_t* __restrict__ w,
                                                        uint32_t* __restrict__ qweight,
                                                        half_t* __restrict__ scales,
                                                        int32_t* __restrict__ qzeros,
                                                        int N, int K, int npad, int perchan, int sym) {
  constexpr int GS = 128 / SUB;
  const int ng = K / 128;
  const int nzw = (N + 7) / 8;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = tid < (int64_t)npad * ng;
  const int g = live ? (int)(tid / npad) : 0;
  const int n = live ? (int)(tid % npad) : 0;
  const bool valid = live && n < N;
  uint32_t zbits[SUB];
#pragma unroll
  for (int u = 0; u < SUB; ++u) zbits[u] = 0;
  u32x4 out[4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  if (valid) {
    const u32x4* src = reinterpret_cast<const u32x4*>(w + (int64_t)n * K + (int64_t)g * 128);
    u32x4 raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) raw[i] = src[i];
    const half_t* h = reinterpret_cast<const half_t*>(raw);
    half_t s16[SUB];
    float z[SUB];
    if (perchan) {
      s16[0] = scales[n];
      z[0] = (float)((((uint32_t)qzeros[n / 8]) >> (4 * (n & 7))) & 15u);
    } else {
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        float mn = (float)h[u * GS], mx = (float)h[u * GS];
#pragma unroll
        for (int i = 1; i < GS; ++i) {
          const float v = (float)h[u * GS + i];
          mn = fminf(mn, v);
          mx = fmaxf(mx, v);
        }
        group_scale_zero(mn, mx, sym, s16[u], z[u]);
      }
    }
    uint32_t* ow = reinterpret_cast<uint32_t*>(out);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int u = (8 * j) / GS;
      const float s = (float)s16[u];
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q = fminf(fmaxf(rintf((float)h[8 * j + i] / s) + z[u], 0.0f), 15.0f);
        word |= ((uint32_t)q) << (4 * ((i >> 1) + 4 * (i & 1)));  // parity-split word
      }
      ow[j] = word;
    }
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      if (!perchan) scales[((int64_t)g * SUB + u) * N + n] = s16[u];
      zbits[u] = ((uint32_t)z[u]) << (4 * (n & 7));
    }
  }
  if (live) {
#pragma unroll
    for (int slot = 0; slot < 4; ++slot) *reinterpret_cast<u32x4*>(qweight + tiled_chunk(n, g, slot, ng)) = out[slot];
  }
  // OR the 8 nibbles of each zero-point word across the 8 consecutive lanes.
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    uint32_t zb = zbits[u];
    zb |= __shfl_xor(zb, 1, kWave);
    zb |= __shfl_xor(zb, 2, kWave);
    zb |= __shfl_xor(zb, 4, kWave);
    if (!perchan && valid && (n & 7) == 0) qzeros[((int64_t)g * SUB + u) * nzw + n / 8] = (int32_t)zb;
  }
}

// One thread per packed word (n, j): eight fp16 outputs.
__global__ __launch_bounds__(256) void awq_unpack_dequant_kernel(const uint32_t* __restrict__ qweight,
                                                                  const half_t* __restrict__ scales,
                                                                  const uint32_t* __restrict__ qzeros,
                                                                  half_t* __restrict__ out, int N, int K,
                                                                  int glog) {
  const int wpr = K / 8;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= (int64_t)N * wpr) return;
  const int n = (int)(tid / wpr);
  const int j = (int)(tid % wpr);
  const int g = j / 16;
  const int nzw = (N + 7) / 8;
  const int64_t row = (8 * j) >> glog;
  const uint32_t z = (qzeros[row * nzw + n / 8] >> (4 * (n & 7))) & 15u;
  const uint16_t sb = reinterpret_cast<const uint16_t*>(scales)[row * N + n];
  const uint32_t word = qweight[tiled_chunk(n, g, (j & 15) >> 2, K / 128) + (j & 3)];
  const half8_t v = dequant8(word, magic_regs(), neg1024z2(z), neg64z2(z), scale2(sb));
  *reinterpret_cast<half8_t*>(out + (int64_t)n * K + (int64_t)j * 8) = v;
}

// One workgroup (256 threads) per row n.  Pass 1: amax over the row.  Pass 2: codes.
// Two-level mode: a group of 128 k is 16 words handled by 16 consecutive lanes.
// Workgroups past N (up to N rounded to 16) write padding rows of q = 0 (word 0x88888888).
__global__ __launch_bounds__(256) void w4a8_pack_kernel(const half_t* __restrict__ w,
                                                         uint32_t* __restrict__ qweight,
                                                         int8_t* __restrict__ gscale,
                                                         half_t* __restrict__ cscale,
                                                         int N, int K, int two_level) {
  __shared__ float red[4];
  const int n = blockIdx.x;
  const int ng = K / 128;
  if (n >= N) {
    for (int j = threadIdx.x; j < K / 8; j += 256)
      qweight[tiled_chunk(n, j / 16, (j & 15) >> 2, ng) + (j & 3)] = 0x88888888u;
    return;
  }
  const half_t* row = w + (int64_t)n * K;
  const int wpr = K / 8;
  float amax = 0.0f;
  for (int j = threadIdx.x; j < wpr; j += 256) {
    const half8_t v = *reinterpret_cast<const half8_t*>(row + 8 * j);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)v[i]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s32 = fmaxf(amax / (two_level ? 127.0f : 7.0f), 1e-5f);
  const half_t s16 = (half_t)s32;
  const float s = (float)s16;
  if (threadIdx.x == 0) cscale[n] = s16;
  // wpr is a multiple of 16 (K multiple of 128) in two-level mode, and 256 is a multiple
  // of 16, so every 16-lane segment holds exactly one group.
  const int jmax = (wpr + 255) / 256 * 256;
  for (int j = threadIdx.x; j < jmax; j += 256) {
    const bool ok = j < wpr;
    float e[8];
    if (ok) {
      const half8_t v = *reinterpret_cast<const half8_t*>(row + 8 * j);
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = (float)v[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = 0.0f;
    }
    uint32_t word = 0;
    if (!two_level) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q = fminf(fmaxf(rintf(e[i] / s), -8.0f), 7.0f);
        word |= ((uint32_t)((int)q + 8)) << (4 * (2 * (i & 3) + (i >> 2)));  // split by halves
      }
    } else {
      float w8[8];
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w8[i] = fminf(fmaxf(rintf(e[i] / s), -127.0f), 127.0f);
        m = fmaxf(m, fabsf(w8[i]));
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
      const float sg = fminf(fmaxf(1.0f, ceilf(m / 7.0f)), 18.0f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q = fminf(fmaxf(rintf(w8[i] / sg), -7.0f), 7.0f);
        word |= ((uint32_t)((int)q + 8)) << (4 * (2 * (i & 3) + (i >> 2)));
      }
      if (ok && (j & 15) == 0) gscale[(int64_t)(j / 16) * N + n] = (int8_t)(int)sg;
    }
    if (ok) qweight[tiled_chunk(n, j / 16, (j & 15) >> 2, ng) + (j & 3)] = word;
  }
}

// One thread per output word (row r, word j): eight bytes of codes -> one word.
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes, uint32_t* __restrict__ out,
                                                          int64_t R, int64_t C) {
  const int64_t W = (C + 7) / 8;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= R * W) return;
  const int64_t r = tid / W, j = tid - r * W;
  const uint8_t* src = codes + r * C + j * 8;
  const int n = (int)min<int64_t>(8, C - j * 8);
  uint32_t word = 0;
  for (int i = 0; i < n; ++i) word |= ((uint32_t)src[i] & 15u) << (4 * i);
  out[tid] = word;
}

hipError_t launch_pack_codes(const uint8_t* codes, int32_t* out, int64_t R, int64_t C, hipStream_t stream) {
  const int64_t total = R * ((C + 7) / 8);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, (uint32_t*)out, R, C);
  return hipGetLastError();
}

hipError_t launch_awq_pack(const void* w, int32_t* qweight, void* scales, int32_t* qzeros, int N, int K,
                           int group_size, bool symmetric, hipStream_t stream) {
  const int perchan = group_size == -1 ? 1 : 0;
  if (perchan) {
    hipLaunchKernelGGL(awq_rowstats_kernel, dim3((N + 7) / 8), dim3(256), 0, stream, (const half_t*)w,
                       (half_t*)scales, qzeros, N, K, symmetric ? 1 : 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int npad = (N + 15) / 16 * 16;
  const int64_t total = (int64_t)npad * (K / 128);
  const int blocks = (int)((total + 255) / 256);
#define W4_AWQ_PACK(SUB)                                                                                   \
  hipLaunchKernelGGL(awq_pack_kernel<SUB>, dim3(blocks), dim3(256), 0, stream, (const half_t*)w,            \
                     (uint32_t*)qweight, (half_t*)scales, qzeros, N, K, npad, perchan, symmetric ? 1 : 0)
  if (group_size == 32) W4_AWQ_PACK(4);
  else if (group_size == 64) W4_AWQ_PACK(2);
  else W4_AWQ_PACK(1);
#undef W4_AWQ_PACK
  return hipGetLastError();
}

hipError_t launch_awq_unpack_dequant(const int32_t* qweight, const void* scales, const int32_t* qzeros,
                                     void* out, int N, int K, int group_size, hipStream_t stream) {
  const int64_t total = (int64_t)N * (K / 8);
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(awq_unpack_dequant_kernel, dim3(blocks), dim3(256), 0, stream,
                     (const uint32_t*)qweight, (const half_t*)scales, (const uint32_t*)qzeros,
                     (half_t*)out, N, K, group_log2(group_size));
  return hipGetLastError();
}

// One workgroup (256 threads) per row: amax over the row, then the codes, 8 per store
// (half of a 16-byte chunk).  Workgroups past N (up to N rounded to 16) write the
// padding rows' zeros.
__global__ __launch_bounds__(256) void w8a8_pack_kernel(const half_t* __restrict__ w, int8_t* __restrict__ qweight,
                                                         half_t* __restrict__ cscale, int N, int K) {
  __shared__ float red[4];
  const int n = blockIdx.x;
  const int ng = K / 128;
  const int nv = K / 8;
  auto dst = [&](int j) {  // 8-byte half j & 1 of chunk j / 2 of row n
    return reinterpret_cast<uint64_t*>(qweight + tiled8_offset(n, j >> 4, (j >> 1) & 7, ng) + (j & 1) * 8);
  };
  if (n >= N) {
    for (int j = threadIdx.x; j < nv; j += 256) *dst(j) = 0;
    return;
  }
  const half8_t* row = reinterpret_cast<const half8_t*>(w + (int64_t)n * K);
  float amax = 0.0f;
  for (int j = threadIdx.x; j < nv; j += 256) {
    const half8_t v = row[j];
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)v[i]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const half_t s16 = (half_t)fmaxf(amax / 127.0f, 1e-5f);
  const float s = (float)s16;
  if (threadIdx.x == 0) cscale[n] = s16;
  for (int j = threadIdx.x; j < nv; j += 256) {
    const half8_t v = row[j];
    uint64_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = fminf(fmaxf(rintf((float)v[i] / s), -127.0f), 127.0f);
      packed |= (uint64_t)(uint8_t)(int8_t)(int)q << (8 * i);
    }
    *dst(j) = packed;
  }
}

hipError_t launch_w8a8_pack(const void* w, int8_t* qweight, void* cscale, int N, int K, hipStream_t stream) {
  hipLaunchKernelGGL(w8a8_pack_kernel, dim3((N + 15) / 16 * 16), dim3(256), 0, stream, (const half_t*)w, qweight,
                     (half_t*)cscale, N, K);
  return hipGetLastError();
}

hipError_t launch_w4a8_pack(const void* w, int32_t* qweight, int8_t* gscale, void* cscale, int N, int K,
                            int two_level, hipStream_t stream) {
  hipLaunchKernelGGL(w4a8_pack_kernel, dim3((N + 15) / 16 * 16), dim3(256), 0, stream, (const half_t*)w,
                     (uint32_t*)qweight, gscale, (half_t*)cscale, N, K, two_level);
  return hipGetLastError();
}

}  // namespace w4
