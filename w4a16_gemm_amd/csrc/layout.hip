// Import of weights quantized elsewhere, given in a plain (untiled) layout, into the
// layout the GEMM kernels read.
//
// "Implement AWQ quantization support for LLaMA" (vllm-project/vllm PR 1032) prints the
// Triton AWQ weight format: codes packed pack_num = 8 per 32-bit word along K, per-group
// scales and per-group zero points packed along the group axis, stored K-major
// (qw (K / 8, N), scales (K / G, N), qzeros (K / G / 8, N)).  Two plain orientations are
// accepted:
//   rows (per output channel): qweight int32 [N, K/8], scales fp16 [N, K/G],
//                              qzeros int32 [N, ceil(K/G / 8)];
//   cols (the printed Triton orientation): qweight int32 [K/8, N], scales fp16 [K/G, N],
//                              qzeros int32 [ceil(K/G / 8), N].
// In both, element k = 8j + i of a row's codes sits in bits 4i..4i+3 of word j and the
// zero point of group g in bits 4 (g % 8).. of word g / 8.  The library keeps the W4A16
// words split by parity (element i in nibble i / 2 + 4 (i % 2)), the W4A8 words split by
// halves (element i in nibble 2 (i % 4) + i / 4), both tiled in 1 KB blocks of 16 rows x
// 128 k, the scales group-major [K/G, N] and the zero points packed
// along N [K/G, ceil(N/8)]; every conversion is a rearrangement of bits (exact).  "[Feature] support qqq(w4a8) for lmdeploy" ("Modification") converts
// exported QQQ weights before its GEMM can load them; here the W4A8 words (biased
// nibbles q + 8) are tiled like the W4A16 ones and the int8 group scales go to [K/G, N].
#include "kernels.hpp"

namespace w4 {

namespace {

// Element (n, i) of a plain array is at in[n * sn + i * si]: rows orientation
// sn = row length, si = 1; cols orientation sn = 1, si = N.
struct Strides {
  int64_t sn, si;
};

// Plain word -> the library's word formats: split by parity (W4A16; element i to nibble
// i / 2 + 4 (i % 2)) or by halves (W4A8; element i to nibble 2 (i % 4) + i / 4).
__device__ __forceinline__ uint32_t split_word(uint32_t w, int split) {
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int to = split == 1 ? (i >> 1) + 4 * (i & 1) : 2 * (i & 3) + (i >> 2);
    o |= ((w >> (4 * i)) & 15u) << (4 * to);
  }
  return o;
}

// One thread per 16-byte chunk of the tiled array, in its order (contiguous stores):
// chunk ((n / 16 * ng + g) * 4 + slot) * 16 + n % 16 holds words 16 g + 4 slot .. + 3 of
// row n.  Rows past N (up to a multiple of 16) hold the pad word.  In the rows
// orientation (si == 1) the four words are one aligned 16-byte load.
__global__ __launch_bounds__(256) void tile_words_kernel(const uint32_t* __restrict__ plain,
                                                         u32x4* __restrict__ tiled, int N, int ng, Strides st,
                                                         uint32_t pad, int split, int64_t total) {
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(c & 15);
    const int64_t blk = c >> 4;  // (n / 16 * ng + g) * 4 + slot
    const int slot = (int)(blk & 3);
    const int64_t tg = blk >> 2;  // n / 16 * ng + g
    const int g = (int)(tg % ng);
    const int64_t n = (tg / ng) * 16 + r;
    const int64_t w0 = (int64_t)g * 16 + slot * 4;
    u32x4 v = {pad, pad, pad, pad};
    if (n < N) {
      const uint32_t* src = plain + n * st.sn + w0 * st.si;
      if (st.si == 1) {
        v = *reinterpret_cast<const u32x4*>(src);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = src[i * st.si];
      }
      if (split) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = split_word(v[i], split);
      }
    }
    tiled[c] = v;
  }
}

// Per-group values (fp16 scales, int8 group scales) to [ng, N]: one thread per output
// element (contiguous stores).
template <typename E>
__global__ __launch_bounds__(256) void groups_to_gn_kernel(const E* __restrict__ in, E* __restrict__ out, int N,
                                                           Strides st, int64_t total) {
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total; o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t g = o / N, n = o - g * N;
    out[o] = in[n * st.sn + g * st.si];
  }
}

// Zero points packed along groups (word g / 8 of row n) -> packed along N
// [ng, ceil(N / 8)]: one thread per output word (8 rows of one group); pad nibbles (rows
// past N) are 0.
__global__ __launch_bounds__(256) void repack_zeros_kernel(const uint32_t* __restrict__ in, uint32_t* __restrict__ out,
                                                           int N, Strides st, int64_t total) {
  const int nzw_out = (N + 7) / 8;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total; o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t g = o / nzw_out;
    const int j = (int)(o - g * nzw_out);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t n = 8 * (int64_t)j + i;
      if (n < N) word |= ((in[n * st.sn + (g >> 3) * st.si] >> (4 * (g & 7))) & 15u) << (4 * i);
    }
    out[o] = word;
  }
}

inline unsigned grid_for(int64_t total) {
  const int64_t b = (total + 255) / 256;
  return (unsigned)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

}  // namespace

hipError_t launch_import_plain(const int32_t* qweight_plain, const void* scales_plain, const int32_t* qzeros_plain,
                               const int8_t* gscale_plain, int32_t* qweight, void* scales, int32_t* qzeros,
                               int8_t* gscale, int N, int K, int ng, int cols, uint32_t pad, int split,
                               hipStream_t stream) {
  const int64_t chunks = (int64_t)((N + 15) / 16) * (K / 128) * 64;
  const Strides sw = cols ? Strides{1, N} : Strides{K / 8, 1};
  hipLaunchKernelGGL(tile_words_kernel, dim3(grid_for(chunks)), dim3(256), 0, stream, (const uint32_t*)qweight_plain,
                     (u32x4*)qweight, N, K / 128, sw, pad, split, chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t vals = (int64_t)N * ng;
  const Strides sg = cols ? Strides{1, N} : Strides{ng, 1};
  if (scales_plain) {
    hipLaunchKernelGGL(groups_to_gn_kernel<uint16_t>, dim3(grid_for(vals)), dim3(256), 0, stream,
                       (const uint16_t*)scales_plain, (uint16_t*)scales, N, sg, vals);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (gscale_plain) {
    hipLaunchKernelGGL(groups_to_gn_kernel<int8_t>, dim3(grid_for(vals)), dim3(256), 0, stream, gscale_plain, gscale,
                       N, sg, vals);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (qzeros_plain) {
    const int64_t words = (int64_t)ng * ((N + 7) / 8);
    const Strides sz = cols ? Strides{1, N} : Strides{(ng + 7) / 8, 1};
    hipLaunchKernelGGL(repack_zeros_kernel, dim3(grid_for(words)), dim3(256), 0, stream,
                       (const uint32_t*)qzeros_plain, (uint32_t*)qzeros, N, sz, words);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace w4
