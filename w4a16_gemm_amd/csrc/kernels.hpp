// Launchers implemented by the .hip translation units and called by the C ABI.
#pragma once

#include "common.hpp"

namespace w4 {

// Split-K arrival.  Every block of a tile stores its fp32 partial sums, then calls
// this; it returns true in exactly one block (the last to arrive), which then sums
// the partials in split order (deterministic) and writes the result.  The last block
// resets the counter to 0, so a zero-filled counter region stays zero across calls.
__device__ __forceinline__ bool splitk_arrive(unsigned* counter, int splits) {
  __shared__ int is_last;
  __threadfence();  // release: this thread's partial stores are visible device-wide
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = atomicAdd(counter, 1u);
    is_last = (old == (unsigned)(splits - 1));
    if (is_last) atomicExch(counter, 0u);
  }
  __syncthreads();
  const bool last = is_last != 0;
  if (last) __threadfence();  // acquire: see the other blocks' partials
  return last;
}

// Tile plan of the skinny (M <= 64) W4A16 kernel.
struct SkinnyPlan {
  int mt;          // 16-row M tiles (1, 2 or 4)
  int row_blocks;  // ceil(N / 64)
  int splits;      // split-K factor over groups
  int gps;         // groups per split
};
SkinnyPlan skinny_plan(int M, int N, int K);

// Tile plan of the large-M W4A16 GEMM.
struct GemmPlan {
  int tiles_m, tiles_n, splits, kt_per_split;
};
GemmPlan gemm_plan(int M, int N, int K);

struct W4A8Plan {
  int tiles_m, tiles_n, splits, kt_per_split, bm;
};
W4A8Plan w4a8_plan(int M, int N, int K, int group_size);

constexpr size_t kCounterBytesAlign = 256;

hipError_t launch_awq_pack(const void* w, int32_t* qweight, void* scales, int32_t* qzeros, int N, int K,
                           hipStream_t stream);
hipError_t launch_awq_unpack_dequant(const int32_t* qweight, const void* scales, const int32_t* qzeros,
                                     void* out, int N, int K, hipStream_t stream);
hipError_t launch_w4a8_pack(const void* w, int32_t* qweight, int8_t* gscale, void* cscale, int N, int K,
                            int two_level, hipStream_t stream);

size_t skinny_workspace_bytes(int M, int N, int K);
hipError_t launch_skinny(const void* x, const int32_t* qweight, const void* scales, const int32_t* qzeros,
                         void* y, void* ws, int M, int N, int K, hipStream_t stream);

size_t gemm_workspace_bytes(int M, int N, int K);
hipError_t launch_gemm(const void* x, const int32_t* qweight, const void* scales, const int32_t* qzeros,
                       void* y, void* ws, int M, int N, int K, hipStream_t stream);

hipError_t launch_w4a8_quant_act(const void* x, const void* gamma, float eps, int8_t* xq, float* s_a, int M,
                                 int K, hipStream_t stream);

size_t w4a8_workspace_bytes(int M, int N, int K, int group_size);
hipError_t launch_w4a8_gemm(const int8_t* xq, const float* s_a, const int32_t* qweight, const int8_t* gscale,
                            const void* cscale, void* y, int32_t* acc_out, void* ws, int M, int N, int K,
                            int group_size, hipStream_t stream);

}  // namespace w4
