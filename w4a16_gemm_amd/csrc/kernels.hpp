// Launchers implemented by the .hip translation units and called by the C ABI.
#pragma once

#include "common.hpp"

namespace w4 {

// Split-K across workgroups.  Every block of a tile writes its partial sums with
// agent-scope relaxed atomic stores, waits for them to complete, and bumps the tile's
// arrival counter; the block that arrives last reads all partials (agent-scope loads)
// in split order -- deterministic -- and writes the result.  Agent-scope stores and
// loads are coherent across the XCDs' L2 caches on their own (the compiler marks them
// for the coherence point), so no whole-cache writeback or invalidate is needed; the
// counter RMW is performed at the coherence point.  The last block resets the counter
// to 0, so a zero-filled counter region stays zero across calls.
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_coherent(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool splitk_arrive(unsigned* counter, int splits) {
  __shared__ int is_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (old == (unsigned)(splits - 1));
    if (is_last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return is_last != 0;
}

// Workspace layout: a fixed region of kMaxCounters uint32 arrival counters at offset 0
// (zero-filled by the caller once; never used for anything else, so reusing one
// workspace for different shapes is safe), then the partial sums.  Plans only split K
// when the number of tiles is below kMaxCounters.
constexpr int kMaxCounters = 4096;
constexpr size_t kCounterRegionBytes = kMaxCounters * sizeof(unsigned);

// Size of the static device workspace of awq_gemm_noalloc (W4_NOALLOC_SCRATCH_BYTES).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// Device address of that workspace on the current GPU (resolved once per device; the
// first call also enqueues the clearing of its counter region on `stream`).
hipError_t noalloc_scratch(void** ptr, hipStream_t stream);

// Host-side tuning knob for sweeps and the variant tests.  Only when the environment
// holds W4_TUNING=1 at the library's first plan does the integer variable `name`
// override `dflt`; otherwise every plan takes its built-in defaults and reads no
// environment variable.
int env_int(const char* name, int dflt);

// Tile plan of the skinny (M <= 32) W4A16 kernel.
struct SkinnyPlan {
  int mt;          // 16-row M tiles (1 or 2)
  int tiles;       // 16-column tiles per workgroup (1, 2, 4; register-X kernel also 8)
  int depth;       // groups in flight per wave (register sets)
  int row_blocks;  // ceil(N / (16 tiles))
  int splits;      // split-K factor over groups
  int gps;         // groups per split
  int lds;         // 1: the kernel with X staged in LDS (M <= 16, mt == 1)
  int wn, wk;      // LDS kernel: waves per workgroup = wn column groups x wk K-waves
  int smem;        // LDS kernel: dynamic LDS bytes per workgroup
  int drain;       // 1: wait for all loads in flight once per D groups
  int waves;       // register-X kernel: waves per workgroup (4 or 8)
  int xs;          // register-X kernel, mt == 1: X loaded as whole rows (ceil(M / 4) loads per group), fragments formed in LDS
};
SkinnyPlan skinny_plan(int M, int N, int K, int group_size);

// Tile plan of the large-M W4A16 GEMM.
struct GemmPlan {
  int mi, nf;  // tile = (32 mi) x (128 nf)
  int tiles_m, tiles_n, splits, kt_per_split;
  int n_full, tail_splits;  // tail split: tiles >= n_full are split tail_splits ways (0: off)
  int depth;                // BK steps of loads in flight (register sets)
};
GemmPlan gemm_plan(int M, int N, int K);

struct W4A8Plan {
  int tiles_m, tiles_n, splits, kt_per_split, bm;
  int skinny, tiles;        // M <= 16 skinny kernel and its 16-column tiles per workgroup
  int n_full, tail_splits;  // tail split of the tiled GEMM (0: off)
  int depth;                // tiled GEMM: groups of loads in flight (register sets)
};
W4A8Plan w4a8_plan(int M, int N, int K, int group_size);

// W4A16 scales and zero points: every kernel reads the row of element k as
// k >> group_log2 (30 for per-channel: every k < 2^30 maps to row 0).
inline int group_log2(int group_size) {
  return group_size == 32 ? 5 : group_size == 64 ? 6 : group_size == 128 ? 7 : 30;
}

hipError_t launch_awq_pack(const void* w, int32_t* qweight, void* scales, int32_t* qzeros, int N, int K,
                           int group_size, bool symmetric, hipStream_t stream);
hipError_t launch_pack_codes(const uint8_t* codes, int32_t* out, int64_t R, int64_t C, hipStream_t stream);
hipError_t launch_awq_unpack_dequant(const int32_t* qweight, const void* scales, const int32_t* qzeros,
                                     void* out, int N, int K, int group_size, hipStream_t stream);
hipError_t launch_w4a8_pack(const void* w, int32_t* qweight, int8_t* gscale, void* cscale, int N, int K,
                            int two_level, hipStream_t stream);
// Measured ceilings: an HBM read stream and an MFMA issue loop (see ceilings.hip).
hipError_t launch_ceiling_read(const void* buf, int64_t bytes, uint32_t* sink, int blocks, int unroll,
                               hipStream_t stream);
hipError_t launch_ceiling_mfma(const void* operands, int64_t operand_bytes, int kind, int iters, float* out,
                               int blocks, hipStream_t stream);
// Plain (untiled) weights -> the library's layout; NULL sources skip that array.
// cols: the K-major orientation (qweight [K/8, N], per-group arrays [., N]); split: the
// word format each plain code word is converted to (1: split by parity, the W4A16 words;
// 2: split by halves, the W4A8 words).
hipError_t launch_import_plain(const int32_t* qweight_plain, const void* scales_plain, const int32_t* qzeros_plain,
                               const int8_t* gscale_plain, int32_t* qweight, void* scales, int32_t* qzeros,
                               int8_t* gscale, int N, int K, int ng, int cols, uint32_t pad, int split,
                               hipStream_t stream);

// Every GEMM entry point plans once per call: the plan sizes the workspace and is then
// handed to the launcher.
size_t skinny_workspace_bytes(const SkinnyPlan& p, int M, int N);
hipError_t launch_skinny(const SkinnyPlan& p, const void* x, const int32_t* qweight, const void* scales,
                         const int32_t* qzeros, void* y, void* ws, int M, int N, int K, int group_size,
                         hipStream_t stream);

size_t gemm_workspace_bytes(const GemmPlan& p, int M, int N);
hipError_t launch_gemm(const GemmPlan& p, const void* x, const int32_t* qweight, const void* scales,
                       const int32_t* qzeros, void* y, void* ws, int M, int N, int K, int group_size,
                       hipStream_t stream);

hipError_t launch_w4a8_quant_act(const void* x, const void* gamma, float eps, int8_t* xq, float* s_a, int M,
                                 int K, hipStream_t stream);
hipError_t launch_w4a8_silu_mul_quant(const void* gate_up, int8_t* xq, float* s_a, int M, int I,
                                      hipStream_t stream);

size_t w4a8_workspace_bytes(const W4A8Plan& p, int M, int N);
hipError_t launch_w4a8_gemm(const W4A8Plan& p, const int8_t* xq, const float* s_a, const int32_t* qweight, const int8_t* gscale,
                            const void* cscale, void* y, int32_t* acc_out, void* ws, int M, int N, int K,
                            int group_size, hipStream_t stream);
// Byte offset of the 16-byte chunk kc (k = 128 g + 16 kc .. + 15) of row n in the tiled
// W8A8 weights int8 [ceil(N/16), K/128, 4, 2, 16, 16]: 2 KB per 16 rows x 128 k, chunk
// (kc % 4, kc / 4) of the 16 rows stored together.
__device__ __forceinline__ int64_t tiled8_offset(int n, int g, int kc, int ng) {
  return (((int64_t)(n >> 4) * ng + g) * 4 + (kc & 3)) * 512 + (kc >> 2) * 256 + (n & 15) * 16;
}

// W8A8: tiled int8 weights with per-channel scales, on the W4A8 kernels.
hipError_t launch_w8a8_gemm(const W4A8Plan& p, const int8_t* xq, const float* s_a, const int8_t* qweight, const void* cscale, void* y,
                            int32_t* acc_out, void* ws, int M, int N, int K, hipStream_t stream);
hipError_t launch_w8a8_pack(const void* w, int8_t* qweight, void* cscale, int N, int K, hipStream_t stream);

}  // namespace w4
