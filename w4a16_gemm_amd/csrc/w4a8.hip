// W4A8 stage: online per-token int8 activation quantization fused with RMSNorm, and
// the int8 x int4 GEMM on the int8 MFMA units with exact int32 accumulation.
//
// "[Feature] support qqq(w4a8) for lmdeploy" (InternLM/lmdeploy issue 2274), section
// "Modification": a W4A8 GEMM kernel; online activation quantization fused with
// element-wise ops such as RMSNorm; section "Benchmark": per-channel and g128 weight
// variants.  "Some fixes for AWQ" (neuralmagic/compressed-tensors PR 269), reply on
// 8-bit matmuls: the int8 product accumulates to int32 and is rescaled by the weight
// and activation scales; activations are quantized dynamically per token.
//
// Weight codes are stored as biased nibbles b = q + 8, each word split by halves
// (elements 0..3 in the even nibbles, 4..7 in the odd ones), so that the int8 bytes of
// a word come out in natural k order without byte permutations.
//   per-channel:  b ^ 8 is the 4-bit two's complement of q; shifted into the high
//                 nibble of a byte it is the int8 value 16 q, so the MFMA accumulates
//                 16 * sum(xq * q) exactly and an exact arithmetic shift by 4 (every
//                 term is a multiple of 16) gives acc = sum_k xq * q.
//   two-level:    each code is expanded per group to the int8 value q * s_g (formed in
//                 16-bit lanes, |q s_g| <= 126), so the MFMA accumulates
//                 acc = sum_k xq * q * s_g directly.
// Both are the exact integer sum_k xq[m,k] * q[n,k] * s_g[n,k/G] (s_g = 1 per-channel).
#include "kernels.hpp"

namespace w4 {

namespace {

// ------------------------------------------------------------ row kernels
// quant_act and silu_mul_quant: one workgroup of T threads per token row.  With R > 0
// the row fits in registers (R vectors of 8 per thread, T * R * 8 >= K): every load is
// issued up front (clamped indexes, so all are in bounds and none waits on a branch), y
// is formed once and kept for the code pass, and each input byte is read once.  R = 0
// streams longer rows through L2 again for each pass.
//
// Codes: t = y * fp32(127 / amax) is rounded to the nearest integer (ties to even) by
// adding 1.5 * 2^23, whose low byte is then the two's complement code; |y| <= amax gives
// |t| <= 127 (1 + 2^-23) < 127.5, so no clamp is needed.

// Row kernels loop over rows; at most 2^20 workgroups are launched.
inline unsigned row_grid(int M) { return (unsigned)(M < (1 << 20) ? M : (1 << 20)); }

template <int T>
__device__ __forceinline__ float block_sum_t(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int w = 1; w < T / 64; ++w) s += red[w];
  return s;
}

template <int T>
__device__ __forceinline__ float block_max_t(float v, float* red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < T / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

// Low byte of rint(t) + 1.5 * 2^23 for four values, packed into one word.  t = y * inv
// is rounded to fp32 before the add (no fma contraction: a single rounding of
// y * inv + 1.5 * 2^23 would differ from rint(fp32(t)) next to half-integers).
__device__ __forceinline__ uint32_t pack_codes4(const float* y, float inv) {
#pragma clang fp contract(off)
  uint32_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = __float_as_uint(y[i] * inv + 12582912.0f);
  return __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
}

__device__ __forceinline__ uint2 pack_codes8(const float* y, float inv) {
  return make_uint2(pack_codes4(y, inv), pack_codes4(y + 4, inv));
}

// Launch a row kernel template K<T, R> for rows of nv vectors of 8 (R8_1024: whether
// K<1024, 8> fits the 128 VGPRs of a 1024-thread workgroup; else such rows stream).
// Rows of 513..640 vectors (K = 5120) take two waves of five vectors per thread: the
// block reductions then span two waves (RMSNorm quant_act at M = 4096: 17.6 -> 15.1 us).
#define W4_ROW_DISPATCH(KERNEL, R8_1024, nv, grid, stream, ...)                                      \
  do {                                                                                               \
    if ((nv) <= 256) hipLaunchKernelGGL((KERNEL<256, 1>), grid, dim3(256), 0, stream, __VA_ARGS__);   \
    else if ((nv) <= 512) hipLaunchKernelGGL((KERNEL<256, 2>), grid, dim3(256), 0, stream, __VA_ARGS__); \
    else if ((nv) <= 640 && env_int("W4_ROW_T128", 1)) hipLaunchKernelGGL((KERNEL<128, 5>), grid, dim3(128), 0, stream, __VA_ARGS__); \
    else if ((nv) <= 1024) hipLaunchKernelGGL((KERNEL<256, 4>), grid, dim3(256), 0, stream, __VA_ARGS__); \
    else if ((nv) <= 2048) hipLaunchKernelGGL((KERNEL<256, 8>), grid, dim3(256), 0, stream, __VA_ARGS__); \
    else if ((nv) <= 4096) hipLaunchKernelGGL((KERNEL<1024, 4>), grid, dim3(1024), 0, stream, __VA_ARGS__); \
    else if ((R8_1024) && (nv) <= 8192)                                                            \
      hipLaunchKernelGGL((KERNEL<1024, R8_1024 ? 8 : 0>), grid, dim3(1024), 0, stream, __VA_ARGS__);  \
    else hipLaunchKernelGGL((KERNEL<1024, 0>), grid, dim3(1024), 0, stream, __VA_ARGS__);            \
  } while (0)

// ------------------------------------------------------------ quant_act
// y = (x * r) * gamma in fp32 with r = 1 / sqrt(sum(x^2) / K + eps) (RMSNorm), or y = x
// without gamma; then amax = max|y|, codes as above, s_a = amax / 127; a zero row gives
// codes 0 and s_a = 1.  Without gamma every step is exact or one fp32 rounding in the
// order of the definition, so the codes are bit-exact.
template <int T, int R>
__global__ __launch_bounds__(T) void quant_act_kernel(const half_t* __restrict__ x, const half_t* __restrict__ gamma,
                                                       float eps, int8_t* __restrict__ xq, float* __restrict__ s_a,
                                                       int M, int K) {
  __shared__ float red[T / 64];
  const int nv = K / 8;
  const half8_t* gr = reinterpret_cast<const half8_t*>(gamma);
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    const half8_t* xr = reinterpret_cast<const half8_t*>(x + row * K);
    uint2* dst = reinterpret_cast<uint2*>(xq + row * K);
    float amax = 0.0f;
    if constexpr (R > 0) {
      half8_t xv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) xv[r] = __builtin_nontemporal_load(xr + min((int)threadIdx.x + r * T, nv - 1));
      float y[R][8];
      if (gamma) {
        half8_t gv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) gv[r] = gr[min((int)threadIdx.x + r * T, nv - 1)];
        float ss = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if ((int)threadIdx.x + r * T < nv) {
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf((float)xv[r][i], (float)xv[r][i], ss);
          }
        }
        ss = block_sum_t<T>(ss, red);
        const float rs = 1.0f / sqrtf(ss / (float)K + eps);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i) y[r][i] = ((float)xv[r][i] * rs) * (float)gv[r][i];
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i) y[r][i] = (float)xv[r][i];
      }
      // clamped duplicates repeat an element of the row: harmless for the max
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[r][i]));
      amax = block_max_t<T>(amax, red);
      const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
      if (threadIdx.x == 0) s_a[row] = amax > 0.0f ? amax / 127.0f : 1.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int j = (int)threadIdx.x + r * T;
        if (j < nv) dst[j] = pack_codes8(y[r], inv);
      }
    } else {
      float rs = 1.0f;
      if (gamma) {
        float ss = 0.0f;
        for (int j = threadIdx.x; j < nv; j += T) {
          const half8_t v = xr[j];
#pragma unroll
          for (int i = 0; i < 8; ++i) ss = fmaf((float)v[i], (float)v[i], ss);
        }
        ss = block_sum_t<T>(ss, red);
        rs = 1.0f / sqrtf(ss / (float)K + eps);
      }
      auto row_y = [&](int j, float* y) {
        const half8_t v = xr[j];
        if (gamma) {
          const half8_t g = gr[j];
#pragma unroll
          for (int i = 0; i < 8; ++i) y[i] = ((float)v[i] * rs) * (float)g[i];
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) y[i] = (float)v[i];
        }
      };
      for (int j = threadIdx.x; j < nv; j += T) {
        float y[8];
        row_y(j, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
      }
      amax = block_max_t<T>(amax, red);
      const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
      if (threadIdx.x == 0) s_a[row] = amax > 0.0f ? amax / 127.0f : 1.0f;
      for (int j = threadIdx.x; j < nv; j += T) {
        float y[8];
        row_y(j, y);
        dst[j] = pack_codes8(y, inv);
      }
    }
  }
}

// ------------------------------------------------------- silu_mul_quant
// The SiLU-gated input of the down projection, quantized per token: row m of the fused
// gate+up output [M, 2I] holds gate in columns 0..I-1 and up in I..2I-1;
// y = silu(g) * u = g u / (1 + exp(-g)), then the per-token int8 rule of quant_act.
//
// The kernel works on y' = 2^64 y: silu of a very negative gate makes y tiny (g = -90
// gives |y| ~ 1e-37 u), and with y' the reciprocal, y' itself and the row maximum stay
// in the fp32 normal range down to the rule's own limit (a zero row only where
// fp32(127 / max|y|) overflows, max|y| below about 2^-121), while the large end stays
// finite (|y'| <= 65504^2 2^64 < 2^97).  y' = g u / ((1 + exp(-g)) 2^-64), with the
// denominator formed as 2^-64 + 2^(xh - 64) (1 + xl ln 2): a power-of-two scaling of
// every factor, so y' carries the rounding of the unscaled formula.  Then
// amax = 2^-64 max|y'| (exact), inv = fp32(127 / amax) and s_a = fp32(amax / 127) as
// in quant_act, and the codes are rint(y' (2^-64 inv)) = rint(y inv).
//
// The kernel is arithmetic-bound unless y is cheap: per element it spends about 16 VALU
// operations.  exp(-g) = 2^xh * 2^xl with xh = fp32(-g log2 e) and xl the rounding
// residual of that product (exact by fma, plus the residual of the fp32 constant), and
// 2^xl = 1 + xl ln 2 to first order (|xl| < 2^-16 wherever 2^xh is neither 0 nor inf);
// 2^xh and the reciprocal are the 1-ulp hardware approximations.  2^(xh - 64) = inf for
// very negative g gives y' = +-0.
__device__ __forceinline__ float silu_mul_scaled(float g, float u) {
  // no contraction: fused into fma(g, -kL, -64), xh - 64 would carry part of the
  // residual xl that the factor (1 + xl ln 2) adds again (2.5e-6 relative at g = -45)
#pragma clang fp contract(off)
  constexpr float kL = 1.44269502162933349609375f;   // fp32(log2 e)
  constexpr float kLlo = 1.925963e-08f;              // log2 e - kL
  constexpr float kLn2 = 0.693147182f;
  const float xh = g * -kL;
  const float xl = fmaf(g, -kLlo, fmaf(g, -kL, -xh));
  const float e = __builtin_amdgcn_exp2f(xh - 64.0f) * fmaf(xl, kLn2, 1.0f);  // 2^-64 exp(-g)
  return (g * u) * __builtin_amdgcn_rcpf(0x1p-64f + e);
}

__device__ __forceinline__ void silu_mul8(const half8_t& g, const half8_t& u, float* y) {
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = silu_mul_scaled((float)g[i], (float)u[i]);
}

// From the row maximum of |y'|: the code multiplier for y' (0 for a zero row) and s_a.
__device__ __forceinline__ float silu_row_scales(float amax_scaled, float* sa) {
  const float amax = amax_scaled * 0x1p-64f;
  const float inv = 127.0f / amax;
  const bool live = amax > 0.0f && inv <= 3.40282347e38f;  // false for inf (and nan)
  *sa = live ? amax / 127.0f : 1.0f;
  return live ? inv * 0x1p-64f : 0.0f;
}

template <int T, int R>
__global__ __launch_bounds__(T) void silu_mul_quant_kernel(const half_t* __restrict__ gu, int8_t* __restrict__ xq,
                                                            float* __restrict__ s_a, int M, int I) {
  __shared__ float red[T / 64];
  const int nv = I / 8;
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    const half8_t* g8 = reinterpret_cast<const half8_t*>(gu + row * 2 * I);
    const half8_t* u8 = g8 + nv;
    uint2* dst = reinterpret_cast<uint2*>(xq + row * I);
    float amax = 0.0f;
    if constexpr (R > 0) {
      half8_t gv[R], uv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int j = min((int)threadIdx.x + r * T, nv - 1);
        // (non-temporal: every input byte is read once; 4096 x 13824 51.1 -> 49.9 us)
        gv[r] = __builtin_nontemporal_load(g8 + j);
        uv[r] = __builtin_nontemporal_load(u8 + j);
      }
      float y[R][8];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        silu_mul8(gv[r], uv[r], y[r]);  // clamped duplicates: harmless for the max
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[r][i]));
      }
      amax = block_max_t<T>(amax, red);
      float sa;
      const float inv = silu_row_scales(amax, &sa);
      if (threadIdx.x == 0) s_a[row] = sa;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int j = (int)threadIdx.x + r * T;
        if (j < nv) dst[j] = pack_codes8(y[r], inv);
      }
    } else {
      for (int j = threadIdx.x; j < nv; j += T) {
        float y[8];
        silu_mul8(g8[j], u8[j], y);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
      }
      amax = block_max_t<T>(amax, red);
      float sa;
      const float inv = silu_row_scales(amax, &sa);
      if (threadIdx.x == 0) s_a[row] = sa;
      for (int j = threadIdx.x; j < nv; j += T) {
        float y[8];
        silu_mul8(g8[j], u8[j], y);
        dst[j] = pack_codes8(y, inv);
      }
    }
  }
}

// ------------------------------------------------------------- the GEMM
// Tile BM x 256 x 128 (one group of 128 k per step), 256 threads; the 4 waves split N
// (64 columns each = two 32-column fragments) and share all BM = 32 * MI rows (MI
// 32-row fragments).  A (xq) tiles go through LDS as 128-byte rows of 8 16-byte
// chunks (chunk c of row r at c ^ ((r / 2) % 8)).  B: lane l (column l % 32, K-slot h = l / 32)
// loads words 8h..8h+7 of its row for this step (two 16-byte chunks); k32-step s uses
// words 8h + 2s, 8h + 2s + 1 (16 codes, k = 8 (8h + 2s) .. + 15), and A is read from
// LDS with the same slot assignment.
//
// Per-channel weights enter the MFMA as 16 q (exact shift at the end); two-level
// weights enter as q * s_g, expanded per group in registers (|q s_g| <= 126 fits int8),
// so both variants accumulate the exact integer sum in one int32 accumulator set.
constexpr int WBN = 256, WBK = 128;
constexpr int kRowTilesPerGroup = 4;  // row tiles per group in the large-M tile order
// Weight formats of the int8 MFMA kernels: int4 per-channel (entering as 16 q), int4
// two-level (entering as q s_g), and plain row-major int8 [N, K] (W8A8).
constexpr int kI4PerChannel = 0, kI4TwoLevel = 1, kI8 = 2;
constexpr int kWThreads = 256;

// chunk c of row r at c ^ ((r / 2) % 8): two consecutive 128-byte rows fill one 256-byte
// bank window, so 16 consecutive rows read at one chunk hit 16 distinct bank groups
// (with c ^ (r % 8), rows r and r + 8 collided: 40 % of LDS cycles were bank conflicts)
__device__ __forceinline__ int swz8(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }
// xq tiles in flight in the direct-to-LDS pipeline, and the s_waitcnt immediate (gfx9
// encoding) that waits until at most n (< 64) vector-memory operations are outstanding.
constexpr int kRing8 = 4;
constexpr int vmcnt_imm8(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
__device__ __forceinline__ half_t cscale_or_one(const half_t* cs, int n) { return cs ? cs[n] : (half_t)1; }

// Two workgroups per CU for the one-group-ahead loop; the deeper variants (mid M, grids
// of a few hundred workgroups) may take a CU's whole register file.
template <int MI, int MODE, int PD>
__global__ __launch_bounds__(kWThreads, (PD == 1 || PD == 5) ? 2 : 1) void w4a8_gemm_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ s_a, const uint32_t* __restrict__ qweight,
    const int8_t* __restrict__ gscale, const half_t* __restrict__ cscale, half_t* __restrict__ y,
    int32_t* __restrict__ acc_out, unsigned* __restrict__ counters, int32_t* __restrict__ partials, int M, int N,
    int K, int tiles_m, int tiles_n, int splits, int gps, int n_full, int tail_splits) {
  constexpr int BM = 32 * MI;
  constexpr bool TWO = MODE == kI4TwoLevel;
  constexpr int NB = MODE == kI8 ? 4 : 2;  // 16-byte weight chunks per lane, fragment and group
  constexpr bool kDma = PD == 0 || PD == 5;
  __shared__ u32x4 lds[kDma ? 1 : 2][kDma ? 1 : BM * 8];

  const int ng = K / WBK;
  // Work item: uniform split-K (tail_splits == 0), or tail mode -- workgroups [0, n_full)
  // take tiles 0 .. n_full - 1 whole, the rest take the remaining tiles split
  // tail_splits ways; each range is remapped for the XCDs on its own.
  int tile, split, nsplit, gpl;
  if (tail_splits == 0) {
    const int id = xcd_remap(blockIdx.x, tiles_m * tiles_n * splits);
    tile = id / splits;
    split = id % splits;
    nsplit = splits;
    gpl = gps;
  } else if ((int)blockIdx.x < n_full) {
    tile = xcd_remap(blockIdx.x, n_full);
    split = 0;
    nsplit = 1;
    gpl = ng;
  } else {
    const int j = xcd_remap(blockIdx.x - n_full, gridDim.x - n_full);
    tile = n_full + j / tail_splits;
    split = j % tail_splits;
    nsplit = tail_splits;
    gpl = (ng + tail_splits - 1) / tail_splits;
  }
  // grouped ordering: walk kRowTilesPerGroup row tiles for each column tile, so the
  // tiles one XCD runs at a time (consecutive ids after xcd_remap: 64 at two workgroups
  // per CU) cover 4 row blocks of xq and 16 column blocks of weights that its L2 shares,
  // instead of every row block against two column blocks (M = 4096, K = 5120,
  // N = 13824: 1161 MB fetched per call with the plain column-major order, ~430 MB
  // grouped; groups of 4 against 8: equal at M = 4096, M = 384 / 8192 44.8 -> 43.4 /
  // 496.6 -> 482.2 us; 16 slower)
  const int per_group = kRowTilesPerGroup * tiles_n;
  const int grp = tile / per_group;
  const int first_m = grp * kRowTilesPerGroup;
  const int gsize = min(tiles_m - first_m, kRowTilesPerGroup);
  const int in_grp = tile % per_group;
  // (wave-uniform: kept in scalar registers)
  const int m0 = __builtin_amdgcn_readfirstlane((first_m + in_grp % gsize) * BM);
  const int n0 = __builtin_amdgcn_readfirstlane((in_grp / gsize) * WBN);
  const int gbeg = split * gpl;
  const int gend = min(ng, gbeg + gpl);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int col = lane & 31;
  const int h = lane >> 5;

  int nrow[2];
  bool nok[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    nrow[f] = n0 + wave * 64 + f * 32 + col;
    nok[f] = nrow[f] < N;
  }

  int16_t_ acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0;

  constexpr int kChunks = BM * 8;  // 16-byte chunks per A tile
  constexpr int kPer = (kChunks + kWThreads - 1) / kWThreads;
  u32x4 areg[kPer];
  auto load_a = [&](int g) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int cid = threadIdx.x + i * kWThreads;
      const int r = cid >> 3, c = cid & 7;
      const int m = min(m0 + r, M - 1);  // branch-free: a clamped row only reaches unstored outputs
      areg[i] = *reinterpret_cast<const u32x4*>(xq + (int64_t)m * K + g * WBK + c * 16);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int cid = threadIdx.x + i * kWThreads;
      if (cid < kChunks) lds[buf][swz8(cid >> 3, cid & 7)] = areg[i];
    }
  };
  // Columns past N read a clamped valid row; their outputs are never stored.
  int nclamp[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) nclamp[f] = min(nrow[f], N - 1);
  u32x4 breg[2][NB];
  auto load_b = [&](int g, u32x4 (&dst)[2][NB]) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (MODE == kI8) {
        // tiled int8: chunks 4 h + c (k = 64 h + 16 c .. + 15) of this lane's row, one
        // per k32-step c; each load of the wave is two contiguous 512-byte runs
        const int8_t* w8 = reinterpret_cast<const int8_t*>(qweight);
#pragma unroll
        for (int c = 0; c < NB; ++c)
          dst[f][c] = *reinterpret_cast<const u32x4*>(w8 + tiled8_offset(nclamp[f], g, 4 * h + c, ng));
      } else {
        // words 8h .. 8h + 7 of the group = slots 2h and 2h + 1 of the tiled layout
        dst[f][0] = *reinterpret_cast<const u32x4*>(qweight + tiled_chunk(nclamp[f], g, 2 * h, ng));
        dst[f][1] = *reinterpret_cast<const u32x4*>(qweight + tiled_chunk(nclamp[f], g, 2 * h + 1, ng));
      }
    }
  };

  // Group scales of this lane's rows, prefetched one step ahead with the codes.
  int sgraw[2] = {1, 1};
  auto load_sg = [&](int g, int (&dst)[2]) {
    if (TWO) {
#pragma unroll
      for (int f = 0; f < 2; ++f) dst[f] = (int)gscale[(int64_t)g * N + nclamp[f]];
    }
  };

  // One group's MFMAs: B chunks of this lane (expanded to int8), A from LDS buffer buf.
  auto compute = [&](const u32x4 (&bq)[2][NB], const int (&sgv)[2], int buf) {
    u16x2 sp[2], cp[2];
    if (TWO) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int sg = sgv[f];
        sp[f] = u16x2{(unsigned short)sg, (unsigned short)sg};
        cp[f] = u16x2{(unsigned short)(-8 * sg), (unsigned short)(-8 * sg)};
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      int4_t bf[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (MODE == kI8) {
          const u32x4 v = bq[f][s];
          bf[f] = int4_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
          continue;
        }
        const uint32_t w0 = bq[f][s >> 1][(s & 1) * 2];
        const uint32_t w1 = bq[f][s >> 1][(s & 1) * 2 + 1];
        uint32_t a0, a1, a2, a3;
        if (TWO) {
          unpack_i4_scaled(w0, sp[f], cp[f], a0, a1);
          unpack_i4_scaled(w1, sp[f], cp[f], a2, a3);
        } else {
          unpack_i4x16(w0, a0, a1);
          unpack_i4x16(w1, a2, a3);
        }
        bf[f] = int4_t{(int)a0, (int)a1, (int)a2, (int)a3};
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const u32x4 av = lds[buf][swz8(i * 32 + col, h * 4 + s)];
        const int4_t a = __builtin_bit_cast(int4_t, av);
#pragma unroll
        for (int f = 0; f < 2; ++f) acc[i][f] = mfma32_i8(a, bf[f], acc[i][f]);
      }
    }
  };

  if constexpr (kDma) {
    // Direct-to-LDS pipeline (as in the fp16 GEMM): the xq tile of group t lands in LDS
    // ring slot t % kRing8 straight from global memory, issued kRing8 - 1 groups ahead, with
    // this lane's weight chunks and group scales in register set t % kRing8.  Every group
    // issues the same kPerStage loads per thread, so "at most 2 kPerStage outstanding" means
    // group t's loads are complete; a barrier then makes the whole tile visible and frees
    // the slot and set of group t - 1 for group t + 3.  Loads past the range are clamped.
    // ring of R tiles: 4 with one workgroup per CU (PD 0), 3 with two (PD 5)
    constexpr int R = PD == 5 ? 3 : kRing8;
    constexpr int kPerStage = kPer + 2 * NB + (TWO ? 2 : 0);
    constexpr int kWaitImm = vmcnt_imm8((R - 2) * kPerStage);
    // chunk i of this thread lands at LDS position P = (4 i + wave) * 64 + lane and holds
    // the xq chunk the swizzle puts there: row r = P / 8 = 32 i + 8 wave + lane / 8,
    // k-chunk (P % 8) ^ ((r / 2) % 8), the same chunk for every i (r / 2 moves by 16 per i);
    // the row offsets are formed at each issue (no registers held for them)
    const int arow0 = m0 + 8 * wave + (lane >> 3);
    const uint32_t acol = (uint32_t)((((lane & 7) ^ (((8 * wave + (lane >> 3)) >> 1) & 7))) * 16);
    // one LDS array per ring slot (the compiler's wait insertion tells loads into distinct
    // arrays apart)
    __shared__ u32x4 ring0[BM * 8], ring1[BM * 8], ring2[BM * 8], ring3[BM * 8];
    auto ring = [&](int j) -> u32x4* { return j == 0 ? ring0 : j == 1 ? ring1 : j == 2 ? ring2 : ring3; };
    struct Stage {
      u32x4 b[2][NB];
      int sg[2];
    };
    Stage st[R];
    auto issue = [&](int g, int slot, Stage& S) {
      load_b(g, S.b);
      S.sg[0] = S.sg[1] = 1;
      load_sg(g, S.sg);
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        __builtin_amdgcn_global_load_lds(
            (void*)(xq + (uint32_t)min(arow0 + 32 * i, M - 1) * (uint32_t)K + acol + g * WBK),
                                         (__attribute__((address_space(3))) void*)(ring(slot) + (4 * i + wave) * 64), 16, 0,
                                         0);
    };
    auto step = [&](int t, int j) {
      __builtin_amdgcn_s_waitcnt(kWaitImm);
      __builtin_amdgcn_s_barrier();
      // nothing that reads this step's registers may be scheduled above the wait (the
      // compiler's own wait for such a read drains every load in flight)
      __builtin_amdgcn_sched_barrier(0);
      issue(min(t + R - 1, gend - 1), (j + R - 1) % R, st[(j + R - 1) % R]);
      const Stage& S = st[j];
      const u32x4* xa = ring(j);
      u16x2 sp[2], cp[2];
      if (TWO) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int sg = S.sg[f];
          sp[f] = u16x2{(unsigned short)sg, (unsigned short)sg};
          cp[f] = u16x2{(unsigned short)(-8 * sg), (unsigned short)(-8 * sg)};
        }
      }
      // A fragments of k32 steps s (in use) and s + 1 (in flight) with one wave per SIMD;
      // with two, the other wave covers the LDS latency and the registers are short
      constexpr bool kAhead = PD == 0;
      int4_t afr[2][MI];
      if (kAhead) {
#pragma unroll
        for (int i = 0; i < MI; ++i) afr[0][i] = __builtin_bit_cast(int4_t, xa[swz8(i * 32 + col, h * 4)]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (kAhead && s < 3) {
#pragma unroll
          for (int i = 0; i < MI; ++i)
            afr[(s + 1) & 1][i] = __builtin_bit_cast(int4_t, xa[swz8(i * 32 + col, h * 4 + s + 1)]);
        }
        if (!kAhead) {
#pragma unroll
          for (int i = 0; i < MI; ++i) afr[s & 1][i] = __builtin_bit_cast(int4_t, xa[swz8(i * 32 + col, h * 4 + s)]);
        }
        int4_t bf[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          if (MODE == kI8) {
            const u32x4 v = S.b[f][s];
            bf[f] = int4_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
            continue;
          }
          const uint32_t w0 = S.b[f][s >> 1][(s & 1) * 2];
          const uint32_t w1 = S.b[f][s >> 1][(s & 1) * 2 + 1];
          uint32_t a0, a1, a2, a3;
          if (TWO) {
            unpack_i4_scaled(w0, sp[f], cp[f], a0, a1);
            unpack_i4_scaled(w1, sp[f], cp[f], a2, a3);
          } else {
            unpack_i4x16(w0, a0, a1);
            unpack_i4x16(w1, a2, a3);
          }
          bf[f] = int4_t{(int)a0, (int)a1, (int)a2, (int)a3};
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int f = 0; f < 2; ++f) acc[i][f] = mfma32_i8(afr[s & 1][i], bf[f], acc[i][f]);
      }
    };
    const int nsteps = gend - gbeg;
    if (nsteps > 0) {
#pragma unroll
      for (int d = 0; d < R - 1; ++d) issue(min(gbeg + d, gend - 1), d, st[d]);
      int it = 0;
      for (; it + R <= nsteps; it += R) {
#pragma unroll
        for (int j = 0; j < R; ++j) step(gbeg + it + j, j);
      }
#pragma unroll
      for (int j = 0; j < R; ++j)
        if (it + j < nsteps) step(gbeg + it + j, j);
      // no LDS write may still be in flight when the workgroup's LDS is released
      __builtin_amdgcn_s_waitcnt(vmcnt_imm8(0));
    }
  } else if constexpr (PD == 1) {
    // the next group's loads are issued at the top of each step (one set of A registers)
    if (gbeg < gend) {
      load_a(gbeg);
      load_b(gbeg, breg);
      load_sg(gbeg, sgraw);
      store_a(0);
    }
    __syncthreads();
    for (int g = gbeg; g < gend; ++g) {
      const int buf = (g - gbeg) & 1;
      const int sgcur[2] = {sgraw[0], sgraw[1]};
      // next group's loads, unconditional (clamped on the last iteration; see the W4A16 GEMM)
      const int gn = min(g + 1, gend - 1);
      u32x4 bnext[2][NB];
      load_a(gn);
      load_b(gn, bnext);
      load_sg(gn, sgraw);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the MFMAs
      compute(breg, sgcur, buf);
      store_a(buf ^ 1);
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int c = 0; c < NB; ++c) breg[f][c] = bnext[f][c];
      __syncthreads();
    }
  } else {
    // PD register sets rotate: group t's MFMAs use set t % PD, then the next group's
    // xq chunks go to the other LDS buffer and, after the barrier, the set is refilled
    // with group t + PD's loads (clamped: no conditional loads).
    struct Stage {
      u32x4 a[kPer];
      u32x4 b[2][NB];
      int sg[2];
    };
    Stage st[PD];
    auto issue = [&](int g, Stage& S) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int cid = threadIdx.x + i * kWThreads;
        const int r = cid >> 3, c = cid & 7;
        const int m = min(m0 + r, M - 1);
        S.a[i] = *reinterpret_cast<const u32x4*>(xq + (int64_t)m * K + g * WBK + c * 16);
      }
      load_b(g, S.b);
      S.sg[0] = S.sg[1] = 1;
      load_sg(g, S.sg);
    };
    auto store_s = [&](const Stage& S, int buf) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int cid = threadIdx.x + i * kWThreads;
        if (cid < kChunks) lds[buf][swz8(cid >> 3, cid & 7)] = S.a[i];
      }
    };
    auto step = [&](int t, Stage& S, const Stage& Snext) {
      const int buf = (t - gbeg) & 1;
      compute(S.b, S.sg, buf);
      store_s(Snext, buf ^ 1);
      __syncthreads();
      issue(min(t + PD, gend - 1), S);
    };
    const int nsteps = gend - gbeg;
    if (nsteps > 0) {
#pragma unroll
      for (int d = 0; d < PD; ++d) issue(min(gbeg + d, gend - 1), st[d]);
      store_s(st[0], 0);
    }
    __syncthreads();
    int it = 0;
    for (; it + PD <= nsteps; it += PD) {
#pragma unroll
      for (int d = 0; d < PD; ++d) step(gbeg + it + d, st[d], st[(d + 1) % PD]);
    }
#pragma unroll
    for (int d = 0; d < PD; ++d)
      if (it + d < nsteps) step(gbeg + it + d, st[d], st[(d + 1) % PD]);
  }
  if (MODE == kI4PerChannel) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][f][r] >>= 4;
  }

  // The epilogue's lane indices are formed again from the thread id (hidden from the
  // compiler, which would otherwise keep the first ones live across the main loop: one
  // register too many for the three-slot ring of the two-level weights).
  int tid_e = (int)threadIdx.x;
  asm volatile("" : "+v"(tid_e));
  const int he = (tid_e >> 5) & 1;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    nrow[f] = n0 + wave * 64 + f * 32 + (tid_e & 31);
    nok[f] = nrow[f] < N;
    nclamp[f] = min(nrow[f], N - 1);
  }
  // element (i, f, r): row m0 + 32 i + 8 (r / 4) + 4 he + (r % 4), column nrow[f]
  if (nsplit > 1) {
    // Split K: every part writes its int32 partial sums, the last arriving workgroup
    // adds the others' to its own (exact in any order).  Uniform mode keeps the partials
    // as [split][M][N]; a tail tile j (tail mode) as a compact [j][split][BM][WBN]
    // region.  One code path for both (two made the compiler spill).
    const bool tail = tail_splits > 0;
    int32_t* pbase = tail ? partials + (int64_t)(tile - n_full) * nsplit * BM * WBN : partials + (int64_t)m0 * N + n0;
    const int64_t ld = tail ? (int64_t)WBN : (int64_t)N;
    const int64_t sstride = tail ? (int64_t)BM * WBN : (int64_t)M * N;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (!nok[f]) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * he + (r & 3);
          if (m < M) st_coherent(pbase + split * sstride + (m - m0) * ld + (nrow[f] - n0), acc[i][f][r]);
        }
      }
    if (!splitk_arrive(counters + (tail ? tile - n_full : tile), nsplit)) return;
    // one 16-value fragment at a time (its loads in flight together)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int f = 0; f < 2; ++f)
        for (int sp_ = 0; sp_ < nsplit; ++sp_) {
          if (sp_ == split) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = min(m0 + i * 32 + 8 * (r >> 2) + 4 * he + (r & 3), M - 1);
            acc[i][f][r] += ld_coherent(pbase + sp_ * sstride + (m - m0) * ld + (nclamp[f] - n0));
          }
        }
  }
  const float cs0 = nok[0] ? (float)cscale_or_one(cscale, nrow[0]) : 0.0f;
  const float cs1 = nok[1] ? (float)cscale_or_one(cscale, nrow[1]) : 0.0f;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (!nok[f]) continue;
      const float cs = f == 0 ? cs0 : cs1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * he + (r & 3);
        if (m < M) {
          if (acc_out) acc_out[(int64_t)m * N + nrow[f]] = acc[i][f][r];
          else y[(int64_t)m * N + nrow[f]] = (half_t)(((float)acc[i][f][r] * s_a[m]) * cs);
        }
      }
    }
}

// ---------------------------------------------------------------------------------
// Skinny W4A8 (M <= 16): bandwidth-bound, every packed byte read once, on
// v_mfma_i32_16x16x64_i8.  Work split as in the register-X W4A16 skinny kernel: a
// workgroup (4 waves) owns 16 T columns and a range of groups, its waves take the groups
// round robin with D register sets prefetched.  Per group a lane loads its 16-byte code
// chunk (row l % 16, k-slot l / 16 = 32 k) of each tile -- one contiguous 1 KB block per
// wave -- and the two 16-byte xq pieces of the same k range; MFMA j uses words 2j, 2j + 1
// of the chunk (16 k) expanded to int8 (16 q per-channel, q s_g two-level).  The int32
// accumulators need no per-group work: the sum is exact, so the cross-wave (LDS) and
// split-K reductions are exact in any order.
template <int T, int MODE>
struct W8Regs {
  u32x4 b[T][MODE == kI8 ? 2 : 1];  // codes of this lane's row and k-slot in each n-tile
  int4_t a[2];                      // xq: k = 32 slot + 16 j .. + 15, j = 0, 1
  int32_t gsc[kChunks<T>];          // two-level: group scale of column n0 + chunk_col(c, lane)
};

template <int T, int MODE>
__device__ __forceinline__ void w8_load(W8Regs<T, MODE>& r, const int8_t* __restrict__ xq,
                                        const uint32_t* __restrict__ qweight, const int8_t* __restrict__ gscale,
                                        int g, int n0, int lane, int M, int N, int K) {
  const int ng = K / 128;
  const int last_tile = (N - 1) >> 4;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (MODE == kI8) {
      // tiled int8 weights: chunks 2 slot and 2 slot + 1 (k = 32 slot .. + 31) of this
      // lane's row; each load of the wave is two contiguous 512-byte runs
      const int8_t* w8 = reinterpret_cast<const int8_t*>(qweight);
      const int nc = min(n0 + 16 * t + (lane & 15), 16 * last_tile + 15);
      const int slot = lane >> 4;
      r.b[t][0] = ld_stream(w8 + tiled8_offset(nc, g, 2 * slot, ng));
      r.b[t][1] = ld_stream(w8 + tiled8_offset(nc, g, 2 * slot + 1, ng));
    } else {
      const int tile = min((n0 >> 4) + t, last_tile);
      r.b[t][0] = ld_stream(qweight + ((int64_t)tile * ng + g) * 256 + lane * 4);
    }
  }
  if (MODE == kI4TwoLevel) {
    // one load per 64 columns; moved to the MFMA layout in w8_compute
#pragma unroll
    for (int c = 0; c < kChunks<T>; ++c) r.gsc[c] = gscale[(int64_t)g * N + min(n0 + chunk_col<T>(c, lane), N - 1)];
  }
  const int m = min(lane & 15, M - 1);
  const int4_t* src = reinterpret_cast<const int4_t*>(xq + (int64_t)m * K + g * 128 + (lane >> 4) * 32);
  r.a[0] = src[0];
  r.a[1] = src[1];
}

template <int T, int MODE>
__device__ __forceinline__ void w8_compute(const W8Regs<T, MODE>& r, int4_t (&acc)[T]) {
  constexpr bool TWO = MODE == kI4TwoLevel;
  uint32_t gsv[T];  // group scale of this lane's column in each n-tile
  if (TWO) {
    uint32_t gsc[kChunks<T>];
#pragma unroll
    for (int c = 0; c < kChunks<T>; ++c) gsc[c] = (uint32_t)r.gsc[c];
    rows_to_tiles<T>(gsc, gsv);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (MODE == kI8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 v = r.b[t][j];
        acc[t] = mfma16_i8(r.a[j], int4_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3]}, acc[t]);
      }
      continue;
    }
    u16x2 sp = {1, 1}, cp = {0, 0};
    if (TWO) {
      const unsigned short g16 = (unsigned short)(int)gsv[t];
      sp = u16x2{g16, g16};
      const unsigned short c16 = (unsigned short)(-8 * (int)gsv[t]);
      cp = u16x2{c16, c16};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t e[4];
      const uint32_t w0 = r.b[t][0][2 * j], w1 = r.b[t][0][2 * j + 1];
      if (TWO) {
        unpack_i4_scaled(w0, sp, cp, e[0], e[1]);
        unpack_i4_scaled(w1, sp, cp, e[2], e[3]);
      } else {
        unpack_i4x16(w0, e[0], e[1]);
        unpack_i4x16(w1, e[2], e[3]);
      }
      const int4_t bv = {(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
      acc[t] = mfma16_i8(r.a[j], bv, acc[t]);
    }
  }
}

template <int T, int D, int MODE>
__global__ __launch_bounds__(256) void w4a8_skinny_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ s_a, const uint32_t* __restrict__ qweight,
    const int8_t* __restrict__ gscale, const half_t* __restrict__ cscale, half_t* __restrict__ y,
    int32_t* __restrict__ acc_out, unsigned* __restrict__ counters, int32_t* __restrict__ partials, int M, int N,
    int K, int splits, int gps) {
  constexpr int WAVES = 4, kT = WAVES * kWave, kCols = 16 * T;
  __shared__ int32_t red[WAVES][T * 4 * kWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = blockIdx.x, split = blockIdx.y;
  const int n0 = rb * kCols;
  const int ng = K / 128;
  const int gbeg = split * gps, gend = min(ng, gbeg + gps);

  int4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = int4_t{0, 0, 0, 0};
  W8Regs<T, MODE> r[D];
  const int glast = gend - 1;
  const int g = gbeg + wave;
#pragma unroll
  for (int d = 0; d < D; ++d) w8_load<T, MODE>(r[d], xq, qweight, gscale, min(g + d * WAVES, glast), n0, lane, M, N, K);
  // steady state without conditions, then the remaining < D groups (wave-uniform counts)
  const int mine = g < gend ? (gend - g + WAVES - 1) / WAVES : 0;
  int it = 0;
  for (; it + D <= mine; it += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      w8_compute<T, MODE>(r[d], acc);
      // (scheduling fences: the next set's MFMAs must not start before this set's loads
      // are issued, or the waits drain nearly every load in flight)
      __builtin_amdgcn_sched_barrier(0);
      w8_load<T, MODE>(r[d], xq, qweight, gscale, min(g + (it + d + D) * WAVES, glast), n0, lane, M, N, K);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (it + d < mine) w8_compute<T, MODE>(r[d], acc);

  // Cross-wave reduction: element (t, i) of lane l is row 4 (l / 16) + i, column
  // n0 + 16 t + l % 16.
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][(t * 4 + i) * kWave + lane] = acc[t][i];
  __syncthreads();
  const int outs = M * kCols;
  for (int o = threadIdx.x; o < outs; o += kT) {
    const int m = o / kCols, nl = o - m * kCols, n = n0 + nl;
    const int idx = ((nl >> 4) * 4 + (m & 3)) * kWave + (m >> 2) * 16 + (nl & 15);
    int32_t v = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][idx];
    if (n >= N) continue;
    if (splits == 1) {
      if (MODE == kI4PerChannel) v >>= 4;  // exact: every term was 16 q
      if (acc_out) acc_out[(int64_t)m * N + n] = v;
      else y[(int64_t)m * N + n] = (half_t)(((float)v * s_a[m]) * (float)cscale[n]);
    } else {
      st_coherent(partials + ((int64_t)split * M + m) * N + n, v);
    }
  }
  if (splits == 1) return;
  if (!splitk_arrive(counters + rb, splits)) return;
  for (int o = threadIdx.x; o < outs; o += kT) {
    const int m = o / kCols, n = n0 + o - m * kCols;
    if (n >= N) continue;
    int32_t v = 0;
    for (int sp_ = 0; sp_ < splits; ++sp_) v += ld_coherent(partials + ((int64_t)sp_ * M + m) * N + n);
    if (MODE == kI4PerChannel) v >>= 4;
    if (acc_out) acc_out[(int64_t)m * N + n] = v;
    else y[(int64_t)m * N + n] = (half_t)(((float)v * s_a[m]) * (float)cscale[n]);
  }
}

}  // namespace

hipError_t launch_w4a8_quant_act(const void* x, const void* gamma, float eps, int8_t* xq, float* s_a, int M,
                                 int K, hipStream_t stream) {
  W4_ROW_DISPATCH(quant_act_kernel, false, K / 8, dim3(row_grid(M)), stream, (const half_t*)x, (const half_t*)gamma, eps,
                  xq, s_a, M, K);
  return hipGetLastError();
}

hipError_t launch_w4a8_silu_mul_quant(const void* gate_up, int8_t* xq, float* s_a, int M, int I,
                                      hipStream_t stream) {
  W4_ROW_DISPATCH(silu_mul_quant_kernel, true, I / 8, dim3(row_grid(M)), stream, (const half_t*)gate_up, xq, s_a, M, I);
  return hipGetLastError();
}

// M <= 16 takes the skinny kernel (tiles of 16 columns per workgroup, split-K towards
// 320 workgroups while each wave keeps a group); larger M the tiled MFMA GEMM.
// group_size: -1 per-channel W4A8, 128 two-level W4A8, 0 W8A8 (8-bit codes).
W4A8Plan w4a8_plan(int M, int N, int K, int group_size) {
  W4A8Plan p;
  p.skinny = 0;
  p.n_full = 0;
  p.tail_splits = 0;
  p.depth = 1;
  if (M <= 16 && env_int("W4_W4A8_SKINNY", 1)) {
    const int ng = K / 128;
    // Tiles and split target from sweeps on the Llama-2-13B decode shapes (M = 1, 4, 16):
    // splitting K never paid once the column blocks give 160 workgroups (the int32
    // partials are M N 4 bytes per split, and their fixup costs ~1.5 us); for M > 1 wide
    // tiles share each xq fragment between more columns, except at M <= 4 on narrow
    // matrices, where one-tile workgroups (more of them in flight) win with the weights
    // streamed from HBM (13824 x 5120 at M = 4: g128 14.5 -> 12.1 us, per-channel
    // 11.8 -> 11.0; 5120 x 5120: 7.3 -> 6.5, 6.3 -> 6.0).
    // W8A8 (group_size 0: 8-bit codes, twice the bytes per tile) keeps two tiles there
    // (13824 x 5120 at M = 1-4: 16.6-17.4 -> 14.6-15.0 us against one tile).
    int t = env_int("W4_W4A8_TILES", 0);
    if (t != 1 && t != 2 && t != 4) {
      if (group_size == 0 && M <= 4 && N <= 5120) t = 2;
      else t = M == 1 ? (N <= 5120 ? 1 : (N <= 16384 ? 2 : 4)) : (N > 8192 ? 4 : (M <= 4 && N <= 5120 ? 1 : 2));
    }
    p.skinny = 1;
    p.bm = 16;
    p.tiles_m = 1;
    p.tiles_n = (N + 16 * t - 1) / (16 * t);
    p.tiles = t;
    const int target = env_int("W4_W4A8_SKINNY_BLOCKS", 160);
    int splits = (target + p.tiles_n - 1) / p.tiles_n;
    splits = max(1, min(splits, ng / 4));
    if (p.tiles_n >= kMaxCounters) splits = 1;
    p.kt_per_split = (ng + splits - 1) / splits;
    p.splits = (ng + p.kt_per_split - 1) / p.kt_per_split;
    return p;
  }
  // Row-tile height and loop, from sweeps at K = 5120, N = 13824 over the three weight
  // formats (clocks warm, weights streamed from HBM): 32-row tiles with four register
  // sets of loads in flight up to M = 128 (M = 128 per-channel 54.0 -> 23.0 us against
  // one ahead); 64-row tiles up to 512 with the four-tile direct-to-LDS ring (depth 0:
  // per-channel / two-level / int8 weights at M = 256 33.9 / 48.0 / 41.9 us with four
  // register sets -> 30.5 / 41.0 / 40.0, at M = 512 58.0 / 72.7 / 65.0 one group ahead
  // -> 46.1 / 62.0 / 61.4); 128-row tiles above 512, int4 weights with the three-tile
  // ring at two workgroups per CU (depth 5, M = 4096: per-channel 321.9 -> 270.5 us,
  // two-level 382.2 -> 328.6), int8 weights one group ahead.
  // (narrow, short-K matrices keep the 32-row tiles up to M = 384: K = 5120, N = 5120
  // per-channel at M = 192 / 256 / 384 26.6 / 25.8 / 26.0 -> 18.3 / 19.9 / 20.1 us, W8A8 at
  // M = 256 28.2 -> 23.2, N = 8192 at M = 256 27.7 -> 21.4; slower at M = 512, at
  // K = 13824 and on N = 13824)
  const bool short_narrow = N <= 8192 && K <= 8192 && M <= 384;
  // (512 < M <= 768: 64-row tiles, for int4 weights on the three-slot ring at two
  // workgroups per CU on wide matrices, otherwise the four-slot ring at one --
  // per-channel on 5120 x 13824 at M = 640 / 768 72.0 / 73.7 -> 58.5 / 60.6 us (two-level
  // 85.7 -> 84.2), on 5120 x 5120 at M = 768 48.8 -> 27.3; W8A8 96.6 / 98.3 -> 82.1 /
  // 84.8, 62.4 -> 33.1, 13824 x 5120 at M = 600 105.8 -> 77.7; 128-row tiles stay faster
  // at M = 1024 on wide matrices; extended for per-channel and W8A8 weights where
  // measured: narrow matrices up to M = 2048 -- 5120 x 5120 at M = 1024 48.5 / 69.8 ->
  // 39.8 / 49.1 us, at M = 1536 / 2048 per-channel 49.2 / 70.1 -> 42.1 / 61.9 and W8A8 at
  // 2048 86.5 -> 77.2, per-channel on 13824 x 5120 at M = 896 / 2048 95.6 / 148.2 ->
  // 81.3 / 135.4 -- and per-channel on wide ones up to M = 896 -- 75.5 -> 61.8; not for
  // two-level weights, 3-8 % slower past M = 768)
  const bool two_level = group_size > 0;
  const int rows64_max = two_level ? 768 : N <= 8192 ? 2048 : (group_size < 0 ? 896 : 768);
  const bool mid_rows = M > 512 && M <= rows64_max;
  p.bm = env_int("W4_W4A8_BM", (M <= 128 || short_narrow) ? 32 : ((M <= 512 || mid_rows) ? 64 : 128));
  if (p.bm != 32 && p.bm != 64) p.bm = 128;
  // int8 weights on 128-row tiles: the four-tile ring at one workgroup per CU (depth 0)
  // beats the one-ahead loop at two per CU on narrow matrices (N <= 8192) with more tiles
  // than one round of two per CU (M = 4096: 5120 x 5120 172.2 -> 163.8 us, K = 8192
  // 226.7 -> 216.9, K = 13824 341.8 -> 319.8; M = 8192 625.0 -> 610.9), not with fewer
  // (M = 2048, 320 tiles: 217.7 -> 231.1) or on N = 13824 (even at K = 13824, slower at
  // K = 5120: 366.1 -> 406.5)
  const bool i8_ring = group_size == 0 && N <= 8192 && (int64_t)((M + 127) / 128) * ((N + 255) / 256) > 512;
  const int dflt =
      p.bm == 32 ? 4 : p.bm == 64 ? (mid_rows && group_size != 0 && N > 8192 ? 5 : 0) : (group_size != 0 ? 5 : (i8_ring ? 0 : 1));
  p.depth = env_int("W4_W4A8_DEPTH", dflt);
  // depth 0: the direct-to-LDS pipeline (64- and 128-row tiles; 32-bit xq offsets)
  if (!((p.depth == 1) || (p.bm == 32 && p.depth == 4) || (p.bm == 64 && (p.depth == 3 || p.depth == 4)) ||
        (p.depth == 0 && p.bm >= 64 && (int64_t)M * K < (int64_t(1) << 31)) ||
        // depth 5: three-tile direct-to-LDS ring, two workgroups per CU (128-row tiles only
        // with int4 weights: the int8 weights' register sets do not fit three deep)
        (p.depth == 5 && (p.bm == 64 || (p.bm == 128 && group_size != 0)) &&
         (int64_t)M * K < (int64_t(1) << 31))))
    p.depth = 1;
  p.tiles_m = (M + p.bm - 1) / p.bm;
  p.tiles_n = (N + WBN - 1) / WBN;
  const int ng = K / WBK;
  const int tiles = p.tiles_m * p.tiles_n;
  const int target = env_int("W4_W4A8_SPLIT_TARGET", 128);  // int32 partials are M N 4 bytes per split
  int splits = 1;
  while (tiles * splits < target && ng / (splits * 2) >= 2) splits *= 2;
  if (tiles >= kMaxCounters) splits = 1;
  p.kt_per_split = (ng + splits - 1) / splits;
  p.splits = (ng + p.kt_per_split - 1) / p.kt_per_split;
  // Tail split (128-row tiles, two resident per CU: 512 slots on 256 CUs): the last
  // round's tiles split in two over their groups.  Taken by default only when that round
  // holds at most a quarter of the slots and K is long (at least 64 groups), where the
  // uneven round costs more than the int32 partials: M = 4096 on 13824 x 5120 (640 tiles,
  // 128 in the last round) per-channel / two-level / W8A8 250.6 / 315.6 / 396.9 ->
  // 234.9 / 292.2 / 356.1 us, K = 8192 165.7 -> 161.0; slower with 192 or 208 tiles in
  // the last round (M = 4096 on 5120 x 13824 253.1 -> 279.6, M = 4608 on 13824 x 5120
  // 257.9 -> 273.5), no faster at K = 5120, and four parts slower than two.
  // W4_W4A8_TAIL = 1 takes it whenever the last round is at most half full, 0 never.
  p.n_full = 0;
  p.tail_splits = 0;
  const int slots = 512 * env_int("W4_W4A8_SLOTS_SCALE", 1) / env_int("W4_W4A8_SLOTS_DIV", 1);
  const int rem = tiles % slots;
  const int tail_env = env_int("W4_W4A8_TAIL", -1);
  const bool tail_ok = tail_env < 0 ? (4 * rem <= slots && ng >= 64) : (tail_env > 0 && 2 * rem <= slots);
  if (p.bm == 128 && p.splits == 1 && tail_ok && tiles > slots && rem > 0 && ng >= 8) {
    p.n_full = tiles - rem;
    p.tail_splits = max(2, min(8, env_int("W4_W4A8_TAIL_PARTS", 2)));
  }
  return p;
}

size_t w4a8_workspace_bytes(const W4A8Plan& p, int M, int N) {
  if (p.tail_splits > 0)
    return kCounterRegionBytes +
           (size_t)(p.tiles_m * p.tiles_n - p.n_full) * p.tail_splits * p.bm * WBN * sizeof(int32_t);
  if (p.splits == 1) return 0;
  return kCounterRegionBytes + (size_t)p.splits * M * N * sizeof(int32_t);
}

namespace {

hipError_t launch_int8_gemm(const W4A8Plan& p, int mode, const int8_t* xq, const float* s_a, const void* qweight,
                            const int8_t* gscale, const void* cscale, void* y, int32_t* acc_out, void* ws, int M,
                            int N, int K, hipStream_t stream) {
  unsigned* counters = (unsigned*)ws;
  int32_t* partials = ws ? (int32_t*)((char*)ws + kCounterRegionBytes) : nullptr;
  const int tiles = p.tiles_m * p.tiles_n;
  const int blocks = p.tail_splits > 0 ? p.n_full + (tiles - p.n_full) * p.tail_splits : tiles * p.splits;
  const dim3 grid(blocks), block(kWThreads);
  const uint32_t* qw = (const uint32_t*)qweight;
  const half_t* cs = (const half_t*)cscale;
  half_t* yh = (half_t*)y;
  const int8_t* gs = mode == kI4TwoLevel ? gscale : nullptr;
  if (p.skinny) {
    const dim3 sgrid(p.tiles_n, p.splits), sblock(256);
#define W4A8_SKINNY(T, D, MODE)                                                                                  \
  hipLaunchKernelGGL((w4a8_skinny_kernel<T, D, MODE>), sgrid, sblock, 0, stream, xq, s_a, qw, gs, cs, yh, acc_out, \
                     counters, partials, M, N, K, p.splits, p.kt_per_split)
#define W4A8_SKINNY_T(MODE)                      \
  if (p.tiles == 4) W4A8_SKINNY(4, 2, MODE);     \
  else if (p.tiles == 2) W4A8_SKINNY(2, 2, MODE); \
  else W4A8_SKINNY(1, 4, MODE)
    if (mode == kI4TwoLevel) { W4A8_SKINNY_T(kI4TwoLevel); }
    else if (mode == kI8) { W4A8_SKINNY_T(kI8); }
    else { W4A8_SKINNY_T(kI4PerChannel); }
#undef W4A8_SKINNY_T
#undef W4A8_SKINNY
    return hipGetLastError();
  }
#define W4A8_LAUNCH(MI, MODE, PD)                                                                              \
  if (mi == MI && p.depth == PD) {                                                                              \
    hipLaunchKernelGGL((w4a8_gemm_kernel<MI, MODE, PD>), grid, block, 0, stream, xq, s_a, qw, gs, cs, yh, acc_out, \
                       counters, partials, M, N, K, p.tiles_m, p.tiles_n, p.splits, p.kt_per_split, p.n_full,    \
                       p.tail_splits);                                                                          \
    return hipGetLastError();                                                                                   \
  }
#define W4A8_LAUNCH_MI(MODE) \
  W4A8_LAUNCH(1, MODE, 1) W4A8_LAUNCH(2, MODE, 1) W4A8_LAUNCH(4, MODE, 1) W4A8_LAUNCH(1, MODE, 4) \
  W4A8_LAUNCH(2, MODE, 3) W4A8_LAUNCH(2, MODE, 4) W4A8_LAUNCH(4, MODE, 0) W4A8_LAUNCH(2, MODE, 0)    \
  W4A8_LAUNCH(2, MODE, 5)
  const int mi = p.bm / 32;
  if (mode == kI4TwoLevel) { W4A8_LAUNCH_MI(kI4TwoLevel); W4A8_LAUNCH(4, kI4TwoLevel, 5); }
  else if (mode == kI8) { W4A8_LAUNCH_MI(kI8); }
  else { W4A8_LAUNCH_MI(kI4PerChannel); W4A8_LAUNCH(4, kI4PerChannel, 5); }
#undef W4A8_LAUNCH_MI
#undef W4A8_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_w4a8_gemm(const W4A8Plan& p, const int8_t* xq, const float* s_a, const int32_t* qweight,
                            const int8_t* gscale, const void* cscale, void* y, int32_t* acc_out, void* ws, int M,
                            int N, int K, int group_size, hipStream_t stream) {
  return launch_int8_gemm(p, group_size == -1 ? kI4PerChannel : kI4TwoLevel, xq, s_a, qweight, gscale, cscale, y,
                          acc_out, ws, M, N, K, stream);
}

hipError_t launch_w8a8_gemm(const W4A8Plan& p, const int8_t* xq, const float* s_a, const int8_t* qweight,
                            const void* cscale, void* y, int32_t* acc_out, void* ws, int M, int N, int K,
                            hipStream_t stream) {
  return launch_int8_gemm(p, kI8, xq, s_a, qweight, nullptr, cscale, y, acc_out, ws, M, N, K, stream);
}

}  // namespace w4
