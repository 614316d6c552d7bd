// Skinny W4A16 GEMM for M <= 64 (decode): bandwidth-bound, every packed weight byte
// is read once.
//
// The pages single out the small-batch regime ("Implement AWQ quantization support
// for LLaMA", vllm-project/vllm PR 1032: the AWQ GEMM is fastest below batch 8 and
// on par with FP16 at batch 16) and say that dequantization is the tricky part.
// Here the dequantization is folded into per-group fp32 arithmetic:
//
//   Y[m,n] = sum_g s[n,g] * ( T_g[m,n] - (1024 + z[n,g]) * S_g[m] ),
//   T_g[m,n] = sum_{k in g} X[m,k] * (1024 + q[n,k]),   S_g[m] = sum_{k in g} X[m,k],
//
// which equals sum_k X[m,k] * (q - z) * s exactly in real arithmetic.  The MFMA
// consumes the raw fp16 values 1024 + q (nine VALU ops per 8 codes, no per-element
// subtract or multiply); S_g comes from one extra MFMA against a B operand of ones.
// fp16 x (1024 + q) products are exact in fp32; only the fp32 sums round.
//
// Work split: a workgroup (8 waves; 4 when M > 16) owns 64 output columns n (4 tiles of 16) and a
// contiguous range of K groups (split-K across workgroups); its waves take the groups
// of that range round robin.  Per group, lane l of a wave loads one 16-byte chunk
// (32 codes) of row n0 + 16t + (l % 16) for each of the 4 tiles t, and the 64 bytes
// of X it needs; the four MFMAs of a group use word j of every lane's chunk, and A
// is loaded with the same K-slot assignment.  Partial sums are reduced across the
// waves in LDS, then across split-K workgroups through the workspace by the last
// arriving workgroup, in a fixed order.
#include "kernels.hpp"

namespace w4 {

namespace {

constexpr int kRows = 64;      // output columns (weight rows) per workgroup
constexpr int kTargetBlocks = 512;

template <int MT>
struct GroupRegs {
  u32x4 b[4];         // packed codes: 4 words (32 k) for each of the 4 n-tiles
  half8_t a[MT][4];   // X fragments: MT m-tiles x 4 MFMAs
  float s[4];         // scale of this lane's row in each n-tile
  float c[4];         // 1024 + zero of this lane's row in each n-tile
};

// Loads are branch-free so that all of them are issued back to back: out-of-range rows
// (n >= N, m >= M) read a clamped, valid row and are zeroed by a select afterwards.
template <int MT>
__device__ __forceinline__ void load_group(GroupRegs<MT>& r, const half_t* __restrict__ x,
                                           const uint32_t* __restrict__ qweight,
                                           const half_t* __restrict__ scales,
                                           const uint32_t* __restrict__ qzeros, int g, int n0, int lane,
                                           int M, int N, int K) {
  const int wpr = K / 8;
  const int nzw = (N + 7) / 8;
  const int slot = lane >> 4;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = n0 + 16 * t + (lane & 15);
    const int nc = min(n, N - 1);
    r.b[t] = *reinterpret_cast<const u32x4*>(qweight + (int64_t)nc * wpr + g * 16 + slot * 4);
    r.s[t] = (float)scales[(int64_t)g * N + nc];
    r.c[t] = __builtin_bit_cast(float, qzeros[(int64_t)g * nzw + (nc >> 3)]);  // raw word, decoded later
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + (lane & 15), M - 1);
    const half8_t* src = reinterpret_cast<const half8_t*>(x + (int64_t)m * K + g * 128 + slot * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) r.a[mt][j] = src[j];
  }
}

// Zero out-of-range rows and decode the zero points (after the loads have landed).
template <int MT>
__device__ __forceinline__ void finish_group(GroupRegs<MT>& r, int n0, int lane, int M, int N) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = n0 + 16 * t + (lane & 15);
    const bool ok = n < N;
    const uint32_t zw = __builtin_bit_cast(uint32_t, r.c[t]);
    r.c[t] = ok ? (float)(1024u + ((zw >> (4 * (n & 7))) & 15u)) : 0.0f;
    r.s[t] = ok ? r.s[t] : 0.0f;
    if (!ok) r.b[t] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const bool ok = mt * 16 + (lane & 15) < M;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (!ok) r.a[mt][j] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

template <int MT>
__device__ __forceinline__ void compute_group(GroupRegs<MT>& r, float4_t (&yacc)[MT][4], int n0, int lane, int M,
                                              int N) {
  finish_group<MT>(r, n0, lane, M, N);
  const half8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};
  float4_t ssum[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    ssum[mt] = float4_t{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) ssum[mt] = mfma16(r.a[mt][j], ones, ssum[mt]);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    half8_t bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = unpack_1024(r.b[t][j]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float4_t tacc = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) tacc = mfma16(r.a[mt][j], bv[j], tacc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = fmaf(-r.c[t], ssum[mt][i], tacc[i]);
        yacc[mt][t][i] = fmaf(r.s[t], d, yacc[mt][t][i]);
      }
    }
  }
}

// WAVES waves per workgroup take the groups of the workgroup's K range round robin.
// Two register sets alternate (loop unrolled by two, no register copies), so while a
// wave computes one group the loads of its next two groups are in flight.
template <int MT, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void skinny_kernel(const half_t* __restrict__ x,
                                                               const uint32_t* __restrict__ qweight,
                                                               const half_t* __restrict__ scales,
                                                               const uint32_t* __restrict__ qzeros,
                                                               half_t* __restrict__ y,
                                                               unsigned* __restrict__ counters,
                                                               float* __restrict__ partials, int M, int N, int K,
                                                               int splits, int gps) {
  constexpr int kT = WAVES * kWave;
  constexpr int kOut = MT * 16 * kRows;  // outputs of one workgroup
  __shared__ float red[WAVES][MT * 16 * kWave];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rb = blockIdx.x;
  const int split = blockIdx.y;
  const int n0 = rb * kRows;
  const int ng = K / 128;
  const int gbeg = split * gps;
  const int gend = min(ng, gbeg + gps);

  float4_t yacc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) yacc[mt][t] = float4_t{0, 0, 0, 0};

  GroupRegs<MT> ra, rbuf;
  int g = gbeg + wave;
  if (g < gend) load_group<MT>(ra, x, qweight, scales, qzeros, g, n0, lane, M, N, K);
  if (g + WAVES < gend) load_group<MT>(rbuf, x, qweight, scales, qzeros, g + WAVES, n0, lane, M, N, K);
  for (; g < gend; g += 2 * WAVES) {
    compute_group<MT>(ra, yacc, n0, lane, M, N);
    if (g + 2 * WAVES < gend) load_group<MT>(ra, x, qweight, scales, qzeros, g + 2 * WAVES, n0, lane, M, N, K);
    if (g + WAVES >= gend) break;
    compute_group<MT>(rbuf, yacc, n0, lane, M, N);
    if (g + 3 * WAVES < gend) load_group<MT>(rbuf, x, qweight, scales, qzeros, g + 3 * WAVES, n0, lane, M, N, K);
  }

  // Cross-wave reduction.  Element (mt, t, i) of lane l is output row
  // m = 16 mt + 4 (l / 16) + i, column n = n0 + 16 t + (l % 16).
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][((mt * 4 + t) * 4 + i) * kWave + lane] = yacc[mt][t][i];
  __syncthreads();

  const int rows = min(M, MT * 16);
  // Walk the outputs with n fastest for coalesced stores.
  float vals[kOut / kT];
#pragma unroll
  for (int it = 0; it < kOut / kT; ++it) {
    const int o = it * kT + threadIdx.x;
    const int m = o / kRows, nl = o % kRows;
    const int t = nl >> 4, ln = nl & 15;
    const int mt = m >> 4, i = m & 3, lq = (m & 15) >> 2;
    const int idx = ((mt * 4 + t) * 4 + i) * kWave + lq * 16 + ln;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][idx];
    vals[it] = v;
  }

  if (splits == 1) {
#pragma unroll
    for (int it = 0; it < kOut / kT; ++it) {
      const int o = it * kT + threadIdx.x;
      const int m = o / kRows, n = n0 + o % kRows;
      if (m < rows && n < N) y[(int64_t)m * N + n] = (half_t)vals[it];
    }
    return;
  }

  // Split-K: publish fp32 partials, the last workgroup of this column block sums them.
#pragma unroll
  for (int it = 0; it < kOut / kT; ++it) {
    const int o = it * kT + threadIdx.x;
    const int m = o / kRows, n = n0 + o % kRows;
    if (m < rows && n < N) st_coherent(partials + ((int64_t)split * M + m) * N + n, vals[it]);
  }
  if (!splitk_arrive(counters + rb, splits)) return;
#pragma unroll
  for (int it = 0; it < kOut / kT; ++it) {
    const int o = it * kT + threadIdx.x;
    const int m = o / kRows, n = n0 + o % kRows;
    if (m < rows && n < N) {
      float s = 0.0f;
      for (int sp = 0; sp < splits; ++sp) s += ld_coherent(partials + ((int64_t)sp * M + m) * N + n);
      y[(int64_t)m * N + n] = (half_t)s;
    }
  }
}

}  // namespace

// Waves per workgroup: 8 for MT = 1, 4 for MT >= 2 (register budget of the two
// prefetch register sets, and LDS for the cross-wave reduction).
static int skinny_waves(int mt) { return mt == 1 ? 8 : 4; }

SkinnyPlan skinny_plan(int M, int N, int K) {
  SkinnyPlan p;
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.row_blocks = (N + kRows - 1) / kRows;
  const int ng = K / 128;
  const int waves = skinny_waves(p.mt);
  const int target = env_int("W4_SKINNY_BLOCKS", kTargetBlocks);
  const int min_gpw = env_int("W4_SKINNY_MIN_GROUPS_PER_WAVE", 1);
  int splits = (target + p.row_blocks - 1) / p.row_blocks;
  // at least min_gpw groups per wave
  splits = min(splits, ng / (waves * max(1, min_gpw)));
  // keep the split-K partial traffic (2 * splits * M * N * 4 bytes) near 10% of the codes
  // (N * K / 2 bytes): splits <= K / (160 M)
  const int pct = env_int("W4_SKINNY_PARTIAL_PCT", 10);
  splits = min(splits, max(1, (int)((int64_t)K * pct / (1600LL * M))));
  splits = max(1, splits);
  if (p.row_blocks >= kMaxCounters) splits = 1;
  p.gps = (ng + splits - 1) / splits;
  p.splits = (ng + p.gps - 1) / p.gps;
  return p;
}

size_t skinny_workspace_bytes(int M, int N, int K) {
  const SkinnyPlan p = skinny_plan(M, N, K);
  if (p.splits == 1) return 0;
  return kCounterRegionBytes + (size_t)p.splits * M * N * sizeof(float);
}

hipError_t launch_skinny(const void* x, const int32_t* qweight, const void* scales, const int32_t* qzeros,
                         void* y, void* ws, int M, int N, int K, hipStream_t stream) {
  const SkinnyPlan p = skinny_plan(M, N, K);
  unsigned* counters = (unsigned*)ws;
  float* partials = ws ? (float*)((char*)ws + kCounterRegionBytes) : nullptr;
  const dim3 grid(p.row_blocks, p.splits);
  const half_t* xh = (const half_t*)x;
  const uint32_t* qw = (const uint32_t*)qweight;
  const half_t* sc = (const half_t*)scales;
  const uint32_t* qz = (const uint32_t*)qzeros;
  half_t* yh = (half_t*)y;
#define SKINNY_LAUNCH(MT)                                                                                   \
  hipLaunchKernelGGL((skinny_kernel<MT, (MT == 1 ? 8 : 4)>), grid, dim3(skinny_waves(MT) * kWave), 0, stream, xh, \
                     qw, sc, qz, yh, counters, partials, M, N, K, p.splits, p.gps)
  if (p.mt == 1) SKINNY_LAUNCH(1);
  else if (p.mt == 2) SKINNY_LAUNCH(2);
  else SKINNY_LAUNCH(4);
#undef SKINNY_LAUNCH
  return hipGetLastError();
}

}  // namespace w4
