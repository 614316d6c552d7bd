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
// Work split: a workgroup (4 waves) owns 16 T output columns n (T = 1, 2 or 4 tiles of 16)
// and a contiguous range of K groups (split-K across workgroups only for narrow N); its
// waves take the groups of that range round robin.  Per group, lane l of a wave loads
// one 16-byte chunk (32 codes) of row n0 + 16t + (l % 16) for each tile t -- with the tiled
// weight layout the 64 lanes read one contiguous 1 KB block -- and the 64 bytes of X
// it needs; the four MFMAs of a group use word j of every lane's chunk, and A is
// loaded with the same K-slot assignment.  Partial sums are reduced across the
// waves in LDS, then across split-K workgroups through the workspace by the last
// arriving workgroup, in a fixed order.
#include "kernels.hpp"

namespace w4 {

namespace {


template <int MT, int T>
struct GroupRegs {
  u32x4 b[T];         // packed codes: 4 words (32 k) for each of the T n-tiles
  half8_t a[MT][4];   // X fragments: MT m-tiles x 4 MFMAs
  half_t s[T];        // scale of this lane's row in each n-tile (raw fp16; converted at use)
  uint32_t zw[T];     // packed zero-point word holding this lane's row in each n-tile
};

// Loads are branch-free so that all of them are issued back to back: out-of-range rows
// (n >= N, m >= M) read a clamped, valid row.  Nothing needs zeroing: an MFMA output
// row depends only on its own A row and an output column only on its own B column
// (and scale / zero point), so clamped data only reaches outputs that are never
// stored.
template <int MT, int T>
__device__ __forceinline__ void load_group(GroupRegs<MT, T>& r, const half_t* __restrict__ x,
                                           const uint32_t* __restrict__ qweight,
                                           const half_t* __restrict__ scales,
                                           const uint32_t* __restrict__ qzeros, int g, int n0, int lane,
                                           int M, int N, int K) {
  const int ng = K / 128;
  const int nzw = (N + 7) / 8;
  const int slot = lane >> 4;
  const int last_tile = (N - 1) >> 4;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int nc = min(n0 + 16 * t + (lane & 15), N - 1);
    // tiled layout: lane l reads chunk l of the 1 KB block (16 rows x 128 k) -- row
    // l % 16 of the tile, words 4 (l / 16) .. + 3 of the group
    const int tile = min((n0 >> 4) + t, last_tile);
    r.b[t] = *reinterpret_cast<const u32x4*>(qweight + ((int64_t)tile * ng + g) * 256 + lane * 4);
    r.s[t] = scales[(int64_t)g * N + nc];
    r.zw[t] = qzeros[(int64_t)g * nzw + (nc >> 3)];
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + (lane & 15), M - 1);
    const half8_t* src = reinterpret_cast<const half8_t*>(x + (int64_t)m * K + g * 128 + slot * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) r.a[mt][j] = src[j];
  }
}

template <int MT, int T>
__device__ __forceinline__ void compute_group(const GroupRegs<MT, T>& r, float4_t (&yacc)[MT][T], int n0, int lane,
                                              int N) {
  float c[T];  // 1024 + zero point of this lane's row in each n-tile
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int nc = min(n0 + 16 * t + (lane & 15), N - 1);
    c[t] = (float)(1024u + ((r.zw[t] >> (4 * (nc & 7))) & 15u));
  }
  const half8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};
  float4_t ssum[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    ssum[mt] = float4_t{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) ssum[mt] = mfma16(r.a[mt][j], ones, ssum[mt]);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
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
        const float d = fmaf(-c[t], ssum[mt][i], tacc[i]);
        yacc[mt][t][i] = fmaf((float)r.s[t], d, yacc[mt][t][i]);
      }
    }
  }
}

// WAVES waves per workgroup take the groups of the workgroup's K range round robin.
// D register sets rotate (loop unrolled by D, no register copies), so while a wave
// computes one group the loads of its next D groups are in flight (D * T KB per wave).
// A workgroup owns 16 T output columns (T 16-row tiles; all its waves share them).
template <int MT, int T, int D, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void skinny_kernel(const half_t* __restrict__ x,
                                                               const uint32_t* __restrict__ qweight,
                                                               const half_t* __restrict__ scales,
                                                               const uint32_t* __restrict__ qzeros,
                                                               half_t* __restrict__ y,
                                                               unsigned* __restrict__ counters,
                                                               float* __restrict__ partials, int M, int N, int K,
                                                               int splits, int gps) {
  constexpr int kT = WAVES * kWave;
  constexpr int kCols = 16 * T;           // output columns of one workgroup
  constexpr int kOut = MT * 16 * kCols;   // outputs of one workgroup
  constexpr int kPer = kOut / kT;         // outputs per thread in the epilogue (MT * T)
  __shared__ float red[WAVES][MT * T * 4 * kWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int rb = blockIdx.x;
  const int split = blockIdx.y;
  const int n0 = rb * kCols;
  const int ng = K / 128;
  const int gbeg = split * gps;
  const int gend = min(ng, gbeg + gps);

  float4_t yacc[MT][T];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t) yacc[mt][t] = float4_t{0, 0, 0, 0};

  // Prefetches are issued unconditionally (a group index past the range is clamped to
  // the last valid group and its data is never used): with no conditional loads in the
  // loop, the waits before each compute only cover the group being computed.
  GroupRegs<MT, T> r[D];
  const int glast = gend - 1;
  int g = gbeg + wave;
  if (g < gend) {
#pragma unroll
    for (int d = 0; d < D; ++d)
      load_group<MT, T>(r[d], x, qweight, scales, qzeros, min(g + d * WAVES, glast), n0, lane, M, N, K);
  }
  for (; g < gend; g += D * WAVES) {
    bool done = false;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (!done) {
        compute_group<MT, T>(r[d], yacc, n0, lane, N);
        load_group<MT, T>(r[d], x, qweight, scales, qzeros, min(g + (d + D) * WAVES, glast), n0, lane, M, N, K);
        done = g + (d + 1) * WAVES >= gend;  // wave-uniform
      }
    }
    if (done) break;
  }

  // Cross-wave reduction.  Element (mt, t, i) of lane l is output row
  // m = 16 mt + 4 (l / 16) + i, column n = n0 + 16 t + (l % 16).
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][((mt * T + t) * 4 + i) * kWave + lane] = yacc[mt][t][i];
  __syncthreads();

  const int rows = min(M, MT * 16);
  // Walk the outputs with n fastest for coalesced stores.
  float vals[kPer];
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int o = it * kT + threadIdx.x;
    const int m = o / kCols, nl = o % kCols;
    const int t = nl >> 4, ln = nl & 15;
    const int mt = m >> 4, i = m & 3, lq = (m & 15) >> 2;
    const int idx = ((mt * T + t) * 4 + i) * kWave + lq * 16 + ln;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][idx];
    vals[it] = v;
  }

  if (splits == 1) {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int o = it * kT + threadIdx.x;
      const int m = o / kCols, n = n0 + o % kCols;
      if (m < rows && n < N) y[(int64_t)m * N + n] = (half_t)vals[it];
    }
    return;
  }

  // Split-K: publish fp32 partials, the last workgroup of this column block sums them.
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int o = it * kT + threadIdx.x;
    const int m = o / kCols, n = n0 + o % kCols;
    if (m < rows && n < N) st_coherent(partials + ((int64_t)split * M + m) * N + n, vals[it]);
  }
  if (!splitk_arrive(counters + rb, splits)) return;
  // Last workgroup: sum in split order (its own partial from registers); splits outer,
  // outputs inner, so the loads of one split are all in flight at once.
  float sum[kPer];
#pragma unroll
  for (int it = 0; it < kPer; ++it) sum[it] = 0.0f;
  for (int sp = 0; sp < splits; ++sp) {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int o = it * kT + threadIdx.x;
      const int m = min(o / kCols, rows - 1), n = min(n0 + o % kCols, N - 1);
      sum[it] += sp == split ? vals[it] : ld_coherent(partials + ((int64_t)sp * M + m) * N + n);
    }
  }
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int o = it * kT + threadIdx.x;
    const int m = o / kCols, n = n0 + o % kCols;
    if (m < rows && n < N) y[(int64_t)m * N + n] = (half_t)sum[it];
  }
}

}  // namespace

// Waves per workgroup: 4.  At ~190 VGPRs two 4-wave workgroups fit per CU, so grids of
// up to ~512 workgroups are resident at once (no second, partly idle round).
static int skinny_waves(int) { return 4; }

// Columns per workgroup (16 T) and split-K.  Split-K costs a serial tail (partial
// stores, arrival counter, reads of the partials by the last workgroup), so the plan
// first narrows the workgroups: the widest T in {4, 2, 1} that still gives at least
// kMinBlocks workgroups; only when even T = 1 does not (N < 16 kMinBlocks) is K split.
SkinnyPlan skinny_plan(int M, int N, int K) {
  SkinnyPlan p;
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  const int ng = K / 128;
  const int waves = skinny_waves(p.mt);
  // Tiles per workgroup.  With few rows of X (M <= 4) the narrowest tiles that still
  // give enough workgroups avoid split-K; with more rows each X fragment should serve
  // several tiles (X traffic is 4 M / T bytes per weight byte), so T >= 2.
  int t = env_int("W4_SKINNY_TILES", 0);
  if (t != 1 && t != 2 && t != 4) {
    if (M <= 4) t = (N <= 16 * 320) ? 1 : ((N <= 32 * 480) ? 2 : 4);
    else t = ((N + 63) / 64 >= 128) ? 4 : 2;
  }
  p.tiles = t;
  p.depth = t == 1 ? 4 : 2;
  p.row_blocks = (N + 16 * t - 1) / (16 * t);
  const int target = env_int("W4_SKINNY_BLOCKS", 320);
  int splits = (target + p.row_blocks - 1) / p.row_blocks;
  splits = min(splits, ng / waves);  // at least one group per wave
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
#define SKINNY_LAUNCH(MT, T, D)                                                                          \
  hipLaunchKernelGGL((skinny_kernel<MT, T, D, 4>), grid, dim3(4 * kWave), 0, stream, xh, qw, sc, qz, yh, counters, \
                     partials, M, N, K, p.splits, p.gps)
#define SKINNY_LAUNCH_T(MT)                    \
  if (p.tiles == 4) SKINNY_LAUNCH(MT, 4, 2);   \
  else if (p.tiles == 2) SKINNY_LAUNCH(MT, 2, 2); \
  else SKINNY_LAUNCH(MT, 1, 4)
  if (p.mt == 1) { SKINNY_LAUNCH_T(1); }
  else if (p.mt == 2) { SKINNY_LAUNCH_T(2); }
  else { SKINNY_LAUNCH_T(4); }
#undef SKINNY_LAUNCH_T
#undef SKINNY_LAUNCH
  return hipGetLastError();
}

}  // namespace w4
