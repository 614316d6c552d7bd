// Large-M W4A16 GEMM (prefill): fp16 X tiles staged through LDS, packed int4 weights
// streamed from global memory straight into registers, dequantized exactly in
// registers (one fp16 rounding per element), fed to v_mfma_f32_32x32x16_f16 with fp32
// accumulation.
//
// "Implement AWQ quantization support for LLaMA" (vllm-project/vllm PR 1032): the AWQ
// GEMM runs dequantized fp16 weights through the tensor cores; dequantization is the
// tricky part and the rest is normal FP16 work.  On gfx950 the same split holds: the
// MFMA does the FP16 work; the dequantization (9 VALU ops to expand a word, 8 packed
// fp16 ops for (q - z) * s) is amortized over the 128 rows of a wave tile.
//
// Tile: BM x BN x BK = 128 x 256 x 64, 256 threads.  The 4 waves split N: wave w owns
// columns [64 w, 64 w + 64) as two 32-column MFMA fragments, and all 128 rows as four
// 32-row fragments (acc = 4 x 2 x 16 fp32 per lane).  Each weight code is therefore
// dequantized exactly once per workgroup.  Per BK step a lane loads one 16-byte chunk
// (4 words = 32 codes) per fragment: lane l (column l % 32, K-slot h = l / 32) takes
// words 4h..4h+3 of the 8 words of its row in this BK step, and k16-step s uses word
// s.  The X fragment for k16-step s is read from LDS with the same K-slot assignment
// (row l % 32, elements k = 8 (4h + s) .. + 7).  X rows live in LDS as 128-byte rows
// of 8 16-byte chunks, chunk c of row r stored at position c ^ (r % 8) so that the
// 32 rows read by one instruction hit distinct banks.
//
// Workgroups are remapped so that the tiles one XCD runs at a time form compact
// groups of 8 M-tiles (they share weight columns in that XCD's L2).  Split-K over BK
// steps is used when there are too few tiles to fill the 256 CUs; partials are summed
// by the last arriving workgroup in split order (deterministic).
#include "kernels.hpp"

namespace w4 {

namespace {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const half_t* __restrict__ x,
                                                            const uint32_t* __restrict__ qweight,
                                                            const half_t* __restrict__ scales,
                                                            const uint32_t* __restrict__ qzeros,
                                                            half_t* __restrict__ y, unsigned* __restrict__ counters,
                                                            float* __restrict__ partials, int M, int N, int K,
                                                            int tiles_m, int tiles_n, int splits, int kps) {
  __shared__ u32x4 lds[2][BM * 8];  // 2 x 16 KB

  const int total = tiles_m * tiles_n * splits;
  const int id = xcd_remap(blockIdx.x, total);
  const int tile = id / splits;
  const int split = id % splits;
  // grouped ordering: walk kGroupM M-tiles for each N-tile
  const int per_group = kGroupM * tiles_n;
  const int grp = tile / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_grp = tile % per_group;
  const int tm = first_m + in_grp % gsize;
  const int tn = in_grp / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int ktiles = K / BK;
  const int kbeg = split * kps;
  const int kend = min(ktiles, kbeg + kps);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int h = lane >> 5;
  const int wpr = K / 8;
  const int nzw = (N + 7) / 8;

  int nrow[2];
  bool nok[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    nrow[f] = n0 + wave * 64 + f * 32 + col;
    nok[f] = nrow[f] < N;
  }

  float16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  // global -> register staging of one X tile: 1024 chunks, 4 per thread.  Loads are
  // branch-free (rows past M read a clamped valid row, zeroed before the LDS store) so
  // they issue back to back.
  u32x4 areg[4];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cid = threadIdx.x + i * kThreads;
      const int r = cid >> 3, c = cid & 7;
      const int m = min(m0 + r, M - 1);
      areg[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)m * K + kt * BK + c * 8);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cid = threadIdx.x + i * kThreads;
      const int r = cid >> 3, c = cid & 7;
      lds[buf][swz(r, c)] = (m0 + r < M) ? areg[i] : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // Columns past N read a clamped valid row; their outputs are never stored.
  int nclamp[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) nclamp[f] = min(nrow[f], N - 1);
  u32x4 breg[2];
  auto load_b = [&](int kt, u32x4 (&dst)[2]) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
      dst[f] = *reinterpret_cast<const u32x4*>(qweight + (int64_t)nclamp[f] * wpr + kt * 8 + h * 4);
  };
  // Scale and zero point of this lane's rows for one 128-group: the raw words are
  // prefetched one BK step ahead together with the codes, then converted to the packed
  // fp16 pairs -(1024 + z) and s used by dequant8.
  uint32_t zraw[2];
  half_t sraw[2];
  auto load_sz = [&](int g, uint32_t (&zr)[2], half_t (&sr)[2]) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      zr[f] = qzeros[(int64_t)g * nzw + (nclamp[f] >> 3)];
      sr[f] = scales[(int64_t)g * N + nclamp[f]];
    }
  };
  half2_t negz2[2], s2[2];
  auto set_sz = [&](const uint32_t (&zr)[2], const half_t (&sr)[2]) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const uint32_t z = (zr[f] >> (4 * (nclamp[f] & 7))) & 15u;
      negz2[f] = splat2(-(half_t)(1024u + z));
      s2[f] = splat2(sr[f]);
    }
  };

  if (kbeg < kend) {
    load_a(kbeg);
    load_b(kbeg, breg);
    load_sz(kbeg >> 1, zraw, sraw);  // 2 BK steps per 128-group
    store_a(0);
    set_sz(zraw, sraw);
  }
  __syncthreads();

  for (int kt = kbeg; kt < kend; ++kt) {
    const int buf = (kt - kbeg) & 1;
    const bool more = kt + 1 < kend;
    const bool new_group = ((kt + 1) & 1) == 0;
    u32x4 bnext[2];
    if (more) {
      load_a(kt + 1);
      load_b(kt + 1, bnext);
      if (new_group) load_sz((kt + 1) >> 1, zraw, sraw);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t bf[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) bf[f] = dequant8(breg[f][s], negz2[f], s2[f]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 av = lds[buf][swz(i * 32 + col, h * 4 + s)];
        const half8_t a = __builtin_bit_cast(half8_t, av);
#pragma unroll
        for (int f = 0; f < 2; ++f) acc[i][f] = mfma32(a, bf[f], acc[i][f]);
      }
    }
    if (more) {
      store_a(buf ^ 1);
      breg[0] = bnext[0];
      breg[1] = bnext[1];
      if (new_group) set_sz(zraw, sraw);
    }
    __syncthreads();
  }

  // Output element (i, f, r): row m0 + 32 i + 8 (r / 4) + 4 h + (r % 4), column nrow[f].
  if (splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (!nok[f]) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m < M) y[(int64_t)m * N + nrow[f]] = (half_t)acc[i][f][r];
        }
      }
    return;
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (!nok[f]) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) st_coherent(partials + ((int64_t)split * M + m) * N + nrow[f], acc[i][f][r]);
      }
    }
  if (!splitk_arrive(counters + tile, splits)) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (!nok[f]) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) {
          float s = 0.0f;
          for (int sp = 0; sp < splits; ++sp) s += ld_coherent(partials + ((int64_t)sp * M + m) * N + nrow[f]);
          y[(int64_t)m * N + nrow[f]] = (half_t)s;
        }
      }
    }
}

}  // namespace

GemmPlan gemm_plan(int M, int N, int K) {
  GemmPlan p;
  p.tiles_m = (M + BM - 1) / BM;
  p.tiles_n = (N + BN - 1) / BN;
  const int ktiles = K / BK;
  const int tiles = p.tiles_m * p.tiles_n;
  const int target = env_int("W4_GEMM_SPLIT_TARGET", 256);
  int splits = 1;
  // fill the CUs when there are few tiles; keep >= 8 BK steps per split
  while (tiles * splits < target && ktiles / (splits * 2) >= 8) splits *= 2;
  if (tiles >= kMaxCounters) splits = 1;
  p.kt_per_split = (ktiles + splits - 1) / splits;
  p.splits = (ktiles + p.kt_per_split - 1) / p.kt_per_split;
  return p;
}

size_t gemm_workspace_bytes(int M, int N, int K) {
  const GemmPlan p = gemm_plan(M, N, K);
  if (p.splits == 1) return 0;
  return kCounterRegionBytes + (size_t)p.splits * M * N * sizeof(float);
}

hipError_t launch_gemm(const void* x, const int32_t* qweight, const void* scales, const int32_t* qzeros,
                       void* y, void* ws, int M, int N, int K, hipStream_t stream) {
  const GemmPlan p = gemm_plan(M, N, K);
  unsigned* counters = (unsigned*)ws;
  float* partials = ws ? (float*)((char*)ws + kCounterRegionBytes) : nullptr;
  const int blocks = p.tiles_m * p.tiles_n * p.splits;
  hipLaunchKernelGGL(gemm_kernel, dim3(blocks), dim3(kThreads), 0, stream, (const half_t*)x,
                     (const uint32_t*)qweight, (const half_t*)scales, (const uint32_t*)qzeros, (half_t*)y, counters,
                     partials, M, N, K, p.tiles_m, p.tiles_n, p.splits, p.kt_per_split);
  return hipGetLastError();
}

}  // namespace w4
