// Large-M W4A16 GEMM (prefill and mid M): fp16 X tiles staged through LDS, packed int4
// weights streamed from global memory into registers (or through an LDS ring, each lane
// reading back its own chunk), dequantized exactly in registers (one fp16 rounding per
// element), fed to v_mfma_f32_32x32x16_f16 with fp32 accumulation.  The loop variants
// (register-staged, or direct-to-LDS rings of 3, 4 or 6 steps) are described at each
// branch below and chosen per shape in gemm_plan.
//
// "Implement AWQ quantization support for LLaMA" (vllm-project/vllm PR 1032): the AWQ
// GEMM runs dequantized fp16 weights through the tensor cores; dequantization is the
// tricky part and the rest is normal FP16 work.  On gfx950 the same split holds: the
// MFMA does the FP16 work; the dequantization is amortized over the 128 rows of a wave
// tile.  A parity-split word is expanded in natural k order in 5 VALU ops to fp16
// (1024 + q) at k = 0, 1 mod 4 (code in the low mantissa bits under exponent 2^10) and
// (64 + q) at k = 2, 3 mod 4 (code in mantissa bits 4..7 under exponent 2^6);
// subtracting 1024 + z or 64 + z is exact, and the multiply by s is the element's single
// fp16 rounding (4 packed adds, 4 packed multiplies).  X stays in natural order.
//
// Tile: BM x BN x BK = (32 MI) x (128 NF) x 64, 256 threads, (MI, NF) in {4, 2} x {2, 1}.
// The 4 waves split N: wave w owns 32 NF columns as NF 32-column MFMA fragments, and
// all BM rows as MI 32-row fragments (acc = MI x NF x 16 fp32 per lane).  Each weight
// code is therefore dequantized exactly once per workgroup.  Per BK step a lane loads
// one 16-byte chunk (4 words = 32 codes) per fragment: lane l (column l % 32, K-slot
// h = l / 32) takes words 4h..4h+3 of the 8 words of its row in this BK step (slot
// 2 (kt % 2) + h of the tiled layout: 16 lanes read 256 contiguous bytes), and k16-step
// s uses word s.  The X fragment for k16-step s is read from LDS with the same K-slot assignment
// (row l % 32, elements k = 8 (4h + s) .. + 7).  X rows live in LDS as 128-byte rows
// of 8 16-byte chunks, chunk c of row r stored at position c ^ ((r / 2) % 8): two
// consecutive rows fill one 256-byte bank window, so any 16 consecutive rows read at
// the same chunk hit 16 distinct 16-byte bank groups.
//
// Workgroups are remapped so that the tiles one XCD runs at a time form compact
// groups of 8 M-tiles (they share weight columns in that XCD's L2).  Smaller tiles are
// chosen before split-K when M or N is small; split-K over BK steps remains for grids
// that are still too small, with partials summed by the last arriving workgroup in
// split order (deterministic).
#include "kernels.hpp"

namespace w4 {

namespace {

constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kRing = 4;  // X tiles in flight in the direct-to-LDS pipeline

// s_waitcnt immediate (gfx9 encoding) that waits until at most n (< 64) vector-memory
// operations are outstanding and leaves the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

// Tile BM x BN = (32 MI) x (128 NF): wave w owns columns [32 NF w, 32 NF (w + 1)) as NF
// 32-column fragments and all BM rows as MI 32-row fragments.
template <int MI, int NF, int PD>
__global__ __launch_bounds__(kThreads, PD == 0 ? 1 : 2) void gemm_kernel(const half_t* __restrict__ x,
                                                            const uint32_t* __restrict__ qweight,
                                                            const half_t* __restrict__ scales,
                                                            const uint32_t* __restrict__ qzeros,
                                                            half_t* __restrict__ y, unsigned* __restrict__ counters,
                                                            float* __restrict__ partials, int M, int N, int K,
                                                            int tiles_m, int tiles_n, int splits, int kps,
                                                            int glog, int n_full, int tail_splits) {
  constexpr int BM = 32 * MI, BN = 128 * NF;
  constexpr int kAPer = BM * 8 / kThreads;  // 16-byte X chunks per thread per BK step
  // PD == 0: X goes global -> LDS directly into a ring of kRing tiles (separate arrays,
  // see below); otherwise two register-staged buffers
  constexpr bool kDma = PD == 0 || PD == 5 || PD == 7 || PD == 8;
  constexpr bool kBLds = PD == 7 || PD == 8;  // the packed weights too go through LDS
  __shared__ u32x4 lds[kDma ? 1 : 2][kDma ? 1 : BM * 8];

  const int ktiles = K / BK;
  // Work item of this workgroup.  Uniform mode (tail_splits == 0): every tile split
  // `splits` ways over its BK steps.  Tail mode: workgroups [0, n_full) take tiles
  // 0 .. n_full - 1 whole, the rest take the remaining tiles split tail_splits ways; each
  // range is remapped for the XCDs on its own, so every XCD gets the same mix.
  int tile, split, nsplit, kpl;
  if (tail_splits == 0) {
    const int id = xcd_remap(blockIdx.x, tiles_m * tiles_n * splits);
    tile = id / splits;
    split = id % splits;
    nsplit = splits;
    kpl = kps;
  } else if ((int)blockIdx.x < n_full) {
    tile = xcd_remap(blockIdx.x, n_full);
    split = 0;
    nsplit = 1;
    kpl = ktiles;
  } else {
    const int j = xcd_remap(blockIdx.x - n_full, gridDim.x - n_full);
    tile = n_full + j / tail_splits;
    split = j % tail_splits;
    nsplit = tail_splits;
    kpl = (ktiles + tail_splits - 1) / tail_splits;
  }
  // grouped ordering: walk kGroupM M-tiles for each N-tile
  const int per_group = kGroupM * tiles_n;
  const int grp = tile / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_grp = tile % per_group;
  const int tm = first_m + in_grp % gsize;
  const int tn = in_grp / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbeg = split * kpl;
  const int kend = min(ktiles, kbeg + kpl);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int col = lane & 31;
  const int h = lane >> 5;
  const int nzw = (N + 7) / 8;
  const int ng = K / 128;

  int nrow[NF], nclamp[NF];
  bool nok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    nrow[f] = n0 + wave * 32 * NF + f * 32 + col;
    nok[f] = nrow[f] < N;
    // columns past N read a clamped valid row; their outputs are never stored
    nclamp[f] = min(nrow[f], N - 1);
  }

  float16_t acc[MI][NF];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  if constexpr (kDma) {
  // Direct-to-LDS pipeline.  The X tile of BK step t lands in LDS slot t % R straight
  // from global memory (global_load_lds_dwordx4: no registers, no VALU), issued R - 1
  // steps ahead; this lane's weight chunks (in register set t % R, or with PD 7 / 8 in
  // LDS slot t % R of a second ring) and raw scale / zero-point words of step t are
  // issued as far ahead.  Each step: wait until the loads of step t are complete (every
  // step issues the same kPerStage loads per thread, so that is "at most (R - 2)
  // kPerStage loads outstanding"), barrier (every wave's part of the tile is in LDS, and
  // every wave is done with the slot and set of step t - 1), issue step t + R - 1's loads
  // into that freed slot and set, then the MFMAs of step t.  Loads past the last step are
  // clamped to it (they refill slots no later step reads), so the counts stay uniform.
  //
    // ring of R tiles: 4 with one workgroup per CU (PD 0); 3 with two (PD 5: weights in
    // registers; PD 7: weights in LDS); 6 with two for 64-row tiles (PD 8, weights in LDS)
    constexpr int R = (PD == 5 || PD == 7) ? 3 : PD == 8 ? 6 : kRing;
    constexpr int kPerStage = kAPer + 3 * NF;  // vector-memory instructions per thread per step
    constexpr int kWaitImm = vmcnt_imm((R - 2) * kPerStage);
    // thread's chunk i of a tile lands at LDS position (4 i + wave) * 64 + lane (each wave
    // instruction writes 1 KB contiguously) and must hold the X chunk that the swizzle puts
    // there: row r = P / 8, k-chunk (P % 8) ^ ((r / 2) % 8)
    // (element offsets fit 32 bits: the plan takes this pipeline only for M K < 2^31)
    uint32_t xoff[kAPer];
  #pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int pos = (4 * i + wave) * 64 + lane;
      const int r = pos >> 3, c = (pos & 7) ^ ((r >> 1) & 7);
      xoff[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + (uint32_t)(c * 8);
    }
    // One LDS array per ring slot: the compiler's wait insertion tells direct-to-LDS loads
    // into distinct arrays apart, so reading slot t does not wait for the loads in flight
    // into the other slots (with one array it waited for all of them).
    constexpr int kA45 = R > 4 ? BM * 8 : 1;
    __shared__ u32x4 ring0[BM * 8], ring1[BM * 8], ring2[BM * 8], ring3[BM * 8], ring4[kA45], ring5[kA45];
    auto ring = [&](int j) -> u32x4* {
      return j == 0 ? ring0 : j == 1 ? ring1 : j == 2 ? ring2 : j == 3 ? ring3 : j == 4 ? ring4 : ring5;
    };
    // PD 7: this lane's weight chunks of step t land in LDS slot t % R at position
    // (4 f + wave) * 64 + lane (each wave instruction writes 1 KB contiguously) and are read
    // back by the same lane: no registers held for them while in flight
    constexpr int kBSlot = kBLds ? NF * 4 * 64 : 1;
    constexpr int kB35 = R > 3 ? kBSlot : 1;
    __shared__ u32x4 bring0[kBSlot], bring1[kBSlot], bring2[kBSlot], bring3[kB35], bring4[kB35], bring5[kB35];
    auto bring = [&](int j) -> u32x4* {
      return j == 0 ? bring0 : j == 1 ? bring1 : j == 2 ? bring2 : j == 3 ? bring3 : j == 4 ? bring4 : bring5;
    };
    struct BSet {
      u32x4 b[kBLds ? 1 : NF];
      uint32_t z[NF], s[NF];
    };
    BSet bs[R];
    const uint16_t* sbits = reinterpret_cast<const uint16_t*>(scales);
    // Every address of step kt is a wave-uniform base (scalar registers) plus a per-lane
    // 32-bit offset fixed for the whole loop, so no per-lane 64-bit address arithmetic is
    // left in the loop (the plan takes these pipelines only while the offsets fit):
    //  * codes: the chunk of (row n, group kt / 2, slot 2 (kt % 2) + h) is word
    //    tiled_chunk(n, 0, h) + 128 kt;
    //  * scale / zero point: row (64 kt + 32 h) >> glog of [K/G, .] = (64 kt) >> glog, plus
    //    h for G = 32 (this lane's 32 k of a BK step lie in one group for G >= 32).
    uint32_t boff[NF], zoff[NF], soff[NF];
    const int hrow = glog == 5 ? h : 0;
  #pragma unroll
    for (int f = 0; f < NF; ++f) {
      boff[f] = (uint32_t)tiled_chunk(nclamp[f], 0, h, ng);
      zoff[f] = (uint32_t)(hrow * nzw + (nclamp[f] >> 3));
      soff[f] = (uint32_t)(hrow * N + nclamp[f]);
    }
    auto issue = [&](int kt, int slot, BSet& S) {
      const uint32_t* qw_kt = qweight + (int64_t)kt * 128;
  #pragma unroll
      for (int f = 0; f < NF; ++f) {
        const uint32_t* src = qw_kt + boff[f];
        if constexpr (kBLds)
          __builtin_amdgcn_global_load_lds((void*)src,
                                           (__attribute__((address_space(3))) void*)(bring(slot) + (4 * f + wave) * 64),
                                           16, 0, 0);
        else
          S.b[f] = *reinterpret_cast<const u32x4*>(src);
      }
      const int64_t row = (int64_t)((kt * BK) >> glog);
      const uint32_t* qz_kt = qzeros + row * nzw;
      const uint16_t* sc_kt = sbits + row * N;
  #pragma unroll
      for (int f = 0; f < NF; ++f) {
        S.z[f] = qz_kt[zoff[f]];
        S.s[f] = sc_kt[soff[f]];
      }
      const half_t* x_kt = x + kt * BK;
  #pragma unroll
      for (int i = 0; i < kAPer; ++i)
        __builtin_amdgcn_global_load_lds((void*)(x_kt + xoff[i]),
                                         (__attribute__((address_space(3))) void*)(ring(slot) + (4 * i + wave) * 64), 16, 0,
                                         0);
    };
    const Magic mc = magic_regs();
    auto step = [&](int t, int j) {
      __builtin_amdgcn_s_waitcnt(kWaitImm);
      __builtin_amdgcn_s_barrier();
      // nothing that reads this step's registers may be scheduled above the wait (the
      // compiler's own wait for such a read drains every load in flight)
      __builtin_amdgcn_sched_barrier(0);
      issue(min(t + R - 1, kend - 1), (j + R - 1) % R, bs[(j + R - 1) % R]);
      const BSet& S = bs[j];
      u32x4 bw[NF];
  #pragma unroll
      for (int f = 0; f < NF; ++f) {
        if constexpr (kBLds) bw[f] = bring(j)[(4 * f + wave) * 64 + lane];
        else bw[f] = S.b[f];
      }
      half2_t c1024[NF], c64[NF], s2[NF];
  #pragma unroll
      for (int f = 0; f < NF; ++f) {
        const uint32_t z = (S.z[f] >> (4 * (nclamp[f] & 7))) & 15u;
        c1024[f] = neg1024z2(z);
        c64[f] = neg64z2(z);
        s2[f] = scale2(S.s[f]);
      }
      const u32x4* xa = ring(j);
      // A fragments of k16 steps s (in use) and s + 1 (in flight) with one wave per SIMD;
      // with two, the other wave covers the LDS latency and the registers are short
      constexpr bool kAhead = PD == 0;
      half8_t afr[2][MI];
      if (kAhead) {
  #pragma unroll
        for (int i = 0; i < MI; ++i) afr[0][i] = __builtin_bit_cast(half8_t, xa[swz(i * 32 + col, h * 4)]);
      }
  #pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (kAhead && s < 3) {
  #pragma unroll
          for (int i = 0; i < MI; ++i)
            afr[(s + 1) & 1][i] = __builtin_bit_cast(half8_t, xa[swz(i * 32 + col, h * 4 + s + 1)]);
        }
        if (!kAhead) {
  #pragma unroll
          for (int i = 0; i < MI; ++i) afr[s & 1][i] = __builtin_bit_cast(half8_t, xa[swz(i * 32 + col, h * 4 + s)]);
        }
        half8_t bf[NF];
  #pragma unroll
        for (int f = 0; f < NF; ++f) bf[f] = dequant8(bw[f][s], mc, c1024[f], c64[f], s2[f]);
  #pragma unroll
        for (int i = 0; i < MI; ++i)
  #pragma unroll
          for (int f = 0; f < NF; ++f) acc[i][f] = mfma32(afr[s & 1][i], bf[f], acc[i][f]);
      }
      if constexpr (PD == 8) {
        // 64 x 128 tiles: the step's A and weight reads first, then every MFMA followed by
        // three VALU operations and every other one by an LDS read, so the dequantization
        // of the next k16 step runs under the MFMAs of this one (K = 5120, N = 13824 at
        // M = 48 / 64 / 96 / 128: 22.6 / 23.2 / 30.8 / 30.8 -> 21.7 / 22.5 / 29.3 /
        // 30.0 us; on the 128-row tiles the same order, or the compiler's own interleaving
        // strategies, was slower)
        __builtin_amdgcn_sched_group_barrier(0x100, 2 + MI, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);      // VALU
  #pragma unroll
        for (int q = 0; q < 4 * MI * NF; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          if (q % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    };
    const int nsteps = kend - kbeg;
    if (nsteps > 0) {
  #pragma unroll
      for (int d = 0; d < R - 1; ++d) issue(min(kbeg + d, kend - 1), d, bs[d]);
      int it = 0;
      for (; it + R <= nsteps; it += R) {
  #pragma unroll
        for (int j = 0; j < R; ++j) step(kbeg + it + j, j);
      }
  #pragma unroll
      for (int j = 0; j < R; ++j)
        if (it + j < nsteps) step(kbeg + it + j, j);
      // no LDS write may still be in flight when the workgroup's LDS is released
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
  } else if constexpr (PD == 1) {
  // PD == 1: the next step's loads are issued at the top of each step (one set of X
  // registers, short lifetimes: the 128 x 256 tile fits two workgroups per CU).
    // global -> register staging of one X tile (BM x 64 halves).  Loads are branch-free
    // so they issue back to back: rows past M read a clamped valid row (it only reaches
    // output rows that are never stored).
    u32x4 areg[kAPer];
    auto load_a = [&](int kt) {
  #pragma unroll
      for (int i = 0; i < kAPer; ++i) {
        const int cid = threadIdx.x + i * kThreads;
        const int r = cid >> 3, c = cid & 7;
        const int m = min(m0 + r, M - 1);
        areg[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)m * K + kt * BK + c * 8);
      }
    };
    auto store_a = [&](int buf) {
  #pragma unroll
      for (int i = 0; i < kAPer; ++i) {
        const int cid = threadIdx.x + i * kThreads;
        lds[buf][swz(cid >> 3, cid & 7)] = areg[i];
      }
    };
    u32x4 breg[NF];
    auto load_b = [&](int kt, u32x4 (&dst)[NF]) {
      // BK step kt is half of group kt / 2: slot 2 (kt % 2) + h of the tiled layout
  #pragma unroll
      for (int f = 0; f < NF; ++f)
        dst[f] = *reinterpret_cast<const u32x4*>(qweight + tiled_chunk(nclamp[f], kt >> 1, (kt & 1) * 2 + h, ng));
    };
    // Scale and zero point of this lane's rows for its group: the raw words are prefetched
    // one BK step ahead together with the codes, then converted (every step, so that the
    // loads are consumed unconditionally and stay with the prefetch) to the packed fp16
    // pairs -(1024 + z), -(64 + z) and s, built as bit patterns: -(1024 + z) is 0xE400 | z
    // (unit steps at 2^10), -(64 + z) is 0xD400 | 16 z (steps of 1/16 at 2^6).
    uint32_t zraw[NF], sraw[NF];
    const uint16_t* sbits = reinterpret_cast<const uint16_t*>(scales);
    auto load_sz = [&](int kt) {
      // this lane's k range in BK step kt is kt * 64 + 32 h .. + 31: one group for G >= 32
      const int64_t row = (int64_t)((kt * BK + 32 * h) >> glog);
  #pragma unroll
      for (int f = 0; f < NF; ++f) {
        zraw[f] = qzeros[row * nzw + (nclamp[f] >> 3)];
        sraw[f] = sbits[row * N + nclamp[f]];
      }
    };
    half2_t c1024[NF], c64[NF], s2[NF];
    auto set_sz = [&]() {
  #pragma unroll
      for (int f = 0; f < NF; ++f) {
        const uint32_t z = (zraw[f] >> (4 * (nclamp[f] & 7))) & 15u;
        c1024[f] = __builtin_bit_cast(half2_t, (0xE400u | z) * 0x00010001u);
        c64[f] = __builtin_bit_cast(half2_t, (0xD400u | (z << 4)) * 0x00010001u);
        s2[f] = __builtin_bit_cast(half2_t, sraw[f] * 0x00010001u);
      }
    };
    const Magic mc = magic_regs();

    if (kbeg < kend) {
      load_a(kbeg);
      load_b(kbeg, breg);
      load_sz(kbeg);
      store_a(0);
      set_sz();
    }
    __syncthreads();

    // The next step's loads are issued unconditionally (clamped to the last step on the
    // final iteration) so that no load sits in a conditional block and the waits before
    // the MFMAs cover only what they consume.
    for (int kt = kbeg; kt < kend; ++kt) {
      const int buf = (kt - kbeg) & 1;
      const int kn = min(kt + 1, kend - 1);
      u32x4 bnext[NF];
      load_a(kn);
      load_b(kn, bnext);
      load_sz(kn);
      // keep these loads here, ahead of the MFMAs (the scheduler would otherwise sink them
      // next to their use at the end of the step and expose the full memory latency)
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int s = 0; s < 4; ++s) {
        half8_t bf[NF];
  #pragma unroll
        for (int f = 0; f < NF; ++f) bf[f] = dequant8(breg[f][s], mc, c1024[f], c64[f], s2[f]);
  #pragma unroll
        for (int i = 0; i < MI; ++i) {
          const u32x4 av = lds[buf][swz(i * 32 + col, h * 4 + s)];
          const half8_t a = __builtin_bit_cast(half8_t, av);
  #pragma unroll
          for (int f = 0; f < NF; ++f) acc[i][f] = mfma32(a, bf[f], acc[i][f]);
        }
      }
      store_a(buf ^ 1);  // the other buffer was last read before the previous barrier
  #pragma unroll
      for (int f = 0; f < NF; ++f) breg[f] = bnext[f];
      set_sz();
      __syncthreads();
    }
  } else {
  // PD >= 2: PD register sets rotate; loads run PD - 1 steps ahead of their use
  // (small tiles at mid M, where one step of compute does not hide the latency).
    // One BK step's loads: the X tile (BM x 64 halves, staged to LDS at the end of the
    // previous step), this lane's weight chunks and the raw scale / zero-point words.
    // Loads are branch-free so they issue back to back: rows past M read a clamped valid
    // row (it only reaches output rows that are never stored).
    struct Stage {
      u32x4 a[kAPer];
      u32x4 b[NF];
      uint32_t z[NF], s[NF];
    };
    const uint16_t* sbits = reinterpret_cast<const uint16_t*>(scales);
    auto issue = [&](int kt, Stage& S) {
  #pragma unroll
      for (int i = 0; i < kAPer; ++i) {
        const int cid = threadIdx.x + i * kThreads;
        const int r = cid >> 3, c = cid & 7;
        const int m = min(m0 + r, M - 1);
        S.a[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)m * K + kt * BK + c * 8);
      }
      // BK step kt is half of group kt / 2: slot 2 (kt % 2) + h of the tiled layout
  #pragma unroll
      for (int f = 0; f < NF; ++f)
        S.b[f] = *reinterpret_cast<const u32x4*>(qweight + tiled_chunk(nclamp[f], kt >> 1, (kt & 1) * 2 + h, ng));
      // this lane's k range in BK step kt is kt * 64 + 32 h .. + 31: one group for G >= 32
      const int64_t row = (int64_t)((kt * BK + 32 * h) >> glog);
  #pragma unroll
      for (int f = 0; f < NF; ++f) {
        S.z[f] = qzeros[row * nzw + (nclamp[f] >> 3)];
        S.s[f] = sbits[row * N + nclamp[f]];
      }
    };
    auto store_a = [&](const Stage& S, int buf) {
  #pragma unroll
      for (int i = 0; i < kAPer; ++i) {
        const int cid = threadIdx.x + i * kThreads;
        lds[buf][swz(cid >> 3, cid & 7)] = S.a[i];
      }
    };
    const Magic mc = magic_regs();
    // One BK step t on register set `cur` (B, scales, zero points) and LDS buffer
    // (t - kbeg) & 1 (its X tile); then the X tile of step t + 1 (set `nxt`) goes to the
    // other buffer, and after the barrier set `cur` is refilled with step t + PD's loads
    // (clamped to the last step: no conditional loads, so every wait covers only what it
    // consumes).  The scale and zero point become the packed fp16 pairs -(1024 + z),
    // -(64 + z) and s, built as bit patterns: -(1024 + z) is 0xE400 | z (unit steps at
    // 2^10), -(64 + z) is 0xD400 | 16 z (steps of 1/16 at 2^6).
    Stage st[PD];
    auto step = [&](int t, Stage& S, const Stage& Snext) {
      const int buf = (t - kbeg) & 1;
      half2_t c1024[NF], c64[NF], s2[NF];
  #pragma unroll
      for (int f = 0; f < NF; ++f) {
        const uint32_t z = (S.z[f] >> (4 * (nclamp[f] & 7))) & 15u;
        c1024[f] = __builtin_bit_cast(half2_t, (0xE400u | z) * 0x00010001u);
        c64[f] = __builtin_bit_cast(half2_t, (0xD400u | (z << 4)) * 0x00010001u);
        s2[f] = __builtin_bit_cast(half2_t, S.s[f] * 0x00010001u);
      }
  #pragma unroll
      for (int s = 0; s < 4; ++s) {
        half8_t bf[NF];
  #pragma unroll
        for (int f = 0; f < NF; ++f) bf[f] = dequant8(S.b[f][s], mc, c1024[f], c64[f], s2[f]);
  #pragma unroll
        for (int i = 0; i < MI; ++i) {
          const u32x4 av = lds[buf][swz(i * 32 + col, h * 4 + s)];
          const half8_t a = __builtin_bit_cast(half8_t, av);
  #pragma unroll
          for (int f = 0; f < NF; ++f) acc[i][f] = mfma32(a, bf[f], acc[i][f]);
        }
      }
      store_a(Snext, buf ^ 1);  // the other buffer was last read before the previous barrier
      __syncthreads();
      issue(min(t + PD, kend - 1), S);
    };

    const int nsteps = kend - kbeg;
    if (nsteps > 0) {
  #pragma unroll
      for (int d = 0; d < PD; ++d) issue(min(kbeg + d, kend - 1), st[d]);
      store_a(st[0], 0);
    }
    __syncthreads();
    int it = 0;
    for (; it + PD <= nsteps; it += PD) {
  #pragma unroll
      for (int d = 0; d < PD; ++d) step(kbeg + it + d, st[d], st[(d + 1) % PD]);
    }
  #pragma unroll
    for (int d = 0; d < PD; ++d)
      if (it + d < nsteps) step(kbeg + it + d, st[d], st[(d + 1) % PD]);
  }

  // Output element (i, f, r): row m0 + 32 i + 8 (r / 4) + 4 h + (r % 4), column nrow[f].
  if (nsplit > 1) {
    // Split K: every part writes its fp32 partial sums, the last arriving workgroup
    // re-reads all of them (its own included) and adds them in split order.  Uniform
    // mode keeps the partials as [split][M][N]; a tail tile j (tail mode) as a compact
    // [j][split][BM][BN] region.  One code path for both (two made the compiler spill).
    const bool tail = tail_splits > 0;
    float* pbase = tail ? partials + (int64_t)(tile - n_full) * nsplit * BM * BN : partials + (int64_t)m0 * N + n0;
    const int64_t ld = tail ? (int64_t)BN : (int64_t)N;
    const int64_t sstride = tail ? (int64_t)BM * BN : (int64_t)M * N;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (!nok[f]) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m < M) st_coherent(pbase + split * sstride + (m - m0) * ld + (nrow[f] - n0), acc[i][f][r]);
        }
      }
    if (!splitk_arrive(counters + (tail ? tile - n_full : tile), nsplit)) return;
    // one 16-value fragment at a time (its 16 loads in flight together)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        float16_t sum;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum[r] = 0.0f;
        for (int sp = 0; sp < nsplit; ++sp) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = min(m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3), M - 1);
            sum[r] += ld_coherent(pbase + sp * sstride + (m - m0) * ld + (nclamp[f] - n0));
          }
        }
        acc[i][f] = sum;
      }
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (!nok[f]) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) y[(int64_t)m * N + nrow[f]] = (half_t)acc[i][f][r];
      }
    }
}

}  // namespace

// Tile shapes, largest first: (MI, NF) = (4, 2) 128 x 256, (4, 1) 128 x 128, (2, 2) 64 x 256,
// (2, 1) 64 x 128.  The plan takes the first shape that gives at least kMinTiles tiles
// (a full wave of workgroups); split-K only when even the smallest does not.
static const int kShapes[4][2] = {{4, 2}, {4, 1}, {2, 2}, {2, 1}};
// Workgroups resident per CU for each shape (2 waves per SIMD at 239 VGPRs, 3 at 152 and
// 167, 4 at 116), and the MI355X's CU count.
static const int kResidentPerCU[4] = {2, 3, 3, 4};
constexpr int kCUs = 256;
// Compiled (MI, NF, prefetch depth) variants.
#define GEMM_VARIANTS(V) \
  V(4, 2, 1) V(4, 1, 1) V(2, 2, 1) V(2, 1, 1) V(2, 1, 3) V(2, 1, 4) V(2, 1, 6) V(4, 2, 0) V(4, 1, 0) V(2, 2, 0) \
  V(2, 1, 0) V(4, 1, 5) V(2, 2, 5) V(2, 1, 5) V(4, 2, 7) V(4, 1, 7) V(2, 2, 7) V(2, 1, 7) V(2, 1, 8)
static bool gemm_variant_compiled(int mi, int nf, int pd) {
#define V(MI, NF, PD) if (mi == MI && nf == NF && pd == PD) return true;
  GEMM_VARIANTS(V)
#undef V
  return false;
}

GemmPlan gemm_plan(int M, int N, int K) {
  GemmPlan p;
  const int min_tiles = env_int("W4_GEMM_MIN_TILES", 256);
  const int forced = env_int("W4_GEMM_SHAPE", 0);  // 1..4 selects kShapes[forced - 1]
  int pick = 3;
  // 32 < M <= 512: narrow (128-column) tiles and split-K to at least 320 workgroups
  // (sweeps on K = 5120, N in {5120, 13824}, M = 96 .. 512).
  const bool mid = M <= 512 && forced == 0;
  if (forced >= 1 && forced <= 4) {
    pick = forced - 1;
  } else if (mid) {
    // 64 x 128 tiles up to M = 128 (K = 5120, N = 13824, with register sets in flight:
    // M = 64 30.2 -> 26.9 us, M = 128 45.2 -> 37.5 against the one-step-ahead 128 x 128 /
    // 64 x 128 plans); 128 x 128 above on wide matrices (M = 256: 52.1 -> 48.8 us, whole
    // K per workgroup) and from M = 384 on
    // (narrow matrices, N < 8192, keep the 64 x 128 tiles up to M = 512: M = 512, K = 5120,
    // N = 5120 52.7 -> 43.6 us against 128 x 128 tiles)
    pick = (M > 128 && N >= 8192) ? 1 : 3;
  } else {
    for (int i = 0; i < 4; ++i) {
      const int tm = (M + 32 * kShapes[i][0] - 1) / (32 * kShapes[i][0]);
      const int tn = (N + 128 * kShapes[i][1] - 1) / (128 * kShapes[i][1]);
      if (tm * tn >= min_tiles) {
        pick = i;
        break;
      }
    }
    // narrow matrices up to M = 1024: 64 x 128 tiles with the X ring at one workgroup per
    // CU (K = 5120, N = 5120 at M = 768 / 1024: 63.3 / 73.0 -> 51.1 / 70.4 us; K = 13824 at
    // M = 1024 181.9 -> 179.2; at M = 2048 the 128 x 256 tiles stay faster)
    if (N < 8192 && M <= 1024) pick = 3;
    // where 128 x 256 tiles fill under 384 of the 512 slots: 128 x 128 tiles (M = 640 /
    // 768 on N = 13824 and M = 768 on N = 15360: 123.8 / 128.3 / 132.6 -> 119.1 / 123.7 /
    // 128.0 us; M = 2048 on N = 5120, K = 5120 / 13824: 128.3 / 328.1 -> 123.5 / 319.0;
    // not on N = 4096: 4096 x 4096 at M = 2048 69.9 against 70.8)
    if (pick == 0 && N > 4096 && ((M + 127) / 128) * ((N + 255) / 256) < 384) pick = 1;
  }
  p.mi = kShapes[pick][0];
  p.nf = kShapes[pick][1];
  // register sets in flight (BK steps of loads ahead of the MFMAs)
  // Loop (K = 5120, N = 13824 unless stated, clocks warm, weights streamed from HBM):
  //  * depth 7 streams both the X tiles and the packed weights into a three-step LDS ring
  //    (two workgroups per CU, nothing held in registers while in flight): the 128-row
  //    tiles at large M, 1.00-1.09 PFLOP/s at M = 4096 (N in {27648, 5120}, and
  //    K = 13824) against 0.96-1.06 for depth 1 (the next step's X tile in registers);
  //    M = 1024, N = 5120 on 128 x 128 tiles 85.4 -> 73.3 us;
  //  * depth 8, X tiles and weights in a six-slot LDS ring (five steps ahead, two
  //    workgroups per CU): the 64 x 128 tiles at 32 < M <= 128, split towards only 160
  //    workgroups (M = 64 / 96 / 128: 23.1 / 29.7 / 30.0 us against 26.1 / 33.6 / 34.5
  //    with depth 5 and 320 workgroups; N = 5120: M = 48 / 64 / 128 17.6 / 18.2 / 22.5
  //    against 20.6 / 18.5 / 23.4);
  //  * depth 5, X tiles direct-to-LDS three steps ahead and the weights in registers, two
  //    or more workgroups per CU (M = 64 / 128 / 256 25.8 / 35.1 / 50.4 us; 27.4 / 36.4 /
  //    52.3 with depth 0);
  //  * depth 0, X tiles direct-to-LDS four steps ahead, one workgroup of 4 waves per CU
  //    for 128-row tiles: the 128 x 128 tiles at 256 < M <= 512 (M = 384 / 512 70.9 /
  //    79.6 us; 95.2 us at M = 512 with register-staged X, 3-4 sets ahead); at
  //    128 < M <= 256 those tiles take depth 7 (M = 256 48.8 us).
  //  * on narrow matrices (N < 8192) the 64 x 128 tiles at mid M take depth 0 instead of
  //    8: one workgroup per CU with X four steps ahead (K = 5120, N = 5120 at
  //    M = 48 / 96 / 128 / 256: 17.0 / 21.5 / 21.6 / 28.4 -> 16.7 / 20.6 / 20.5 / 26.0 us;
  //    K = 13824 at M = 64 / 128 / 256: 27.3 / 41.3 / 68.3 -> 26.4 / 38.7 / 62.8; no gain
  //    at N = 8192).
  // Depths 1, 3, 4, 6 (register sets in flight) stay compiled for sweeps and other shapes.
  p.depth = env_int("W4_GEMM_DEPTH", mid ? (pick == 3 ? (N < 8192 ? 0 : 8) : (M <= 256 ? 7 : 0))
                                         : (pick <= 1 ? 7 : (pick == 3 && N < 8192 && M <= 1024 ? 0 : 1)));
  if (!gemm_variant_compiled(p.mi, p.nf, p.depth)) p.depth = 1;
  // the direct-to-LDS pipelines address X, the codes, scales and zero points with 32-bit
  // per-lane offsets
  if ((p.depth == 0 || p.depth == 5 || p.depth == 7 || p.depth == 8) &&
      ((int64_t)M * K >= (int64_t(1) << 31) || (int64_t)N * K >= (int64_t(1) << 33)))
    p.depth = 1;
  p.tiles_m = (M + 32 * p.mi - 1) / (32 * p.mi);
  p.tiles_n = (N + 128 * p.nf - 1) / (128 * p.nf);
  const int ktiles = K / BK;
  const int tiles = p.tiles_m * p.tiles_n;
  int splits = 1;
  // fill the CUs when there are few tiles; keep >= 8 BK steps per split
  // (mid M: 64 x 128 tiles split towards 160 workgroups -- two resident per CU with the
  // six-slot ring, fewer split-K partials; 128 x 128 tiles from 192 on)
  const int want = mid ? (pick == 1 ? 192 : 160) : min_tiles / 2;
  while (tiles * splits < want && ktiles / (splits * 2) >= 8) splits *= 2;
  const int forced_splits = env_int("W4_GEMM_SPLITS", 0);
  if (forced_splits > 0) splits = min(forced_splits, ktiles);
  if (tiles >= kMaxCounters) splits = 1;
  p.kt_per_split = (ktiles + splits - 1) / splits;
  p.splits = (ktiles + p.kt_per_split - 1) / p.kt_per_split;
  // Tail split: with `slots` workgroups resident at once, tiles = q * slots + R with a
  // small remainder R leaves the last round mostly empty (M = 4096, N = 5120: 640 tiles
  // on 512 slots is 1.25 rounds).  The R last tiles are then split in two over their BK
  // steps, so that the last round is shorter and spread over more CUs (measured at
  // M = 4096: O 5120 x 5120 290 -> 262 us, down 13824 x 5120 739 -> 657 us; four parts
  // gave 295 / 685 us, the partial sums costing more than the finer balance).
  p.n_full = 0;
  p.tail_splits = 0;
  const int slots = kCUs * kResidentPerCU[pick] * env_int("W4_GEMM_SLOTS_SCALE", 1) /
                    env_int("W4_GEMM_SLOTS_DIV", 1);
  // Taken when the last round holds at most a quarter of the slots: with 192 or 208 of
  // 512 it was slower (M = 4096 on 5120 x 13824 524.3 -> 547.8 us, M = 4608 on
  // 13824 x 5120 586.3 -> 605.9), with 128 faster (O above; K = 8192 335.8 -> 321.4).
  // W4_GEMM_TAIL = 1 takes it whenever the last round is at most half full, 0 never.
  const int rem = tiles % slots;
  const int tail_env = env_int("W4_GEMM_TAIL", -1);
  const bool tail_ok = tail_env < 0 ? 4 * rem <= slots : (tail_env > 0 && 2 * rem <= slots);
  if (p.splits == 1 && !mid && tail_ok && tiles > slots && rem > 0 && ktiles >= 16) {
    const int ts = max(2, min(8, env_int("W4_GEMM_TAIL_PARTS", 2)));
    p.n_full = tiles - rem;
    p.tail_splits = ts;
  }
  return p;
}

// Workspace of the tail split: counters, then [R][tail_splits][BM][BN] fp32 partials.
static size_t tail_bytes(const GemmPlan& p) {
  const int tiles = p.tiles_m * p.tiles_n;
  return kCounterRegionBytes + (size_t)(tiles - p.n_full) * p.tail_splits * (32 * p.mi) * (128 * p.nf) * sizeof(float);
}

size_t gemm_workspace_bytes(const GemmPlan& p, int M, int N) {
  if (p.tail_splits > 0) return tail_bytes(p);
  if (p.splits == 1) return 0;
  return kCounterRegionBytes + (size_t)p.splits * M * N * sizeof(float);
}

hipError_t launch_gemm(const GemmPlan& p, const void* x, const int32_t* qweight, const void* scales,
                       const int32_t* qzeros, void* y, void* ws, int M, int N, int K, int group_size,
                       hipStream_t stream) {
  const int glog = group_log2(group_size);
  unsigned* counters = (unsigned*)ws;
  float* partials = ws ? (float*)((char*)ws + kCounterRegionBytes) : nullptr;
  const int tiles = p.tiles_m * p.tiles_n;
  const int blocks = p.tail_splits > 0 ? p.n_full + (tiles - p.n_full) * p.tail_splits : tiles * p.splits;
#define GEMM_LAUNCH(MI, NF, PD)                                                                               \
  if (p.mi == MI && p.nf == NF && p.depth == PD) {                                                            \
    hipLaunchKernelGGL((gemm_kernel<MI, NF, PD>), dim3(blocks), dim3(kThreads), 0, stream, (const half_t*)x,     \
                       (const uint32_t*)qweight, (const half_t*)scales, (const uint32_t*)qzeros, (half_t*)y,   \
                       counters, partials, M, N, K, p.tiles_m, p.tiles_n, p.splits, p.kt_per_split, glog, p.n_full, \
                       p.tail_splits);                                                                        \
    return hipGetLastError();                                                                                 \
  }
  GEMM_VARIANTS(GEMM_LAUNCH)
#undef GEMM_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace w4
