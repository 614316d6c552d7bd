// Skinny W4A16 GEMM for M <= 32 (decode): bandwidth-bound, every packed weight byte
// is read once.
//
// The pages single out the small-batch regime ("Implement AWQ quantization support
// for LLaMA", vllm-project/vllm PR 1032: the AWQ GEMM is fastest below batch 8 and
// on par with FP16 at batch 16) and say that dequantization is the tricky part.
// Here the dequantization is folded into per-group fp32 arithmetic:
//
//   Y[m,n] = sum_g s[n,g] * ( T_g[m,n] - P_g[m] - z[n,g] * S_g[m] ),
//   T_g[m,n] = sum_{k in g} X[m,k] * (c_k + q[n,k]),   S_g[m] = sum_{k in g} X[m,k],
//   P_g[m] = sum_{k in g} c_k X[m,k],   c_k = 1024 for k = 0, 1 mod 4, 64 for k = 2, 3 mod 4,
//
// which equals sum_k X[m,k] * (q - z) * s exactly in real arithmetic.  The MFMA
// consumes the raw fp16 values c_k + q (five VALU ops per 8 codes of a parity-split
// word, in natural k order like X; no per-element subtract or multiply); fp16
// x (c_k + q) products are exact in fp32, only the fp32 sums round.
//
// Work split (register-X kernel, M <= 32; the kernel further below stages X in LDS and
// is kept behind a tuning variable): a workgroup (4, 8 or 12 waves) owns 16 T output
// columns n (T = 1 .. 8 tiles of 16) and a contiguous range of K groups (split-K across
// workgroups only for narrow N); its waves take the groups of that range round robin.  Per group, lane l of a wave
// loads one 16-byte chunk (32 codes) of row n0 + 16t + (l % 16) for each tile t -- with
// the tiled weight layout the 64 lanes read one contiguous 1 KB block -- the 64 bytes of
// X it needs, and one scale and one zero-point word per 64 columns; the four MFMAs of a
// group use word j of every lane's chunk, and A is loaded with the same K-slot
// assignment.  S_g and -P_g come from two MFMA chains against constant B operands.
// Partial sums are reduced across the waves in LDS, then across split-K workgroups
// through the workspace by the last arriving workgroup, in a fixed order.
#include "kernels.hpp"

namespace w4 {

namespace {


template <int MT, int T>
struct GroupRegs {
  u32x4 b[T];              // packed codes: 4 words (32 k) for each of the T n-tiles
  half8_t a[MT][4];        // X fragments: MT m-tiles x 4 MFMAs
  half_t s[T];             // dequantizing variant: scale of this lane's row in each n-tile
  uint32_t zw[T];          // dequantizing variant: zero-point word of that row
  uint16_t sc[kChunks<T>]; // scale bits of column n0 + 64 c + (lane % (16 T)), per chunk c
  uint32_t zc[kChunks<T>]; // zero-point word holding that column
};

// Loads are branch-free so that all of them are issued back to back: out-of-range rows
// (n >= N, m >= M) read a clamped, valid row.  Nothing needs zeroing: an MFMA output
// row depends only on its own A row and an output column only on its own B column
// (and scale / zero point), so clamped data only reaches outputs that are never
// stored.
template <int MT, int T, bool DQ, int XS = 0>
__device__ __forceinline__ void load_group(GroupRegs<MT, T>& r, const half_t* __restrict__ x,
                                           const uint32_t* __restrict__ qweight,
                                           const half_t* __restrict__ scales,
                                           const uint32_t* __restrict__ qzeros, int g, int n0, int lane,
                                           int M, int N, int K, int glog) {
  const int ng = K / 128;
  const int nzw = (N + 7) / 8;
  const int slot = lane >> 4;
  const int last_tile = (N - 1) >> 4;
  // scale / zero-point row: of the 128-k unit (group sizes 128 and -1), or, in the
  // dequantizing variant, of this lane's 32 k (any group size >= 32)
  const int64_t row = (((int64_t)g << 7) + (DQ ? 32 * slot : 0)) >> glog;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    // tiled layout: lane l reads chunk l of the 1 KB block (16 rows x 128 k) -- row
    // l % 16 of the tile, words 4 (l / 16) .. + 3 of the group
    const int tile = min((n0 >> 4) + t, last_tile);
    r.b[t] = ld_stream(qweight + ((int64_t)tile * ng + g) * 256 + lane * 4);
    if (DQ) {
      const int nc = min(n0 + 16 * t + (lane & 15), N - 1);
      r.s[t] = scales[row * N + nc];
      r.zw[t] = qzeros[row * nzw + (nc >> 3)];
    }
  }
  if (!DQ) {
#pragma unroll
    for (int c = 0; c < kChunks<T>; ++c) {
      const int nc = min(n0 + chunk_col<T>(c, lane), N - 1);
      r.sc[c] = __builtin_bit_cast(uint16_t, scales[row * N + nc]);
      r.zc[c] = qzeros[row * nzw + (nc >> 3)];
    }
  }
  if (XS) {
    // M <= 4 XS: XS loads bring the group's X, all rows -- load i of lane l takes 16-byte
    // chunk l % 16 of row 4 i + l / 16 into a[i / 4][i % 4] (rows past M clamped; each
    // load reads four whole 256-byte rows); compute_group forms the fragments in LDS
#pragma unroll
    for (int i = 0; i < XS; ++i)
      r.a[i >> 2][i & 3] = *reinterpret_cast<const half8_t*>(x + (int64_t)min(4 * i + (lane >> 4), M - 1) * K +
                                                             g * 128 + (lane & 15) * 8);
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + (lane & 15), M - 1);
    const half8_t* src = reinterpret_cast<const half8_t*>(x + (int64_t)m * K + g * 128 + slot * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) r.a[mt][j] = src[j];
  }
}

// The 8 codes of a (parity-split) word as the fp16 B fragment (1024 + q0, 1024 + q1,
// 64 + q2, 64 + q3, 1024 + q4, 1024 + q5, 64 + q6, 64 + q7): natural k order, one shift
// and four v_and_or_b32.
__device__ __forceinline__ half8_t unpack_mixed(uint32_t w, const Magic& c) {
  return __builtin_bit_cast(half8_t, expand_word(w, c));
}

// One group.  Each code word costs five VALU operations and X enters the MFMAs as
// loaded (both in natural k order).  Two MFMA chains against constant B operands give,
// per row, S_g (ones) and -P_g (-1024 at k = 0, 1 mod 4, -64 at k = 2, 3 mod 4); -P_g
// seeds every n-tile's chain, which then holds T_g - P_g = sum_k X q and the fold is
// y += s (T_g - P_g - z S_g).
template <int MT, int T, int XS = 0>
__device__ __forceinline__ void compute_group(const GroupRegs<MT, T>& r, float4_t (&yacc)[MT][T],
                                              const int (&zsh)[kChunks<T>], half_t* xb = nullptr, int lane = 0) {
  const half8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};
  const half8_t negmagic = {-1024, -1024, -64, -64, -1024, -1024, -64, -64};
  const Magic mc = magic_regs();
  half8_t a[MT][4];
  float4_t ssum[MT], negp[MT];
  if (XS) {
    // The group's 4 XS rows x 256 bytes through this wave's XS KB of LDS: chunk c of row
    // q at chunk c ^ (q mod 16) (the rows of one fragment read, and the chunks of one row
    // written, fall in distinct banks).  Fragment j of lane l in m-tile mt is chunk
    // 4 (l / 16) + j of row (l % 16) mod 4 XS with one m-tile (MFMA rows past 4 XS only
    // reach outputs that are never stored: M <= 4 XS), of row 16 mt + l % 16 with two
    // (XS = 8).  LDS operations of one wave execute in order, so the reads see the whole
    // wave's writes.
    const int q = lane >> 4, c = lane & 15;
#pragma unroll
    for (int i = 0; i < XS; ++i) {
      const int row = 4 * i + q;
      *reinterpret_cast<half8_t*>(xb + row * 128 + (c ^ (row & 15)) * 8) = r.a[i >> 2][i & 3];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int rr = MT == 1 ? lane & (4 * XS - 1) : 16 * mt + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a[mt][j] = *reinterpret_cast<const half8_t*>(xb + rr * 128 + ((4 * q + j) ^ (rr & 15)) * 8);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    ssum[mt] = float4_t{0, 0, 0, 0};
    negp[mt] = float4_t{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!XS) a[mt][j] = r.a[mt][j];
      ssum[mt] = mfma16(a[mt][j], ones, ssum[mt]);
      negp[mt] = mfma16(a[mt][j], negmagic, negp[mt]);
    }
  }
  // scale bits | zero point << 16 of the loaded column, moved to the MFMA layout
  uint32_t szc[kChunks<T>], sz[T];
#pragma unroll
  for (int c = 0; c < kChunks<T>; ++c) szc[c] = (uint32_t)r.sc[c] | (((r.zc[c] >> zsh[c]) & 15u) << 16);
  rows_to_tiles<T>(szc, sz);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    half8_t bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = unpack_mixed(r.b[t][j], mc);
    const float z = (float)((sz[t] >> 16) & 0xffu);
    const float sc = (float)__builtin_bit_cast(half2_t, sz[t])[0];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float4_t tacc = negp[mt];
#pragma unroll
      for (int j = 0; j < 4; ++j) tacc = mfma16(a[mt][j], bv[j], tacc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = fmaf(-z, ssum[mt][i], tacc[i]);
        yacc[mt][t][i] = fmaf(sc, d, yacc[mt][t][i]);
      }
    }
  }
}

// Dequantizing variant (group sizes 64 and 32, whose groups split the k range of one
// MFMA): every word becomes fp16 (q - z) s in registers (one rounding per element, the
// large-M GEMM's dequantization) with the scale and zero point of this lane's own 32 k,
// and the MFMAs accumulate Y directly.
template <int MT, int T>
__device__ __forceinline__ void compute_group_dq(const GroupRegs<MT, T>& r, float4_t (&yacc)[MT][T], int n0,
                                                 int lane, int N) {
  const Magic mc = magic_regs();
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int nc = min(n0 + 16 * t + (lane & 15), N - 1);
    // fp16 bit patterns built with integer ops: -(1024 + z), -(64 + z), the scale twice
    const uint32_t z = (r.zw[t] >> (4 * (nc & 7))) & 15u;
    const half2_t c1024 = neg1024z2(z), c64 = neg64z2(z);
    const half2_t s2 = scale2(__builtin_bit_cast(uint16_t, r.s[t]));
    half8_t bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = dequant8(r.b[t][j], mc, c1024, c64, s2);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) yacc[mt][t] = mfma16(r.a[mt][j], bv[j], yacc[mt][t]);
  }
}

// WAVES waves per workgroup take the groups of the workgroup's K range round robin.
// D register sets rotate (loop unrolled by D, no register copies), so while a wave
// computes one group the loads of its next D groups are in flight (D * T KB per wave).
// A workgroup owns 16 T output columns (T 16-row tiles; all its waves share them).
//
// Workgroups resident per CU that the register allocation must allow, for the plans
// that pick these variants: three 4-wave workgroups (<= 168 VGPRs) or two 8-wave ones
// (<= 128 VGPRs); the others take what they need.
constexpr int skinny_min_blocks(int mt, int t, int d, int waves, bool dq, int xs) {
  if (mt != 1 || dq || xs) return 1;
  if (waves == 4 && ((t == 4 && d <= 3) || (t == 2 && d == 2) || (t == 1 && d == 4))) return 3;
  if (waves == 8 && ((t == 2 && d <= 3) || (t == 4 && d == 2) || (t == 1 && d == 4))) return 2;
  return 1;
}
template <int MT, int T, int D, int WAVES, bool DQ, int XS = 0>
__global__ __launch_bounds__(WAVES * kWave, skinny_min_blocks(MT, T, D, WAVES, DQ, XS)) void skinny_kernel(const half_t* __restrict__ x,
                                                               const uint32_t* __restrict__ qweight,
                                                               const half_t* __restrict__ scales,
                                                               const uint32_t* __restrict__ qzeros,
                                                               half_t* __restrict__ y,
                                                               unsigned* __restrict__ counters,
                                                               float* __restrict__ partials, int M, int N, int K,
                                                               int splits, int gps, int drain, int glog) {
  constexpr int kT = WAVES * kWave;
  constexpr int kCols = 16 * T;           // output columns of one workgroup
  constexpr int kOut = MT * 16 * kCols;   // outputs of one workgroup
  // outputs per thread in the epilogue (MT * T; 1 when the workgroup has more threads than
  // outputs: threads past the last output only read a clamped entry and store nothing)
  constexpr int kPer = (kOut + kT - 1) / kT;
  __shared__ float red[WAVES][MT * T * 4 * kWave];
  __shared__ __align__(16) half_t xbuf[XS ? WAVES : 1][XS ? 512 * XS : 8];  // M <= 4 XS: X rows of a group
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
  int zsh[kChunks<T>];  // bit offset of the loaded column's zero point in its word, per chunk
#pragma unroll
  for (int c = 0; c < kChunks<T>; ++c) zsh[c] = 4 * (min(n0 + chunk_col<T>(c, lane), N - 1) & 7);
  GroupRegs<MT, T> r[D];
  const int glast = gend - 1;
  const int g = gbeg + wave;
#pragma unroll
  for (int d = 0; d < D; ++d)
    load_group<MT, T, DQ, XS>(r[d], x, qweight, scales, qzeros, min(g + d * WAVES, glast), n0, lane, M, N, K, glog);
  // Steady state without conditions (the wait before each compute then covers only its
  // own register set), then the remaining < D groups; all counts are wave-uniform.
  const int mine = g < gend ? (gend - g + WAVES - 1) / WAVES : 0;
  int it = 0;
  for (; it + D <= mine; it += D) {
    if (drain) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (DQ) compute_group_dq<MT, T>(r[d], yacc, n0, lane, N);
      else compute_group<MT, T, XS>(r[d], yacc, zsh, xbuf[wave], lane);
      // (scheduling fences: without them the compiler starts the next set's MFMAs before
      // this set's loads are issued, and its waits then drain nearly every load in flight)
      __builtin_amdgcn_sched_barrier(0);
      load_group<MT, T, DQ, XS>(r[d], x, qweight, scales, qzeros, min(g + (it + d + D) * WAVES, glast), n0, lane, M, N,
                            K, glog);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (it + d < mine) {
      if (DQ) compute_group_dq<MT, T>(r[d], yacc, n0, lane, N);
      else compute_group<MT, T, XS>(r[d], yacc, zsh, xbuf[wave], lane);
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
    const int o = min(it * kT + (int)threadIdx.x, kOut - 1);
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


// ---------------------------------------------------------------------------------
// M <= 16: X staged in LDS, codes unpacked in five VALU operations per word (no default
// plan takes this kernel; it is kept for every M <= 16 behind its tuning variable and
// tested that way).
//
// The workgroup copies its slice of X (M rows x its K range) into LDS once; the
// per-group register sets that are prefetched D deep then carry only what comes from
// HBM: T x 16 bytes of codes, T scales and T zero-point words per lane.
//
// B operand: for the 8 codes of a parity-split word, v_and_or_b32 with mask 0x000f000f
// and fp16 1024 in both halves gives (1024 + q_0, 1024 + q_1) -- a code in the low
// mantissa bits under exponent 2^10 -- and with mask 0x00f000f0 and fp16 64 gives
// (64 + q_2, 64 + q_3) -- a code in mantissa bits 4..7 under exponent 2^6 is worth q
// exactly.  The same on the word shifted right by 8 gives k = 4, 5 and 6, 7: four
// v_and_or_b32 and one shift per word, in natural k order, as X is stored in LDS.  One
// MFMA chain forms, exactly up to its fp32 sums,
//   T_g[m,n] = sum_k X[m,k] q[n,k] + P_g[m],
//   P_g[m] = 1024 sum_{k = 0,1 mod 4} X[m,k] + 64 sum_{k = 2,3 mod 4} X[m,k],
// and the group's contribution to Y is s (T_g - P_g - z S_g), S_g[m] = sum_{k in g} X[m,k].
// P_g and S_g depend on X only: they are summed in fp32 while X is staged, reduced over
// the 16 chunks of a group with DPP moves (fixed order, deterministic) and kept in LDS.
// LDS rows of X are padded by 16 bytes, so the 16 rows of an A fragment fall in
// distinct banks.
//
// A workgroup is WN x WK waves: WN column groups of 16 T columns each, and WK waves that
// take the groups of the K range round robin; partial sums are reduced across the WK
// waves in LDS (reusing the X region), then across split-K workgroups as above.
template <int T>
struct WStage {
  u32x4 b[T];      // packed codes: chunk of this lane's row / K-slot in each n-tile
  half_t s[T];     // scale of this lane's row in each n-tile (raw fp16)
  uint32_t zw[T];  // packed zero-point word holding this lane's row in each n-tile
};

template <int T>
__device__ __forceinline__ void load_wstage(WStage<T>& r, const uint32_t* __restrict__ qweight,
                                            const half_t* __restrict__ scales,
                                            const uint32_t* __restrict__ qzeros, int g, int tile0, int lane,
                                            int N, int ng, int nzw, int glog) {
  const int last_tile = (N - 1) >> 4;
  const int64_t row = ((int64_t)g << 7) >> glog;  // group sizes 128 and -1
  const half_t* srow = scales + row * N;
  const uint32_t* zrow = qzeros + row * nzw;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int tile = min(tile0 + t, last_tile);
    const int nc = min(16 * (tile0 + t) + (lane & 15), N - 1);
    r.b[t] = ld_stream(qweight + ((int64_t)tile * ng + g) * 256 + lane * 4);
    r.s[t] = srow[nc];
    r.zw[t] = zrow[nc >> 3];
  }
}

// DPP row moves (16-lane rows): quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_half_mirror,
// row_mirror; the four partial sums below make every lane of a row hold the row total.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

// cc / cpr for 0 <= cc < 16 cpr, cpr < 2^16: (cc + 0.5) / cpr lies at least 0.5 / cpr
// away from an integer, far more than the fp32 rounding of the product.
__device__ __forceinline__ int chunk_row(int cc, int cpr) {
  return (int)(((float)cc + 0.5f) * (1.0f / (float)cpr));
}

// Stage one 16-byte chunk (8 halves of X) of chunk index cc (clamped into the slice) to
// LDS, and add its sums over k = 0, 1 mod 4 (e) and k = 2, 3 mod 4 (od) to the group's
// S, P (written by the first lane of the 16 lanes that hold the group's 16 chunks;
// `live` is false for the clamped copies past the slice, which are rewritten, not summed).
__device__ __forceinline__ void stage_chunk(u32x4 v, int cc, bool live, int cpr, int rs, half_t* xs, float* sp) {
  const int row = chunk_row(cc, cpr), col = cc - row * cpr;
  *reinterpret_cast<u32x4*>(xs + row * rs + col * 8) = v;
  // (vector elements are copied to scalars before __builtin_bit_cast: applied directly
  // to an element of an ext_vector this hipcc reads element 0)
  const uint32_t o0 = v[0], o1 = v[1], o2 = v[2], o3 = v[3];  // (x0, x1), (x2, x3), (x4, x5), (x6, x7)
  const half2_t one2 = {1, 1};
  float e = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, o0), one2, 0.0f, false);
  e = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, o2), one2, e, false);
  float od = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, o1), one2, 0.0f, false);
  od = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, o3), one2, od, false);
  e = row16_sum(e);
  od = row16_sum(od);
  if (live && (col & 15) == 0) {
    float* g = sp + (col >> 4) * 32;
    g[row] = e + od;
    g[16 + row] = 1024.0f * e + 64.0f * od;
  }
}

// One group: A fragments and S, P from LDS, then per n-tile T_g and the fold into the
// accumulators.  ONE_ROW: M == 1, only accumulator element 0 of lanes 0..15 is an output.
template <int T, bool ONE_ROW>
__device__ __forceinline__ void compute_wstage(const WStage<T>& r, const half_t* xrow, const float* spg,
                                               float4_t (&yacc)[T], const int (&zsh)[T], int lane) {
  half8_t a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const half8_t*>(xrow + 8 * j);
  const float4_t S = *reinterpret_cast<const float4_t*>(spg + 4 * (lane >> 4));
  const float4_t P = *reinterpret_cast<const float4_t*>(spg + 16 + 4 * (lane >> 4));
  const Magic mc = magic_regs();
#pragma unroll
  for (int t = 0; t < T; ++t) {
    half8_t bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = unpack_mixed(r.b[t][j], mc);
    float4_t tacc = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) tacc = mfma16(a[j], bv[j], tacc);
    const float z = (float)((r.zw[t] >> zsh[t]) & 15u);
    const float sc = (float)r.s[t];
#pragma unroll
    for (int i = 0; i < (ONE_ROW ? 1 : 4); ++i) {
      const float d = fmaf(-z, S[i], tacc[i] - P[i]);
      yacc[t][i] = fmaf(sc, d, yacc[t][i]);
    }
  }
}

constexpr int kXChunksPerPass = 8;  // 16-byte chunks of X each thread stages per pass

template <int T, int D, bool ONE_ROW>
__global__ __launch_bounds__(512) void skinny_lds_kernel(const half_t* __restrict__ x,
                                                         const uint32_t* __restrict__ qweight,
                                                         const half_t* __restrict__ scales,
                                                         const uint32_t* __restrict__ qzeros,
                                                         half_t* __restrict__ y, unsigned* __restrict__ counters,
                                                         float* __restrict__ partials, int M, int N, int K,
                                                         int splits, int gps, int wn_count, int drain, int glog) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nthreads = blockDim.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WN = wn_count;
  const int WK = (nthreads >> 6) / WN;
  const int wn = wave % WN, wk = wave / WN;
  const int cols = 16 * T * WN;
  const int n0 = blockIdx.x * cols;
  const int tile0 = (n0 >> 4) + wn * T;
  const int split = blockIdx.y;
  const int ng = K / 128;
  const int nzw = (N + 7) / 8;
  const int gbeg = split * gps;
  const int gend = min(ng, gbeg + gps);
  const int kb = (gend - gbeg) * 128;
  const int rs = kb + 8;  // padded LDS row stride in halves
  half_t* xs = reinterpret_cast<half_t*>(smem);
  float* sp = reinterpret_cast<float*>(smem + M * rs * 2);  // [group][S rows 0..15, P rows 0..15]

  // The first pass of the X slice is issued before the weight prefetch, so that it
  // arrives first and the first compute waits only for it and its own weights.  Every
  // load and LDS store is unconditional: chunk indices past the slice are clamped to its
  // last chunk (rewritten with the same value), group indices past the range to the
  // last group.
  const int cpr = kb >> 3;  // 16-byte chunks per row (a multiple of 16)
  const int total = M * cpr;
  const int64_t xoff = (int64_t)gbeg * 128;
  u32x4 xv[kXChunksPerPass];
#pragma unroll
  for (int i = 0; i < kXChunksPerPass; ++i) {
    const int cc = min((int)threadIdx.x + i * nthreads, total - 1);
    const int row = chunk_row(cc, cpr), col = cc - row * cpr;
    xv[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)row * K + xoff + col * 8);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the X loads ahead of the weight loads
  WStage<T> r[D];
  const int glast = gend - 1;
  const int g = gbeg + wk;
#pragma unroll
  for (int d = 0; d < D; ++d) load_wstage<T>(r[d], qweight, scales, qzeros, min(g + d * WK, glast), tile0, lane, N, ng, nzw, glog);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kXChunksPerPass; ++i) {
    const int c = threadIdx.x + i * nthreads;
    stage_chunk(xv[i], min(c, total - 1), c < total, cpr, rs, xs, sp);
  }
  // further passes (M * K-range larger than one pass of the workgroup)
  for (int c0 = threadIdx.x + kXChunksPerPass * nthreads; c0 < total; c0 += kXChunksPerPass * nthreads) {
#pragma unroll
    for (int i = 0; i < kXChunksPerPass; ++i) {
      const int cc = min(c0 + i * nthreads, total - 1);
      const int row = chunk_row(cc, cpr), col = cc - row * cpr;
      xv[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)row * K + xoff + col * 8);
    }
#pragma unroll
    for (int i = 0; i < kXChunksPerPass; ++i) {
      const int c = c0 + i * nthreads;
      stage_chunk(xv[i], min(c, total - 1), c < total, cpr, rs, xs, sp);
    }
  }
  __syncthreads();

  float4_t yacc[T];
  int zsh[T];  // bit offset of this lane's zero point in its packed word
#pragma unroll
  for (int t = 0; t < T; ++t) {
    yacc[t] = float4_t{0, 0, 0, 0};
    zsh[t] = 4 * (min(16 * (tile0 + t) + (lane & 15), N - 1) & 7);
  }
  // this lane's A row (rows past M read row M - 1; those outputs are never stored)
  const half_t* xrow = xs + min(lane & 15, M - 1) * rs + (lane >> 4) * 32;
  // Steady state without conditions (so that the wait before each compute covers only
  // its own register set), then the remaining < D groups; all counts are wave-uniform.
  const int mine = g < gend ? (gend - g + WK - 1) / WK : 0;
  int it = 0;
  for (; it + D <= mine; it += D) {
    if (drain) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int gl = g + (it + d) * WK - gbeg;
      compute_wstage<T, ONE_ROW>(r[d], xrow + gl * 128, sp + gl * 32, yacc, zsh, lane);
      __builtin_amdgcn_sched_barrier(0);  // (as in the register-X kernel)
      load_wstage<T>(r[d], qweight, scales, qzeros, min(gbeg + gl + D * WK, glast), tile0, lane, N, ng, nzw,
                     glog);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (it + d < mine) {
      const int gl = g + (it + d) * WK - gbeg;
      compute_wstage<T, ONE_ROW>(r[d], xrow + gl * 128, sp + gl * 32, yacc, zsh, lane);
    }
  }

  // Cross-wave reduction in LDS (the X slice is dead after this barrier).
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * T + t) * 256 + i * 64 + lane] = yacc[t][i];
  __syncthreads();

  // Outputs (m < M, n fastest).  Element (t, i) of lane l of wave (wn, wk) is row
  // 4 (l / 16) + i, column 16 (wn T + t) + l % 16 of the workgroup.
  const int outs = M * cols;
  for (int o = threadIdx.x; o < outs; o += nthreads) {
    const int m = o / cols, nl = o - m * cols;
    const int wn_ = nl / (16 * T), t = (nl >> 4) % T;
    const int idx = t * 256 + (m & 3) * 64 + (m >> 2) * 16 + (nl & 15);
    float v = 0.0f;
    for (int k = 0; k < WK; ++k) v += red[(k * WN + wn_) * T * 256 + idx];
    const int n = n0 + nl;
    if (n >= N) continue;
    if (splits == 1) y[(int64_t)m * N + n] = (half_t)v;
    else st_coherent(partials + ((int64_t)split * M + m) * N + n, v);
  }
  if (splits == 1) return;
  if (!splitk_arrive(counters + blockIdx.x, splits)) return;
  for (int o = threadIdx.x; o < outs; o += nthreads) {
    const int m = o / cols, n = n0 + o - m * cols;
    if (n >= N) continue;
    float v = 0.0f;
    for (int sp_ = 0; sp_ < splits; ++sp_) v += ld_coherent(partials + ((int64_t)sp_ * M + m) * N + n);
    y[(int64_t)m * N + n] = (half_t)v;
  }
}

}  // namespace

// Compiled register-X variants (m-tiles, n-tiles, depth, waves, X loaded as whole rows);
// the dequantizing kernels (group sizes 64, 32) are compiled for the default depth and
// 4 waves only.
#define SKINNY_VARIANTS(V)                                                                                   \
  V(1, 4, 2, 4, 0) V(1, 2, 2, 4, 0) V(1, 1, 4, 4, 0) V(2, 4, 2, 4, 0) V(2, 2, 2, 4, 0) V(2, 1, 4, 4, 0)          \
  V(1, 8, 2, 4, 0) V(1, 4, 3, 4, 0) V(1, 2, 4, 4, 0) V(1, 1, 8, 4, 0) V(1, 4, 2, 8, 0) V(1, 2, 2, 8, 0)          \
  V(1, 8, 2, 8, 0) V(2, 8, 2, 4, 0) V(1, 7, 2, 4, 0) V(1, 7, 2, 8, 0) V(1, 7, 2, 4, 1)       \
  V(1, 6, 2, 4, 0) V(1, 6, 2, 8, 0) V(1, 5, 2, 4, 0) V(1, 5, 2, 8, 0)  \
  V(1, 3, 2, 8, 0) V(1, 3, 2, 8, 1) V(1, 4, 2, 4, 1) V(1, 2, 2, 4, 1) V(1, 1, 4, 4, 1) V(1, 2, 2, 8, 1)          \
  V(1, 4, 2, 8, 1) V(1, 2, 3, 8, 0) V(1, 2, 4, 8, 0) V(1, 2, 6, 8, 0)          \
  V(1, 4, 3, 8, 0) V(1, 4, 4, 4, 0) V(1, 1, 4, 8, 0) V(1, 1, 8, 8, 0) V(1, 1, 4, 8, 1)   \
  V(1, 1, 8, 8, 1) V(1, 2, 4, 8, 1) V(1, 2, 2, 12, 1) V(2, 2, 2, 4, 1) V(2, 4, 2, 4, 1)
static int variant_key(int mt, int t, int d, int w, int xs) { return (((mt * 10 + t) * 10 + d) * 100 + w) * 2 + xs; }
static bool skinny_variant_compiled(const SkinnyPlan& p) {
  const int key = variant_key(p.mt, p.tiles, p.depth, p.waves, p.xs);
#define V(MT, T, D, W, XS) if (key == variant_key(MT, T, D, W, XS)) return true;
  SKINNY_VARIANTS(V)
#undef V
  return false;
}

// Waves per workgroup: 4.  At ~190 VGPRs two 4-wave workgroups fit per CU, so grids of
// up to ~512 workgroups are resident at once (no second, partly idle round).
static int skinny_waves(int) { return 4; }

// Kernel, columns per workgroup (16 T) and split-K.  Split-K costs a serial tail
// (partial stores, arrival counter, reads of the partials by the last workgroup), so
// at small M the plan first narrows the workgroups until the column blocks alone give
// ~160 workgroups, and splits K only when they still do not.
SkinnyPlan skinny_plan(int M, int N, int K, int group_size) {
  SkinnyPlan p;
  const int ng = K / 128;
  p.lds = 0;
  p.wn = 1;
  p.wk = 4;
  p.smem = 0;
  p.drain = env_int("W4_SKINNY_DRAIN", 0);
  p.waves = 4;
  p.xs = 0;
  // (Very wide N with a K too long for one LDS slice would need more arrival counters
  // than the workspace holds; such shapes take the register-X kernel below.)
  constexpr int kLdsBudget = 65536 - 256;  // dynamic LDS; the split-K flag is static
  // X slice M (128 gps + 8) halves plus S, P (32 floats per group) within the budget
  const int lds_gmax = max(1, (kLdsBudget - 16 * M) / (256 * M + 128));
  // (group sizes below 128 take the dequantizing register-X kernel)
  const bool lds_ok = M <= 16 && !(ng > lds_gmax && (N + 15) / 16 >= kMaxCounters) &&
                      (group_size == 128 || group_size == -1);
  // Default kernel and shape, from sweeps on the MI355X over the Llama-2-13B projection
  // shapes at M = 1, 4, 8, 16: the register-X kernel (one scale and one zero-point load
  // per 64 columns, five-op unpack) wins everywhere (the last case the LDS kernel held,
  // gate+up 5120 x 27648 at M = 1, went to 7-tile register-X workgroups: 15.7 -> 14.9 us).
  int use_lds = 0;
  int t = 1, d = 4, wn = 1, wk = 4, target = 256;
  if (N > 16384) { t = 4; d = 2; }
  else if (N > 8192) { wn = 2; }
  else if (M == 1) { wk = 8; }  // narrow N, long K, one row: 8 K-waves, no split-K
  else { wn = 2; wk = 2; target = 512; }
  use_lds = env_int("W4_SKINNY_LDS", use_lds) && lds_ok;
  if (use_lds) {
    // X slice in LDS: under 64 KB per workgroup (two resident per CU), which bounds
    // the groups per split.
    p.lds = 1;
    p.mt = 1;
    const int te = env_int("W4_SKINNY_TILES", 0);
    if (te == 1 || te == 2 || te == 4) t = te;
    p.tiles = t;
    // compiled (tiles, depth) pairs: (1, 4), (1, 8), (2, 4), (4, 2)
    d = env_int("W4_SKINNY_DEPTH", d);
    if (t == 4) d = 2;
    else if (t == 2 || d != 8) d = 4;
    p.depth = d;
    p.wn = max(1, env_int("W4_SKINNY_WN", wn));
    p.wk = max(1, env_int("W4_SKINNY_WK", wk));
    if (p.wn * p.wk > 8) { p.wn = 1; p.wk = 4; }
    p.row_blocks = (N + 16 * t * p.wn - 1) / (16 * t * p.wn);
    const int min_splits = (ng + lds_gmax - 1) / lds_gmax;
    target = env_int("W4_SKINNY_BLOCKS", target);
    int splits = (target + p.row_blocks - 1) / p.row_blocks;
    splits = min(splits, max(1, ng / p.wk));
    const int pct = env_int("W4_SKINNY_PARTIAL_PCT", 10);
    splits = min(splits, max(1, (int)((int64_t)K * pct / (1600LL * M))));
    const int forced = env_int("W4_SKINNY_SPLITS", 0);
    if (forced > 0) splits = forced;
    splits = max(max(1, splits), min_splits);
    if (p.row_blocks >= kMaxCounters) splits = 1;  // then min_splits == 1 (lds_ok)
    p.gps = (ng + splits - 1) / splits;
    p.splits = (ng + p.gps - 1) / p.gps;
    const int xbytes = M * (p.gps * 128 + 8) * 2 + p.gps * 128;  // X slice + per-group S, P
    const int rbytes = p.wn * p.wk * t * 1024;
    p.smem = max(xbytes, rbytes);
    return p;
  }
  p.mt = M <= 16 ? 1 : 2;  // M <= 32
  const int waves = skinny_waves(p.mt);
  // Tiles per workgroup: with more rows each X fragment should serve more tiles (X
  // traffic is 4 M / T bytes per weight byte); split K only below 160 column blocks.
  // From sweeps on the Llama-2-13B projection shapes and 4096 x 4096 at M = 1 .. 16,
  // with enough weight copies rotated that every call streams its weights from HBM.
  const int pct = env_int("W4_SKINNY_PARTIAL_PCT", 10);
  // Split-K factor for tile width tt (row blocks of 16 tt columns in rb).
  auto plan_splits = [&](int tt, int& rb) {
    rb = (N + 16 * tt - 1) / (16 * tt);
    // (split only below 160 column blocks: the fixup and the partial traffic cost more
    // than the extra parallelism above that, on every decode shape swept)
    const int tgt = env_int("W4_SKINNY_BLOCKS", 160);
    int sp = (tgt + rb - 1) / rb;
    sp = min(sp, ng / max(waves, p.waves));  // at least one group per wave
    // keep the split-K partial traffic (2 * splits * M * N * 4 bytes) near 10% of the
    // codes (N * K / 2 bytes): splits <= K / (160 M)
    sp = min(sp, max(1, (int)((int64_t)K * pct / (1600LL * M))));
    sp = max(1, sp);
    // a full wave of workgroups needs no split (the fixup costs ~1.5 us on short calls)
    if (rb >= 256 || rb >= kMaxCounters) sp = 1;
    return sp;
  };
  const bool narrow = p.mt == 1 && N <= 8192;
  t = env_int("W4_SKINNY_TILES", 0);
  if (t < 1 || t > 8) {
    // (4 < M <= 8 with long K: 4 tiles, 8 waves, split K -- down 13824 x 5120 at M = 8:
    // 13.1 -> 11.9 us)
    const bool longk = M > 4 && M <= 8 && K > 8192;
    if (M <= 8) t = (N > 8192 || longk) ? 4 : 2;
    else if (M <= 16) t = 4;  // (2 below when 4 leaves under 128 workgroups)
    // 16 < M <= 32 (two m-tiles): 8 tiles on wide matrices, 4 when N gives >= 128
    // column blocks or K is long (gate+up at M = 32 31.0 -> 23.9 us, down 30.0 -> 21.0)
    else t = N > 16384 ? 8 : (((N + 63) / 64 >= 128 || K > 8192) ? 4 : 2);
    int rb1 = 0, rb2 = 0;
    // M <= 8: narrower tiles while the column blocks alone give under 160 workgroups
    // and half the width does not
    while (M <= 8 && !longk && t > 1 && (N + 16 * t - 1) / (16 * t) < 160 && (N + 8 * t - 1) / (8 * t) >= 160) t /= 2;
    // 8 < M <= 16: 4 tiles share each X fragment, unless that leaves under 128 workgroups
    if (M > 8 && M <= 16 && t == 4 && plan_splits(4, rb1) * rb1 < 128 && plan_splits(2, rb2) * rb2 >= 128) t = 2;
    // wide matrices at M <= 16: the fewest tiles (at most 8) that still give one column
    // block per CU, so that every CU streams the same share (gate+up 5120 x 27648: 7
    // tiles, 247 workgroups; at M = 1 / 8 / 16 15.1-15.7 -> 14.9, 16.5 -> 15.9, 18.1 ->
    // 17.7 us against 4 tiles on 432 workgroups or 8 tiles on 216)
    if (M <= 16 && N > 16384) t = min(8, (N + 4095) / 4096);
    // narrow matrices (N <= 8192) at 4 < M <= 16: 2 tiles, or 4 on long K past M = 8, with
    // X loaded as whole rows (below; O 5120 x 5120 at M = 8 / 16 7.2 -> 6.6 / 9.1 -> 8.0 us,
    // down 13824 x 5120 13.2 -> 12.1 / 15.2 -> 14.3, single 4096 x 4096 at M = 8 7.7 -> 6.8)
    if (narrow && M > 4) t = (M > 8 && K > 8192) ? 4 : 2;
  }
  // (the dequantizing kernel exists for 1, 2 and 4 tiles)
  if ((group_size == 64 || group_size == 32) && t != 1 && t != 2 && t != 4) t = t > 4 ? 4 : 2;
  p.tiles = t;
  p.depth = t == 1 ? 4 : 2;
  // 8 waves for narrow workgroups at M <= 8 (more groups in flight per column block:
  // O 5120 x 5120 at M = 1 6.4 -> 5.5 us, down 13824 x 5120 at M = 4 12.2 -> 10.1 us)
  // and for the 8-tile ones
  p.waves = (p.mt == 1 && ((M <= 8 && (t <= 2 || K > 8192)) || t == 8 || narrow)) ? 8 : 4;
  p.xs = 0;
  if (!skinny_variant_compiled(p) || group_size == 64 || group_size == 32) p.waves = 4;
  if (group_size != 64 && group_size != 32) {
    // 4-tile, 4-wave workgroups below 16384 columns keep a third group of loads in
    // flight (weights streamed from HBM: QKV 5120 x 15360 at M = 1-8 ~11.0 -> ~9.9 us,
    // O 5120 x 5120 at M = 16 9.7 -> 9.2 us, down 13824 x 5120 at M = 16 15.9 -> 15.5 us)
    // (at 8 < M <= 16 two deep with X loaded as whole rows: QKV 5120 x 15360 at M = 16
    // 11.9 -> 11.3 us)
    if (p.mt == 1 && p.tiles == 4 && p.waves == 4 && N <= 16384 && M <= 8) p.depth = 3;
    // variants (sweeps): prefetch depth, 8-wave workgroups
    SkinnyPlan q = p;
    q.depth = env_int("W4_SKINNY_RDEPTH", p.depth);
    // one row on narrow matrices: 12 waves (three per SIMD) with X as whole rows (down
    // 13824 x 5120 10.5 -> 9.9 us, O 5120 x 5120 5.9 -> 5.8; at M = 4 no better)
    q.waves = env_int("W4_SKINNY_WAVES", narrow && M == 1 && p.tiles == 2 && p.depth == 2 ? 12 : p.waves);
    // X loaded as whole rows, ceil(M / 4) 16-byte loads per lane and group (fragments
    // formed in LDS) instead of four fragment loads: at 8 < M <= 16 (QKV 5120 x 15360 at
    // M = 16 11.9 -> 11.3 us; gate+up 5120 x 27648 with 7 tiles and 4 waves 17.4 -> 16.8
    // against 8 waves without), and on narrow matrices with two or more tiles (down
    // 13824 x 5120 at M = 1 / 4 11.5 -> 10.5 / 12.1 -> 10.6 us); slower on QKV at M <= 8
    // and with 7 tiles on wide matrices at M <= 8 (gate+up at M = 4: 14.9 against 16.4 us)
    const bool xs_dflt = M > 8 || (narrow && q.tiles >= 2);
    q.xs = p.mt == 1 && ((q.tiles > 1 && q.depth <= 2 && q.waves <= 8) || M <= 4) ? env_int("W4_SKINNY_XS", xs_dflt) : 0;
    // (two m-tiles: all 32 rows in eight loads per lane and group, whatever M, so it pays
    // only near 32 rows: at M = 32 O 5120 x 5120 14.5 -> 11.6 us, QKV 5120 x 15360 16.9 ->
    // 15.7, down 13824 x 5120 21.1 -> 20.4; it pays from M = 21 on O, 27 on QKV, 29 on down,
    // and is slower below)
    if (p.mt == 2 && q.tiles > 1 && q.depth <= 2 && q.waves <= 8)
      q.xs = env_int("W4_SKINNY_XS", M > (K > 8192 ? 28 : N <= 8192 ? 20 : 26));
    if (skinny_variant_compiled(q)) p = q;
    // (a tile width forced by a tuning variable without a compiled variant for its m-tiles
    // falls back to the widest power of two below it, 4 waves)
    if (!skinny_variant_compiled(p)) {
      t = t >= 4 ? 4 : t >= 2 ? 2 : 1;
      p.tiles = t;
      p.depth = t == 1 ? 4 : 2;
      p.waves = 4;
      p.xs = 0;
    }
  }
  int splits = plan_splits(t, p.row_blocks);
  p.gps = (ng + splits - 1) / splits;
  p.splits = (ng + p.gps - 1) / p.gps;
  return p;
}

size_t skinny_workspace_bytes(const SkinnyPlan& p, int M, int N) {
  if (p.splits == 1) return 0;
  return kCounterRegionBytes + (size_t)p.splits * M * N * sizeof(float);
}

hipError_t launch_skinny(const SkinnyPlan& p, const void* x, const int32_t* qweight, const void* scales,
                         const int32_t* qzeros, void* y, void* ws, int M, int N, int K, int group_size,
                         hipStream_t stream) {
  const int glog = group_log2(group_size);
  const bool dq = group_size == 64 || group_size == 32;
  unsigned* counters = (unsigned*)ws;
  float* partials = ws ? (float*)((char*)ws + kCounterRegionBytes) : nullptr;
  const dim3 grid(p.row_blocks, p.splits);
  const half_t* xh = (const half_t*)x;
  const uint32_t* qw = (const uint32_t*)qweight;
  const half_t* sc = (const half_t*)scales;
  const uint32_t* qz = (const uint32_t*)qzeros;
  half_t* yh = (half_t*)y;
  if (p.lds) {
    const dim3 block(64 * p.wn * p.wk);
#define LDS_LAUNCH1(T, D, ONE)                                                                                \
  hipLaunchKernelGGL((skinny_lds_kernel<T, D, ONE>), grid, block, p.smem, stream, xh, qw, sc, qz, yh, counters, \
                     partials, M, N, K, p.splits, p.gps, p.wn, p.drain, glog)
#define LDS_LAUNCH(T, D) \
  if (M == 1) LDS_LAUNCH1(T, D, true); else LDS_LAUNCH1(T, D, false)
    if (p.tiles == 1) { if (p.depth == 4) LDS_LAUNCH(1, 4); else LDS_LAUNCH(1, 8); }
    else if (p.tiles == 2) { LDS_LAUNCH(2, 4); }
    else { LDS_LAUNCH(4, 2); }
#undef LDS_LAUNCH
#undef LDS_LAUNCH1
    return hipGetLastError();
  }
  const int key = variant_key(p.mt, p.tiles, p.depth, p.waves, p.xs);
  if (dq) {
#define DQ_LAUNCH(MT, T, D)                                                                                    \
  hipLaunchKernelGGL((skinny_kernel<MT, T, D, 4, true>), grid, dim3(4 * kWave), 0, stream, xh, qw, sc, qz, yh, \
                     counters, partials, M, N, K, p.splits, p.gps, p.drain, glog)
    switch (p.mt * 10 + p.tiles) {
      case 14: DQ_LAUNCH(1, 4, 2); break;
      case 12: DQ_LAUNCH(1, 2, 2); break;
      case 11: DQ_LAUNCH(1, 1, 4); break;
      case 24: DQ_LAUNCH(2, 4, 2); break;
      case 22: DQ_LAUNCH(2, 2, 2); break;
      default: DQ_LAUNCH(2, 1, 4); break;
    }
#undef DQ_LAUNCH
    return hipGetLastError();
  }
#define V(MT, T, D, W, XS)                                                                                   \
  if (key == variant_key(MT, T, D, W, XS)) {                                                                 \
    if constexpr (XS == 0) {                                                                                 \
      hipLaunchKernelGGL((skinny_kernel<MT, T, D, W, false, 0>), grid, dim3(W * kWave), 0, stream, xh, qw, sc, qz, \
                         yh, counters, partials, M, N, K, p.splits, p.gps, p.drain, glog);                   \
    } else if constexpr (MT == 2) { /* two m-tiles: the 32 rows in 8 loads */                              \
      if constexpr (T > 1 && D <= 2 && W <= 8)                                                               \
        hipLaunchKernelGGL((skinny_kernel<MT, T, D, W, false, 8>), grid, dim3(W * kWave), 0, stream, xh, qw, sc, qz, \
                           yh, counters, partials, M, N, K, p.splits, p.gps, p.drain, glog);                 \
      else                                                                                                   \
        return hipErrorInvalidValue;                                                                         \
    } else if (M > 4) { /* (the plan takes XS at M > 4 only with two-deep, multi-tile variants of at most 8 waves) */ \
      if constexpr (T > 1 && D <= 2 && W <= 8) {                                                             \
        if (M > 8)                                                                                           \
          hipLaunchKernelGGL((skinny_kernel<MT, T, D, W, false, 4>), grid, dim3(W * kWave), 0, stream, xh, qw, sc, \
                             qz, yh, counters, partials, M, N, K, p.splits, p.gps, p.drain, glog);           \
        else                                                                                                 \
          hipLaunchKernelGGL((skinny_kernel<MT, T, D, W, false, 2>), grid, dim3(W * kWave), 0, stream, xh, qw, sc, \
                             qz, yh, counters, partials, M, N, K, p.splits, p.gps, p.drain, glog);           \
      } else {                                                                                               \
        return hipErrorInvalidValue;                                                                         \
      }                                                                                                      \
    } else {                                                                                                 \
      hipLaunchKernelGGL((skinny_kernel<MT, T, D, W, false, 1>), grid, dim3(W * kWave), 0, stream, xh, qw, sc, qz, \
                         yh, counters, partials, M, N, K, p.splits, p.gps, p.drain, glog);                   \
    }                                                                                                        \
    return hipGetLastError();                                                                                \
  }
  SKINNY_VARIANTS(V)
#undef V
  return hipErrorInvalidValue;
}

}  // namespace w4
