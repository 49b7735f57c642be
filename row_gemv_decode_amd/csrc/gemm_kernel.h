// gemm_kernel.h -- the MFMA GEMM (f16 / bf16 / block-quantised weights) for
// the m >= 17 regime on gfx950 (MI355X): the kernel template, the tile list
// and the per-weight-kind launcher that gemm_inst.hip instantiates (once per
// weight kind, so the many kernels compile in parallel).
//
// C[M,N] = A[M,K] . W[K,N] with W stored [N][K] (both operands k-contiguous),
// fp32 accumulation in the matrix cores, f32/f16/bf16 output.
//
// What the pages fix, and how it is met here:
//   * opus r35 track A, section 2 ("gemm_f16 tiles"): a family of tiles
//     TM x TN whose results are bitwise identical, chosen per M.  Here every
//     tile issues the same instruction, v_mfma_f32_32x32x16_{f16,bf16}, with
//     the same operand layout, and accumulates every output in one register
//     over k = 0, 16, 32, ... in increasing order, and every tile origin is a
//     multiple of 32 rows and columns.  So an output element sees the same
//     arithmetic under every tile and every M (tile- and M-invariance).
//   * the same section's tail rule (a 128-row tile whose last block is up to
//     half padding loses): rows past M lie outside the block's buffer
//     resource and reach only outputs that are never stored; the plan's
//     selector counts padded tiles when it picks a tile.
//   * opus r35 track A, section 1 (`dq_f16` before the router GEMM): Q8_0
//     codes and scales are loaded into LDS as stored and each B fragment is
//     dequantised as it is read, with the same function as the standalone
//     dequant, so no separate dequant pass or f16 copy of the weight exists.
//   * a plan may cut k into chunks (fixed per plan from N, K and the CU
//     count, never from M, so M-invariance holds within a plan).  Each m then
//     runs either one block per chunk writing fp32 partial sums, added in
//     chunk order by a second launch, or one launch whose blocks walk all
//     chunks and fold each chunk's sum into a running total at the chunk's
//     end -- the same additions in the same order, so both give the same
//     bits.  Chunking changes the rounding against an unchunked sum, never
//     between tiles, launch shapes or calls.
//
// Structure (64-wide wavefronts, 1 to 8 waves per block):
//   * k-tiles of 64 (four MFMA steps per barrier);
//   * global loads go straight into LDS (buffer_load ... lds) through buffer
//     resources that cover exactly the block's rows, NS k-tiles in flight; one
//     barrier per k-tile (below);
//   * blocks are renumbered so that each XCD (blocks b, b + 8, ... share one)
//     runs a contiguous range of tiles, ordered so that the larger operand's
//     tiles an XCD needs stay in its own L2 instead of all eight;
//   * LDS rows are 128 bytes (eight 16-byte chunks); chunk c of row r is
//     stored at c ^ ((r >> 1) & 7), so the sixteen rows read by sixteen
//     consecutive lanes at one logical chunk hit sixteen different 16-byte
//     bank groups (the bank-conflict counter reads zero);
//   * MFMA operand fragments are read ahead of their MFMAs: one k-step ahead
//     for large wave tiles, one whole k-tile ahead for small ones.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace skinny {

namespace {

// buffer resource word 3 for raw (unstrided) 32-bit buffers on gfx9-family
// parts; out-of-range offsets read as zero
constexpr int kBufferFlags = 0x00020000;

constexpr int kBK = 64;        // k per LDS tile: four 32x32x16 MFMA steps
constexpr int kCPR = kBK / 8;  // 16-byte chunks per tile row (8)
constexpr int kSteps = kBK / 16;

// LDS rows are 128 bytes; gfx950 serves 16 lanes of a ds_read_b128 per cycle
// from 64 banks (256 bytes), i.e. two rows.  Chunk c of row r goes to
// c ^ ((r >> 1) & 7): the 16 rows read by 16 consecutive lanes at one logical
// chunk then cover all 16 bank groups of the two-row window.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ h8_t as_h8(u32x4 v) { return __builtin_bit_cast(h8_t, v); }
__device__ __forceinline__ b8_t as_b8(u32x4 v) { return __builtin_bit_cast(b8_t, v); }

template <int WK>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (WK == WK_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_b8(a), as_b8(b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(a), as_h8(b), c, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// The GEMM kernel: global loads go straight into LDS (buffer_load ... lds),
// so NS k-tiles can be in flight without staging registers.  Per k-tile: wait until this wave's loads of tile kt have
// landed (NS - 2 later tiles may stay in flight), one barrier (every wave's
// part of tile kt is in LDS and every wave is done with tile kt - 1), issue
// tile kt + NS - 1 into the stage tile kt - 1 used, run tile kt's MFMAs.
// A lane's 16 bytes land at the wave's LDS base + 16 * lane, so the chunk
// swizzle is applied on the global side: lane l of a load fills slot l % 8 of
// row l / 8 with global chunk (l % 8) ^ swz(row).  Rows past M or N lie
// outside the buffer resources: whatever their LDS slots hold reaches only
// outputs that are never stored.  For a K % 64 != 0 shape the chunks past K
// of the last k-tile are zeroed in LDS before its fragments are read.  The
// MFMA sequence of every output is the same under every tile: same bits.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) not waited on
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// a workgroup barrier without the memory fence __syncthreads() adds (the
// fence would wait for every load in flight); the signal fences keep the
// compiler from moving LDS accesses across it
__device__ __forceinline__ void barrier_only() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// 32-bit LDS address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// buffer resource for raw 16-byte loads of `bytes` bytes from `base`
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xFFFFu, (uint32_t)bytes, (uint32_t)kBufferFlags};
}

// The kernel body is written as lambdas; each must be inlined: a lambda the
// inliner leaves out of line becomes a call whose arguments the compiler can
// no longer prove wave-uniform, so the scalar operands of the LDS DMA asm
// below would not compile (and a call in the k loop would cost far more).
#define INLINE_LAMBDA __attribute__((always_inline))

// One 16-byte-per-lane load straight into LDS: lane l's bytes land at
// lds + 16 * l.  Issued from asm so that the compiler neither counts it nor
// orders LDS reads after it: the kernel waits for it explicitly (vmcnt and a
// barrier) before any wave reads the stage.  There is no output register;
// M0, which holds the LDS address, is restored before the asm ends.
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, uint32_t lds, int voff, int soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// the same for 4 bytes per lane (lane l's word lands at lds + 4 * l)
__device__ __forceinline__ void lds_dma4(const u32x4& rsrc, uint32_t lds, int voff, int soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}


// Q8_0 weights: each k-tile of a weight row is 64 codes (four 16-byte slots,
// slot s of row r holding code piece s ^ q8_swz(r)) plus its two f16 scales
// (one 32-bit word per row).  A B fragment is dequantised when it is read from
// LDS, by the same function as every other path, so it equals the f16 weight.
__device__ __forceinline__ int q8_swz(int r) { return (r >> 2) & 3; }

// Q4_0 weights: a row's k-tile is 64 codes in 32 bytes (two 16-byte slots,
// slot s of row r holding chunks 4 s .. 4 s + 3 at s ^ q4_swz(r)) plus the
// same two scales per row as Q8_0.
__device__ __forceinline__ int q4_swz(int r) { return (r >> 3) & 1; }

// Q2_0 weights: a row's k-tile is 64 codes in one 16-byte slot (chunk c in
// bits 16 (c & 1) .. 16 (c & 1) + 15 of its dword c >> 1) plus the same two
// scales per row; one load instruction of a wave fills 64 rows.

// four adjacent outputs in one store (8 bytes of f16 / bf16, 16 of fp32),
// each rounded exactly as store_out rounds it; idx is a multiple of 4
template <int CK>
__device__ __forceinline__ void store_out4(void* base, int64_t idx, const float (&v)[4]) {
  if constexpr (CK == CK_F32) {
    *(u32x4*)((float*)base + idx) = u32x4{__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                                          __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
  } else if constexpr (CK == CK_F16) {
    const h2_t lo = {(_Float16)v[0], (_Float16)v[1]};
    const h2_t hi = {(_Float16)v[2], (_Float16)v[3]};
    *(u32x2*)((uint16_t*)base + idx) = u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  } else {
    const b2_t lo = {(__bf16)v[0], (__bf16)v[1]};
    const b2_t hi = {(__bf16)v[2], (__bf16)v[3]};
    *(u32x2*)((uint16_t*)base + idx) = u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  }
}

// eight adjacent f16 / bf16 outputs in one 16-byte store; idx is a multiple of 8
template <int CK>
__device__ __forceinline__ void store_out8(void* base, int64_t idx, const float (&lo)[4], const float (&hi)[4]) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    if constexpr (CK == CK_F16) {
      w[e] = __builtin_bit_cast(uint32_t, h2_t{(_Float16)lo[2 * e], (_Float16)lo[2 * e + 1]});
      w[2 + e] = __builtin_bit_cast(uint32_t, h2_t{(_Float16)hi[2 * e], (_Float16)hi[2 * e + 1]});
    } else {
      w[e] = __builtin_bit_cast(uint32_t, b2_t{(__bf16)lo[2 * e], (__bf16)lo[2 * e + 1]});
      w[2 + e] = __builtin_bit_cast(uint32_t, b2_t{(__bf16)hi[2 * e], (__bf16)hi[2 * e + 1]});
    }
  }
  *(u32x4*)((uint16_t*)base + idx) = w;
}

template <int TM, int TN, int WM, int WN, int NS, bool XT, bool CH, int WK, int CK, bool FD = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_lds_kernel(GemmArgs g) {
  static_assert(!(CH && FD), "a launch folds chunk sums in-block or across blocks, not both");
  constexpr bool Q8 = WK == WK_Q8;
  constexpr bool Q4 = WK == WK_Q4;
  constexpr bool Q2 = WK == WK_Q2;
  constexpr bool QB = Q8 || Q4 || Q2;  // block-quantised: codes + per-32 scales
  // block-quantised code rows: bytes per row per k-tile, lanes per row in one
  // 16-byte-per-lane load, rows per load instruction
  constexpr int kBpr = Q2 ? 16 : Q4 ? 32 : 64;
  constexpr int kLpr = kBpr / 16;
  constexpr int kRpl = 64 / kLpr;
  constexpr int NW = WM * WN;
  constexpr int WTM = TM / WM;
  constexpr int WTN = TN / WN;
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  // one load instruction of one wave fills 8 rows of 16-bit data (64 lanes x
  // 16 bytes), 16 rows of Q8_0 codes (32 of Q4_0, 64 of Q2_0), or the scale
  // words of 64 rows; a block-quantised stage rounds its code and scale rows
  // up to whole instructions (rows past the tile lie outside the weight's
  // buffer resource, read as 0 and are never used)
  static_assert(TM % (8 * NW) == 0 && (QB || TN % (8 * NW) == 0), "tile rows must split evenly over the waves");
  constexpr int A_ITERS = TM / (8 * NW);
  constexpr int B_ITERS = QB ? (TN + kRpl * NW - 1) / (kRpl * NW) : TN / (8 * NW);
  constexpr int S_ITERS = QB ? (TN + 64 * NW - 1) / (64 * NW) : 0;
  constexpr int LOADS = A_ITERS + B_ITERS + S_ITERS;  // per lane per k-tile
  static_assert(NS >= 2 && (NS - 2) * LOADS < 64, "stages");
  // XT: read the next k-tile's fragments during this one's MFMAs (small wave
  // tiles; needs a third stage and (FM + FN) * 32 fragment registers)
  constexpr bool kCrossTile = XT;
  constexpr bool kMfmaPriority = TM == 256 && TN == 256 && NW == 8;
  static_assert(!XT || (FM + FN <= 4 && NS >= 3), "cross-tile fragment reads");
  constexpr int SA = TM * kCPR;                              // u32x4 per stage
  constexpr int SB = QB ? B_ITERS * 64 * NW : TN * kCPR;  // u32x4 per stage (1 KiB per wave load)
  constexpr int SS = QB ? S_ITERS * 64 * NW : 1;          // scale words per stage

  __shared__ u32x4 sA[NS][SA];
  __shared__ u32x4 sB[NS][SB];
  __shared__ uint32_t sS[NS][SS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid / WN;
  const int wn = wid - wm * WN;

  // XCD-aware renumbering: hardware block b runs on XCD b % 8; XCD x gets the
  // tiles [x * per, (x + 1) * per) of one tile order (the last XCDs may get
  // one fewer).  The order keeps the larger operand's tiles together on an
  // XCD, so that XCD's L2 serves them to its blocks: column-major (blocks of
  // one XCD share W columns) when N >= M, row-major (they share A rows) when
  // M > N.  The order changes no result.
  const int64_t tiles_m = (g.M + TM - 1) / TM;
  const int64_t tiles_n = (g.N + TN - 1) / TN;
  const int64_t nblocks = (int64_t)gridDim.x;
  const int64_t per = (nblocks + 7) / 8;
  const int64_t xcd = blockIdx.x & 7;
  const int64_t full = nblocks - 8 * (per - 1);
  const int64_t local = blockIdx.x >> 3;
  const int64_t tv = xcd < full ? xcd * per + local : full * per + (xcd - full) * (per - 1) + local;
  // split-major: the blocks of one k range sit together, so neighbours share
  // operand k-slices
  const int64_t tiles = tiles_m * tiles_n;
  const int split = (int)(tv / tiles);
  const int64_t t = tv - (int64_t)split * tiles;
  int64_t bm, bn;
  if (g.M > g.N) {
    bm = t / tiles_n;
    bn = t - bm * tiles_n;
  } else {
    bn = t / tiles_m;
    bm = t - bn * tiles_m;
  }
  const int64_t row0 = bm * TM;
  const int64_t col0 = bn * TN;

  const int64_t K = g.K;  // <= 2^20 (checked by the plan), so offsets fit in 32 bits
  const int nk_all = (int)((K + kBK - 1) / kBK);
  // this block's k-tiles: [kb, kb + nk) -- one chunk per block in a split
  // launch, all of k otherwise (a chunked launch folds at chunk ends)
  const int span = g.splits > 1 ? g.kt_per_split : nk_all;
  const int kb = split * span;
  const int nk = (nk_all - kb) < span ? (nk_all - kb) : span;
  const bool last_split = kb + nk == nk_all;
  const int64_t rows_a = (g.M - row0) < TM ? (g.M - row0) : TM;
  const int64_t rows_b = (g.N - col0) < TN ? (g.N - col0) : TN;
  const u32x4 rsrc_a = buffer_rsrc(g.A + row0 * g.lda, ((rows_a - 1) * g.lda + K) * 2);
  const int64_t wrow = QB ? K * kBpr / 64 : K * 2;  // bytes of a stored weight row
  const u32x4 rsrc_b = buffer_rsrc((const uint8_t*)g.W + col0 * wrow, rows_b * wrow);
  const u32x4 rsrc_s = QB ? buffer_rsrc(g.scales + col0 * (K >> 5), rows_b * (K >> 5) * 2) : rsrc_b;
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);

  // per-lane global offsets of each load (row r = 8 * (i * NW + wid) + lane / 8)
  const int lr = lane >> 3;
  const int ls = lane & 7;
  int voff_a[A_ITERS];
  int voff_b[B_ITERS];
  int voff_s[S_ITERS > 0 ? S_ITERS : 1];
#pragma unroll
  for (int i = 0; i < A_ITERS; ++i) {
    const int r = 8 * (i * NW + wid) + lr;
    voff_a[i] = (int)(((int64_t)r * g.lda + (ls ^ swz(r)) * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < B_ITERS; ++i) {
    if constexpr (QB) {
      const int r = kRpl * (i * NW + wid) + lane / kLpr;
      const int slot = Q2 ? 0 : (lane % kLpr) ^ (Q4 ? q4_swz(r) : q8_swz(r));
      voff_b[i] = (int)((int64_t)r * wrow + slot * 16);
    } else {
      const int r = 8 * (i * NW + wid) + lr;
      voff_b[i] = (int)(((int64_t)r * K + (ls ^ swz(r)) * 8) * 2);
    }
  }
#pragma unroll
  for (int i = 0; i < S_ITERS; ++i) {
    const int r = 64 * (i * NW + wid) + lane;
    voff_s[i] = (int)((int64_t)r * (K >> 5) * 2);
  }

  // An odd number of scales per row (K % 64 == 32) leaves one scale in the
  // matrix's last k-tile; the word at its usual place would run 2 bytes past
  // the row (past the buffer for the tile's last row, which then reads as 0),
  // so that k-tile's word is fetched 2 bytes earlier and its scale is the
  // high half.  The other half belongs to k past K, whose products are masked.
  const bool qb_odd = QB && ((K >> 5) & 1) != 0;
  auto scale_shift = [&](int kc) INLINE_LAMBDA -> bool { return qb_odd && kc == nk_all - 1; };

  // local k-tile kt (0 .. nk - 1; later ones are clamped to the last, so
  // every k-tile issues the same number of loads and the waits count
  // exactly) into stage st
  auto issue = [&](int st, int kt) INLINE_LAMBDA {
    const int kc = kb + (kt < nk ? kt : nk - 1);
    const int koff = kc * kBK * 2;  // bytes of a 16-bit row
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i)
      lds_dma16(rsrc_a, lds_addr(&sA[st][(8 * (i * NW + wid_u)) * kCPR]), voff_a[i], koff);
    if constexpr (QB) {
#pragma unroll
      for (int i = 0; i < B_ITERS; ++i)
        lds_dma16(rsrc_b, lds_addr(&sB[st][64 * (i * NW + wid_u)]), voff_b[i], kc * kBpr);
#pragma unroll
      for (int i = 0; i < S_ITERS; ++i)
        lds_dma4(rsrc_s, lds_addr(&sS[st][64 * (i * NW + wid_u)]), voff_s[i],
                 kc * 4 - (scale_shift(kc) ? 2 : 0));
    } else {
#pragma unroll
      for (int i = 0; i < B_ITERS; ++i)
        lds_dma16(rsrc_b, lds_addr(&sB[st][(8 * (i * NW + wid_u)) * kCPR]), voff_b[i], koff);
    }
  };

  // one B fragment: 8 weights of row `row` at k-chunk c (of 8) of a stage;
  // sh: the stage holds a k-tile whose scale word was fetched shifted
  auto read_b = [&](int st, bool sh, int row, int c) INLINE_LAMBDA -> u32x4 {
    if constexpr (Q8) {
      const uint32_t* codes = reinterpret_cast<const uint32_t*>(&sB[st][0]);
      const int w = row * 16 + (((c >> 1) ^ q8_swz(row)) * 4) + (c & 1) * 2;
      const u32x2 q = *reinterpret_cast<const u32x2*>(codes + w);
      const uint32_t sc = sS[st][row];
      const int hi = (c >> 2) | (int)sh;
      return q8_dequant8(q, half_from_bits((uint16_t)(hi ? (sc >> 16) : sc)));
    } else if constexpr (Q4) {
      const uint32_t* codes = reinterpret_cast<const uint32_t*>(&sB[st][0]);
      const uint32_t q = codes[row * 8 + (((c >> 2) ^ q4_swz(row)) * 4) + (c & 3)];
      const uint32_t sc = sS[st][row];
      const int hi = (c >> 2) | (int)sh;
      return q4_dequant8(q, half_from_bits((uint16_t)(hi ? (sc >> 16) : sc)));
    } else if constexpr (Q2) {
      const uint32_t* codes = reinterpret_cast<const uint32_t*>(&sB[st][0]);
      const uint32_t w = codes[row * 4 + (c >> 1)];
      const uint32_t sc = sS[st][row];
      const int hi = (c >> 2) | (int)sh;
      return q2_dequant8((c & 1) ? (w >> 16) : w, half_from_bits((uint16_t)(hi ? (sc >> 16) : sc)));
    } else {
      return sB[st][row * kCPR + (c ^ swz(row))];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // CH (one launch for a plan whose k is cut into chunks of kt_per_split
  // k-tiles): acc holds the current chunk's sum, started from zero as a
  // split block would; at each chunk end it is folded into tot -- the first
  // chunk copied, later ones added in order -- exactly the additions the
  // split-k reduce launch makes, so both launch shapes give the same bits.
  f32x16 tot[CH ? FM : 1][CH ? FN : 1];
  bool have_tot = false;
  auto fold = [&]() INLINE_LAMBDA {
    if constexpr (CH) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            tot[i][j][v] = have_tot ? tot[i][j][v] + acc[i][j][v] : acc[i][j][v];
            acc[i][j][v] = 0.0f;
          }
      have_tot = true;
    }
  };

  const int lrow = lane & 31;
  const int lk = lane >> 5;
  int a_row[FM];
  int b_row[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_row[i] = wm * WTM + i * 32 + lrow;
#pragma unroll
  for (int j = 0; j < FN; ++j) b_row[j] = wn * WTN + j * 32 + lrow;

  const bool k_tail = (K % kBK) != 0;

  // prologue: tiles 0 .. NS - 2 into stages 0 .. NS - 2
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) issue(st, st);

  // K % 64 != 0: the last k-tile runs outside the loop, and there the
  // fragments past K are zeroed (in both operands) before its MFMAs
  auto mask_tail = [&](int ks, u32x4 (&af)[FM], u32x4 (&bf)[FN]) INLINE_LAMBDA {
    if (k_tail && last_split && (int64_t)(kb + nk - 1) * kBK + ks * 16 + lk * 8 >= K) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = zero;
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = zero;
    }
  };

  if constexpr (kCrossTile) {
    // Small wave tiles: one MFMA per fragment pair cannot hide an LDS read,
    // so tile kt + 1's fragments (all four k-steps) are read while tile kt's
    // MFMAs run on the fragments read one iteration earlier.  Iteration kt:
    // wait for this lane's part of tile kt + 1 (NS - 3 later tiles may stay in
    // flight), barrier (tile kt + 1 is in LDS; every wave has its tile-kt
    // fragments in registers, so the stages of tiles kt - 1 and kt are free),
    // refill the stage of tile kt - 1 with tile kt + NS - 1, read tile kt + 1,
    // multiply tile kt.
    u32x4 fa[2][kSteps][FM];
    u32x4 fb[2][kSteps][FN];
    auto read_tile = [&](int st, bool sh, u32x4 (&ta)[kSteps][FM], u32x4 (&tb)[kSteps][FN]) INLINE_LAMBDA {
      const u32x4* a_s = sA[st];
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) {
        const int c = ks * 2 + lk;
#pragma unroll
        for (int i = 0; i < FM; ++i) ta[ks][i] = a_s[a_row[i] * kCPR + (c ^ swz(a_row[i]))];
#pragma unroll
        for (int j = 0; j < FN; ++j) tb[ks][j] = read_b(st, sh, b_row[j], c);
      }
    };
    auto mma_tile = [&](u32x4 (&ta)[kSteps][FM], u32x4 (&tb)[kSteps][FN], bool last) INLINE_LAMBDA {
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) {
        if (last) mask_tail(ks, ta[ks], tb[ks]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<WK>(tb[ks][j], ta[ks][i], acc[i][j]);
      }
    };
    wait_vmcnt<(NS - 2) * LOADS>();  // tile 0
    barrier_only();
    read_tile(0, false, fa[0], fb[0]);
    int stage = 0;  // stage of tile kt
    int kt = 0;
    // one trip: tile kt's MFMAs on fragment set H while tile kt + 1 is read
    // into the other set
    auto trip = [&](auto hc) INLINE_LAMBDA {
      constexpr int H = decltype(hc)::value;
      wait_vmcnt<(NS - 3) * LOADS>();
      barrier_only();
      issue(stage == 0 ? NS - 1 : stage - 1, kt + NS - 1);
      stage = stage + 1 == NS ? 0 : stage + 1;
      read_tile(stage, false, fa[H ^ 1], fb[H ^ 1]);
      mma_tile(fa[H], fb[H], false);
      ++kt;
    };
    // tiles kt .. stop - 1 (kt even on entry): trips in pairs, so the loop
    // body is one straight-line block with the fragment sets named at compile
    // time and the loop has a single exit; an odd count leaves one trip after
    auto run_to = [&](const int stop) INLINE_LAMBDA {
      while (kt + 1 < stop) {
        trip(std::integral_constant<int, 0>{});
        trip(std::integral_constant<int, 1>{});
      }
      if (kt < stop) trip(std::integral_constant<int, 0>{});
    };
    if constexpr (CH) {
      // chunks hold an even number of k-tiles, so kt is even at each chunk
      // start; the fold sits between chunks; the global last tile is peeled
      for (;;) {
        const int cend = kt + g.kt_per_split < nk ? kt + g.kt_per_split : nk;
        run_to(cend < nk ? cend : nk - 1);
        if (cend == nk) break;
        fold();
      }
    } else {
      run_to(nk - 1);
    }
    // the last tile, read by the last trip (or the prologue) -- read again
    // from its stage, which nothing refills, when its scale word was fetched
    // shifted
    const bool last_sh = scale_shift(kb + nk - 1);
    if ((nk - 1) & 1) {
      if (last_sh) read_tile(stage, true, fa[1], fb[1]);
      mma_tile(fa[1], fb[1], true);
    } else {
      if (last_sh) read_tile(stage, true, fa[0], fb[0]);
      mma_tile(fa[0], fb[0], true);
    }
    fold();
  } else {
    // per k-tile: wait for this lane's part of tile kt (NS - 2 later tiles may
    // stay in flight), barrier (every wave's part has landed, and every wave is
    // done with the stage tile kt - 1 used), refill that stage with tile
    // kt + NS - 1, then the MFMAs of tile kt
    auto tile = [&](int kt, int st, bool last) INLINE_LAMBDA {
      wait_vmcnt<(NS - 2) * LOADS>();
      barrier_only();
      issue(st == 0 ? NS - 1 : st - 1, kt + NS - 1);
      const u32x4* a_s = sA[st];
      const bool sh = scale_shift(kb + kt);
      auto read_frags = [&](int ks, u32x4 (&af)[FM], u32x4 (&bf)[FN]) INLINE_LAMBDA {
        const int c = ks * 2 + lk;
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = a_s[a_row[i] * kCPR + (c ^ swz(a_row[i]))];
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = read_b(st, sh, b_row[j], c);
      };
      u32x4 af[2][FM];
      u32x4 bf[2][FN];
      read_frags(0, af[0], bf[0]);
      // the 8-wave 256 x 256 tile: a wave in its MFMA run goes first (2-3 % at
      // M = 2048; the other tiles measured the same or slower with it)
      if constexpr (kMfmaPriority) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) {
        if (ks + 1 < kSteps) read_frags(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
        if (last) mask_tail(ks, af[ks & 1], bf[ks & 1]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<WK>(bf[ks & 1][j], af[ks & 1][i], acc[i][j]);
      }
      if constexpr (kMfmaPriority) __builtin_amdgcn_s_setprio(0);
    };
    int stage = 0;
    int kt = 0;
    for (;;) {
      const int cend = CH ? (kt + g.kt_per_split < nk ? kt + g.kt_per_split : nk) : nk;
      const int stop = cend < nk ? cend : nk - 1;
      for (; kt < stop; ++kt) {
        tile(kt, stage, false);
        stage = stage + 1 == NS ? 0 : stage + 1;
      }
      if (cend == nk) break;
      fold();
    }
    tile(nk - 1, stage, true);
    fold();
  }
  wait_vmcnt<0>();  // the re-reads past the end land before the block exits

  // FD (one block per (tile, chunk), folded in this launch): every block
  // parks its chunk sum in the workspace slot of its (tile, chunk), in
  // register order (each lane's own values, so the stores and the loads
  // below are 256-byte rows per wave instruction), with device-coherent
  // stores; waits for them; and counts itself in on its tile.  The block
  // that arrives last adds the tile's chunk sums in chunk order -- the first
  // copied, each later one added -- exactly the additions of the reduce
  // launch and of the in-block chunk fold, so every launch shape gives the
  // same bits -- and writes C below.  The others are done.  No block waits
  // for another; the counter is left at zero.
  if constexpr (FD) {
    constexpr int64_t kSlot = (int64_t)TM * TN;
    const int64_t tile_id = bm * tiles_n + bn;
    float* slots = g.partial + tile_id * g.splits * kSlot;
    auto at = [&](int c, int i, int j, int v) INLINE_LAMBDA -> float* {
      return slots + c * kSlot + (((wid * FM + i) * FN + j) * 16 + v) * 64 + lane;
    };
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) st_dev(at(split, i, j, v), acc[i][j][v]);
    wait_mem();
    __shared__ uint32_t s_last;
    __syncthreads();  // every wave's chunk sum has reached the device-coherent level
    if (tid == 0) s_last = atomicAdd(&g.counters[tile_id], 1u) == (uint32_t)(g.splits - 1) ? 1u : 0u;
    __syncthreads();
    if (s_last == 0u) return;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        f32x16 tot;
        f32x16 p;
#pragma unroll
        for (int v = 0; v < 16; ++v) tot[v] = split == 0 ? acc[i][j][v] : ld_dev(at(0, i, j, v));
        for (int c = 1; c < g.splits; ++c) {
#pragma unroll
          for (int v = 0; v < 16; ++v) p[v] = c == split ? acc[i][j][v] : ld_dev(at(c, i, j, v));
#pragma unroll
          for (int v = 0; v < 16; ++v) tot[v] = tot[v] + p[v];
        }
        acc[i][j] = tot;
      }
    if (tid == 0) g.counters[tile_id] = 0u;  // every block of the tile has counted in
  }

  // The weight fragment is the MFMA's first operand, so lane l of a 32 x 32
  // block holds output row l % 32 and, in each group q of four registers,
  // the four adjacent columns 8 q + 4 (l / 32) .. + 3.  Stores are as wide as
  // the row stride's alignment allows: 16 bytes per lane (fp32, or 16-bit
  // output after the swap below), else element by element.  Where a value is
  // stored changes no bits.
  if (CK != CK_F32 && (CH || FD || g.splits == 1)) {
    // 16-bit output: lanes l and l + 32 trade halves of two groups
    // (v_permlane32_swap), so lane l holds columns 8 q .. 8 q + 7 of its row
    // and lane l + 32 the next eight: one 16-byte store per lane per group
    // pair.  Every lane takes part in the swap; the stores are masked after.
    const bool vec8 = (g.ldc & 7) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t row = row0 + wm * WTM + i * 32 + lrow;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; q += 2) {
          float lo[4], hi[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = CH ? tot[i][j][4 * q + e] : acc[i][j][4 * q + e];
            const float y = CH ? tot[i][j][4 * q + 4 + e] : acc[i][j][4 * q + 4 + e];
            const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                            __builtin_bit_cast(uint32_t, y), false, false);
            lo[e] = __builtin_bit_cast(float, (uint32_t)r[0]);
            hi[e] = __builtin_bit_cast(float, (uint32_t)r[1]);
          }
          const int64_t col = col0 + wn * WTN + j * 32 + 8 * (q + lk);
          const int64_t rem = g.N - col;
          if (row < g.M && rem > 0) {
            if (vec8 && rem >= 8) {
              store_out8<CK>(g.C, row * g.ldc + col, lo, hi);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (e < rem) store_out<CK>(g.C, row * g.ldc + col + e, lo[e]);
                if (4 + e < rem) store_out<CK>(g.C, row * g.ldc + col + 4 + e, hi[e]);
              }
            }
          }
        }
      }
    }
  } else {
    const bool vec_c = (g.ldc & 3) == 0;
    const bool vec_p = (g.N & 3) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t row = row0 + wm * WTM + i * 32 + lrow;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = col0 + wn * WTN + j * 32 + 8 * q + 4 * lk;
          const int64_t rem = g.N - col;
          float v4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = CH ? tot[i][j][4 * q + e] : acc[i][j][4 * q + e];
          if (row < g.M && rem > 0) {
            if (!CH && !FD && g.splits > 1) {
              float* dst = g.partial + ((int64_t)split * g.M + row) * g.N + col;
              if (vec_p && rem >= 4) {
                *(u32x4*)dst = u32x4{__builtin_bit_cast(uint32_t, v4[0]), __builtin_bit_cast(uint32_t, v4[1]),
                                     __builtin_bit_cast(uint32_t, v4[2]), __builtin_bit_cast(uint32_t, v4[3])};
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (e < rem) dst[e] = v4[e];
              }
            } else if (vec_c && rem >= 4) {
              store_out4<CK>(g.C, row * g.ldc + col, v4);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (e < rem) store_out<CK>(g.C, row * g.ldc + col + e, v4[e]);
            }
          }
        }
      }
    }
  }
}

typedef void (*gemm_fn)(GemmArgs);

// The tile family (one row per tile: TM, TN, WM, WN, NS, XT, name; indexed
// by tile id).  Stage counts: (TM + TN) * 128 bytes of LDS per stage, at
// most 144 KiB per block; the small tiles keep two blocks per CU.  XT where
// it measured faster on MI355X (K = 2560, N = 96 and 7680).
#define SKINNY_GEMM_TILE_LIST(X)                  \
  X(256, 256, 2, 2, 2, false, "256x256_w2x2")     \
  X(256, 256, 2, 4, 2, false, "256x256_w2x4")     \
  X(256, 128, 4, 2, 3, false, "256x128_w4x2")     \
  X(256, 128, 2, 2, 3, false, "256x128_w2x2")     \
  X(128, 256, 2, 2, 3, false, "128x256_w2x2")     \
  X(128, 128, 2, 2, 4, true, "128x128_w2x2")      \
  X(128, 64, 2, 2, 3, false, "128x64_w2x2")       \
  X(64, 128, 2, 2, 3, false, "64x128_w2x2")       \
  X(64, 64, 2, 2, 4, true, "64x64_w2x2")          \
  X(128, 96, 4, 1, 5, true, "128x96_w4x1")        \
  X(64, 96, 2, 1, 3, false, "64x96_w2x1")         \
  X(32, 96, 1, 1, 5, true, "32x96_w1x1")          \
  X(32, 64, 1, 2, 5, true, "32x64_w1x2")          \
  X(192, 128, 2, 2, 3, false, "192x128_w2x2")     \
  X(192, 256, 2, 4, 2, false, "192x256_w2x4")     \
  X(192, 192, 3, 2, 3, false, "192x192_w3x2")     \
  X(32, 32, 1, 1, 6, true, "32x32_w1x1")          \
  X(192, 96, 6, 1, 4, false, "192x96_w6x1")

// the chunked one-launch variant keeps a second set of accumulators, so only
// tiles with at most four 32 x 32 blocks per wave get it; the fold launch
// (which serves the same narrow-n plans) is built for the same tiles
constexpr bool gemm_chunkable(int tm, int tn, int wm, int wn) { return (tm / wm / 32) * (tn / wn / 32) <= 4; }

// one tile's kernels for weight kind WK, by output kind
struct TileKernels {
  gemm_fn fn[3];     // one block per tile (or per (tile, chunk) with partial sums)
  gemm_fn fn_ch[3];  // one launch folding the chunk sums in-block (null: not chunkable)
  gemm_fn fn_fd[3];  // one block per (tile, chunk), folded by the last (null: not built)
};

template <int TM, int TN, int WM, int WN, int NS, bool XT, int WK>
TileKernels make_tile_kernels() {
  TileKernels t;
  t.fn[CK_F32] = gemm_lds_kernel<TM, TN, WM, WN, NS, XT, false, WK, CK_F32>;
  t.fn[CK_F16] = gemm_lds_kernel<TM, TN, WM, WN, NS, XT, false, WK, CK_F16>;
  t.fn[CK_BF16] = gemm_lds_kernel<TM, TN, WM, WN, NS, XT, false, WK, CK_BF16>;
  if constexpr (gemm_chunkable(TM, TN, WM, WN)) {
    t.fn_ch[CK_F32] = gemm_lds_kernel<TM, TN, WM, WN, NS, XT, true, WK, CK_F32>;
    t.fn_ch[CK_F16] = gemm_lds_kernel<TM, TN, WM, WN, NS, XT, true, WK, CK_F16>;
    t.fn_ch[CK_BF16] = gemm_lds_kernel<TM, TN, WM, WN, NS, XT, true, WK, CK_BF16>;
    t.fn_fd[CK_F32] = gemm_lds_kernel<TM, TN, WM, WN, NS, XT, false, WK, CK_F32, true>;
    t.fn_fd[CK_F16] = gemm_lds_kernel<TM, TN, WM, WN, NS, XT, false, WK, CK_F16, true>;
    t.fn_fd[CK_BF16] = gemm_lds_kernel<TM, TN, WM, WN, NS, XT, false, WK, CK_BF16, true>;
  } else {
    for (int c = 0; c < 3; ++c) t.fn_ch[c] = t.fn_fd[c] = nullptr;
  }
  return t;
}

template <int WK>
const TileKernels* tile_kernels() {
#define SKINNY_GEMM_MAKE(TM, TN, WM, WN, NS, XT, NAME) make_tile_kernels<TM, TN, WM, WN, NS, XT, WK>(),
  static const TileKernels table[] = {SKINNY_GEMM_TILE_LIST(SKINNY_GEMM_MAKE)};
#undef SKINNY_GEMM_MAKE
  return table;
}

// Launch one tile's kernel of weight kind WK (the arguments were checked by
// launch_gemm; shape picks the plain, chunked or fold kernel)
template <int WK>
hipError_t launch_gemm_kind(int tile_id, const GemmArgs& args, int c_kind, int shape, int64_t blocks,
                            int threads, hipStream_t stream) {
  const TileKernels& t = tile_kernels<WK>()[tile_id];
  const gemm_fn fn = shape == kGemmChunked ? t.fn_ch[c_kind] : shape == kGemmFold ? t.fn_fd[c_kind] : t.fn[c_kind];
  if (fn == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(threads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

}  // namespace skinny
