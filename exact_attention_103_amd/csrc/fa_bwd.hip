// Exact attention backward for gfx950 (CDNA4, wave64, bf16 MFMA).
//
// Pages cited (short names):
//   [Comparison] "FlashAttention 1-4 generation comparison"
//                (phantomic12.github.io, inference-research)
//   [Evolution]  "FlashAttention evolution" (sandeep007734.github.io,
//                posts/flashattention-evolution)
//
// Gradients of the forward's output O for a loss whose gradient with respect
// to O is dO.  As the pages describe for the backward pass ([Comparison]
// "Notes", FlashAttention-1 entry: recompute instead of store), the
// probabilities are rebuilt from Q, K and the forward's per-row LSE; nothing
// of size N x N is ever stored.  With S = scale Q K^T (masked entries have
// P = 0) and P = exp(S - LSE):
//   dV = P^T dO     dP = dO V^T     dS = P (dP - Delta),  Delta = rowsum(dO * O)
//   dQ = scale dS K                 dK = scale dS^T Q
// Two kernels and no atomics, so results are deterministic:
//   fa_bwd_dq_*    one workgroup of 4 waves per (128-row query block,
//                  batch*head).  Each wave owns 32 query rows: it computes
//                  Delta for them (stored for the second kernel), streams the
//                  K/V tiles of its KV head through LDS and accumulates dQ in
//                  registers (S^T, dP^T and dQ^T as in the forward: one query
//                  per lane).
//   fa_bwd_dkdv_*  one workgroup of 4 waves per (64-key block, batch*KV
//                  head).  Each wave owns 16 keys whose K and V stay in
//                  registers as the B operands of 16x16x32 MFMAs; the wave
//                  streams 32-row Q/dO tiles of every query head of the group
//                  and accumulates dK and dV (S, dP with one key per lane;
//                  dV^T, dK^T).  Three waves per SIMD.
// In both kernels the bf16 probability / score-gradient registers feed the
// next MFMA directly as its B operand (the contraction order is free), and
// the transposed A operands (K^T, dO^T, Q^T) come from gfx950's transposing
// LDS read on row-major tiles.

#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// LDS layout of every bwd tile: 16-byte chunk c of row r sits at c ^ X(r).
// Every tile is read two ways, and X serves both:
//  * row-major MFMA operands: 16 lanes read one chunk of 16 consecutive rows,
//    so X must take a different value on each row that shares a 256-byte
//    bank line position (X is a bijection on r mod 16 for 256-byte rows);
//  * transposing reads: a 16-lane group reads 4 consecutive chunks of 4
//    consecutive rows, so those rows must land in different 64-byte bank
//    groups (bits 2..3 of X differ between rows that share a line half).
// For 256-byte rows X swaps the two 2-bit digits of r mod 16; for 128-byte
// rows (two per line) it does the same on the row's line index; 64-byte rows
// fill a line with four different rows and need only the first property.
//
// The dK/dV kernel reads its tiles with the 16x16x32 operand shapes: 16
// rows per 16-lane group for the row-major reads, 2 chunks of 4 rows per
// group for the transposing reads.  Measured with rocprofv3 on gfx950
// (SQ_LDS_BANK_CONFLICT, one probe kernel per pattern and swizzle), X = i
// (the row index i within the bank-line period) is conflict-free for the
// first pattern only, the digit swap and rotations for the second only, and
// SW = 1, X = i ^ (i << 1), for both.
template <int RB, int SW = 0>
__device__ __forceinline__ int bwd_xor(int r) {
  if constexpr (SW == 1) {
    constexpr int mask = RB >= 256 ? 15 : RB == 128 ? 7 : 3;
    const int i = (r / (RB >= 256 ? 1 : 256 / RB)) & mask;
    return (i ^ (i << 1)) & mask;
  } else if constexpr (RB >= 256) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else if constexpr (RB == 128) {
    const int i = (r >> 1) & 7;
    return ((i & 1) << 2) | (i >> 1);
  } else {
    return (r >> 2) & 3;
  }
}

// Sum of lane l's and lane l ^ 32's values.
__device__ __forceinline__ float lane_pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct BwdShape {
  static constexpr int RB = 2 * D;       // bytes per row in LDS
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int KSTEPS = D / 16;  // 32x32x16 k-steps over d
  static constexpr int DB = D / 32;      // 32-wide d blocks of the transposed accumulators
};

constexpr int kBwdWaves = 4;
constexpr int kDqRows = 32 * kBwdWaves;    // query rows per dQ workgroup
// Keys per K/V tile in the dQ kernel: 64, or 32 at d = 256, where the Q^T,
// dO^T and dQ^T registers alone take 256 of the wave's 512.
template <int D>
constexpr int dq_keys() { return D == 256 ? 32 : 64; }
constexpr int kDkvKeys = 16 * kBwdWaves;   // keys per dK/dV workgroup (16 per wave)
constexpr int kDkvRows = 32;               // query rows per Q/dO tile in the dK/dV kernel

// Direct global -> LDS copy of a ROWS-row tile of a row-major [.][D] bf16
// matrix, swizzled with bwd_xor.  Wave load i writes 1 KB block i*NW + wave
// of the tile; lane l of it fetches the global chunk whose swizzled position
// is that block's l-th chunk.  The per-lane byte offsets within a tile do
// not depend on which tile is copied, so they are computed once
// (dma_offsets); a copy is then one buffer load per block, through a buffer
// resource whose size ends at the matrix's last row: rows past it read as
// zero, which the kernels mask (probability 0) like any other row past the
// end.
template <int D, int ROWS, int NW>
struct Dma {
  static constexpr int CPR = D / 8;
  static constexpr int BLKS = ROWS * CPR / 64;
  static constexpr int LOADS = (BLKS + NW - 1) / NW;
  static_assert((ROWS * CPR) % 64 == 0, "whole 1 KB blocks");
};

template <int D, int ROWS, int SW = 0, int NW = kBwdWaves>
__device__ __forceinline__ void dma_offsets(int wave, int lane, int* off) {
  using T = Dma<D, ROWS, NW>;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    const int P = (i * NW + wave) * 64 + lane;
    const int row = P / T::CPR;
    const int c = (P % T::CPR) ^ bwd_xor<2 * D, SW>(row);
    off[i] = row * 2 * D + c * 16;
  }
}

// Buffer resource over rows r0 .. r0 + ROWS - 1 of a row-major [.][D] bf16
// matrix of `nrows` rows (rows at or past nrows read as zero).
template <int D, int ROWS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int r0,
                                                            int nrows) {
  const int rows = max(0, min(nrows - r0, ROWS));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + (size_t)r0 * D), 0,
                                           rows * D * 2, 0x00020000);
}

template <int D, int ROWS, int NW = kBwdWaves>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, const int* off,
                                         lds_char* tile, int wave) {
  using T = Dma<D, ROWS, NW>;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    const int blk = i * NW + wave;   // uniform across the wave
    if (T::BLKS % NW != 0 && blk >= T::BLKS) break;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(tile + blk * 1024), 16, off[i], 0, 0, 0);
  }
}

// Byte offsets of the transposing reads of a 32-wide d block of a bwd tile,
// for the rows 4*hl + (lane%16)/4 (+8 for the upper half) of every 16-row
// group: lane (hl, g1, j16) receives, for k = 0..3, element d = 32*db + 16*g1
// + j16 of rows 16*kc + 4*hl + k (+8).  Those are the rows (queries or keys)
// that the B-operand registers 8*(kc%2).. of a transposed accumulator hold,
// in the same order.  The XOR of a row depends only on the row within its
// 16-row group, so one offset per (half, db) serves every group kc.
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int (&off)[2][BwdShape<D>::DB]) {
  using S = BwdShape<D>;
  const int hl = lane >> 5, g1 = (lane >> 4) & 1, j16 = lane & 15;
  const int r0 = 4 * hl + (j16 >> 2);
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int r = r0 + 8 * hi;
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
      const int c = 4 * db + 2 * g1 + ((j16 & 3) >> 1);
      off[hi][db] = r * S::RB + ((c ^ bwd_xor<S::RB>(r)) << 4) + 8 * (j16 & 1);
    }
  }
}

__device__ __forceinline__ bf16x8 tr_read(const lds_char* t, int lo_off, int hi_off) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(t + lo_off));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(t + hi_off));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row-major MFMA A operand: 8 bf16 of row r, logical chunk c, of a bwd tile.
template <int RB, int SW = 0>
__device__ __forceinline__ bf16x8 row_read(const lds_char* t, int r, int c) {
  return *(const __attribute__((address_space(3))) bf16x8*)(t + r * RB +
                                                            ((c ^ bwd_xor<RB, SW>(r)) << 4));
}

// ---------------------------------------------------------------------------
// dQ (and Delta)
// ---------------------------------------------------------------------------
// Compile-time loop (every unrolled step's LDS stages are then constants).
template <int I>
struct BwdInt {
  static constexpr int value = I;
};
template <int I, int N, typename F>
__device__ __forceinline__ void bwd_static_for(F&& f) {
  if constexpr (I < N) {
    f(BwdInt<I>{});
    bwd_static_for<I + 1, N>(f);
  }
}

template <int D, bool CAUSAL>
__device__ __forceinline__ void bwd_dq_body(const BwdParams& p, lds_char* kb0, lds_char* kb1,
                                            lds_char* kb2, lds_char* vb0, lds_char* vb1,
                                            lds_char* vb2) {
  using S = BwdShape<D>;
  constexpr int BN = dq_keys<D>(), BM = kDqRows;
  constexpr int KB = BN / 32, KC = BN / 16;
  // At d = 256 (one wave per SIMD) the K/V tiles are copied two steps ahead
  // into three stages and a step's barrier waits only for the previous
  // step's copies, as in the dK/dV kernel.
  constexpr bool kThree = D == 256;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int n = lane & 31;

  const int BH = p.B * p.Hq;
  const int nqb = (p.Nq + BM - 1) / BM;
  const int bh = blockIdx.x % BH;
  const int qi = blockIdx.x / BH;
  const int qblk = CAUSAL ? (nqb - 1 - qi) : qi;   // heaviest causal blocks first
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int g = h / p.group;
  const int q0 = qblk * BM;
  const int qw = q0 + 32 * wave;
  const int row = qw + n;
  const int off = p.Nk - p.Nq;                     // key j allowed for row i iff j <= i + off
  const bool live = row < p.Nq;

  const uint16_t* kbase = p.k + (size_t)(b * p.Hkv + g) * p.Nk * D;
  const uint16_t* vbase = p.v + (size_t)(b * p.Hkv + g) * p.Nk * D;
  const size_t rbase = ((size_t)bh * p.Nq + row) * D;

  int nkt = (p.Nk + BN - 1) / BN;
  if (CAUSAL) nkt = min(nkt, (min(q0 + BM, p.Nq) - 1 + off) / BN + 1);

  // Q^T and dO^T as MFMA B operands (lane (hl, n): row `row`, d = 16t + 8hl
  // .. +7), and Delta = rowsum(dO * O) in fp32.  Rows past Nq are zero.
  bf16x8 qf[S::KSTEPS], df[S::KSTEPS];
  float dsum = 0.f;
#pragma unroll
  for (int t = 0; t < S::KSTEPS; ++t) {
    if (live) {
      qf[t] = *reinterpret_cast<const bf16x8*>(p.q + rbase + 16 * t + 8 * hl);
      df[t] = *reinterpret_cast<const bf16x8*>(p.dout + rbase + 16 * t + 8 * hl);
      const bf16x8 ov = *reinterpret_cast<const bf16x8*>(p.o + rbase + 16 * t + 8 * hl);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = fmaf((float)df[t][e], (float)ov[e], dsum);
    } else {
      qf[t] = bf16x8{};
      df[t] = bf16x8{};
    }
  }
  const float delta = lane_pair_sum(dsum);
  const float nlse2 = live ? -p.lse[(size_t)bh * p.Nq + row] * kLog2e : 0.f;
  if (live && hl == 0) p.delta[(size_t)bh * p.Nq + row] = delta;

  const int koff = n * S::RB;
  int toff[2][S::DB];
  tr_offsets<D>(lane, toff);
  int doff[Dma<D, BN, kBwdWaves>::LOADS];
  dma_offsets<D, BN>(wave, lane, doff);

  f32x16 dq[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db) dq[db] = f32x16{};

  // X^T = T B^T for one 64-key tile T (K or V) and this wave's B (Q or dO).
  auto xt_tile = [&](const lds_char* t, const bf16x8 (&bf)[S::KSTEPS], f32x16 (&acc)[KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      acc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < S::KSTEPS; ++s)
        acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            row_read<S::RB>(t, kb * 32 + n, 2 * s + hl), bf[s], acc[kb], 0, 0, 0);
    }
  };

  auto step = [&](const lds_char* kr, const lds_char* vr, lds_char* kw, lds_char* vw, int j) {
    const int j0 = j * BN;
    FA_STAGE_FENCE();
    if (kThree) {
      dma_tile<D, BN>(rows_rsrc<D, BN>(kbase, j0 + 2 * BN, p.Nk), doff, kw, wave);
      dma_tile<D, BN>(rows_rsrc<D, BN>(vbase, j0 + 2 * BN, p.Nk), doff, vw, wave);
    } else if (j + 1 < nkt) {
      dma_tile<D, BN>(rows_rsrc<D, BN>(kbase, j0 + BN, p.Nk), doff, kw, wave);
      dma_tile<D, BN>(rows_rsrc<D, BN>(vbase, j0 + BN, p.Nk), doff, vw, wave);
    }
    FA_STAGE_FENCE();
    f32x16 sacc[KB], dpacc[KB];
    xt_tile(kr, qf, sacc);    // S^T  = K Q^T
    xt_tile(vr, df, dpacc);   // dP^T = V dO^T
    // Interleave the tile reads of both products one read ahead of the
    // product that consumes them, so each LDS read overlaps an MFMA instead
    // of all reads issuing up front.
    {
      constexpr int NM = 2 * KB * S::KSTEPS;
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
      bwd_static_for<0, NM>([&](auto c) {
        if constexpr (decltype(c)::value + 1 < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
      });
    }
    // Keys past Nk, or past the diagonal when causal, get P = 0.
    if ((j0 + BN > p.Nk) || (CAUSAL && j0 + BN - 1 > qw + off)) {
      const int lim = (CAUSAL ? min(p.Nk - 1, row + off) : p.Nk - 1) - j0 - 4 * hl;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = -INFINITY;
    }
    // Per 16-key chunk: dS^T = P^T (dP^T - Delta) as the bf16 B operand, then
    // dQ^T += K^T dS^T with K^T from transposing reads of the K tile.
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      bf16x8 dsb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * (kc & 1) + i;
        const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[kc >> 1][r], p.c, nlse2));
        dsb[i] = (__bf16)(pr * (dpacc[kc >> 1][r] - delta));
      }
#pragma unroll
      for (int db = 0; db < S::DB; ++db) {
        const bf16x8 a = tr_read(kr, toff[0][db] + 16 * kc * S::RB, toff[1][db] + 16 * kc * S::RB);
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb, dq[db], 0, 0, 0);
      }
    }
    if constexpr (kThree) {
      // Only the copies issued in this step (K and V tiles) may be in flight.
      copies_in_flight_barrier<2 * Dma<D, BN, kBwdWaves>::LOADS>();
    } else {
      __syncthreads();
    }
  };

  dma_tile<D, BN>(rows_rsrc<D, BN>(kbase, 0, p.Nk), doff, kb0, wave);
  dma_tile<D, BN>(rows_rsrc<D, BN>(vbase, 0, p.Nk), doff, vb0, wave);
  if constexpr (kThree) {
    // Tile j lives in stage j % 3; step j copies tile j + 2 (tiles past Nk
    // read zero rows, so every step issues the same number of copies).
    dma_tile<D, BN>(rows_rsrc<D, BN>(kbase, BN, p.Nk), doff, kb1, wave);
    dma_tile<D, BN>(rows_rsrc<D, BN>(vbase, BN, p.Nk), doff, vb1, wave);
    __syncthreads();
    lds_char* const kbs[3] = {kb0, kb1, kb2};
    lds_char* const vbs[3] = {vb0, vb1, vb2};
    for (int j0 = 0; j0 < nkt; j0 += 3) {
      bwd_static_for<0, 3>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if (u == 0 || j0 + u < nkt)
          step(kbs[u], vbs[u], kbs[(u + 2) % 3], vbs[(u + 2) % 3], j0 + u);
      });
    }
    // No copy into this workgroup's LDS may still be in flight when it ends.
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    __syncthreads();
    for (int j = 0; j < nkt; j += 2) {
      step(kb0, vb0, kb1, vb1, j);
      if (j + 1 < nkt) step(kb1, vb1, kb0, vb0, j + 1);
    }
  }

  // dQ = scale * acc, bf16 (round to nearest even); lane holds d rows
  // 32db + 8(r/4) + 4hl + r%4 of its query row.
  if (live) {
    uint16_t* drow = p.dq + rbase;
#pragma unroll
    for (int db = 0; db < S::DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x2 lo = {(__bf16)(dq[db][4 * r4 + 0] * p.scale), (__bf16)(dq[db][4 * r4 + 1] * p.scale)};
        bf16x2 hi = {(__bf16)(dq[db][4 * r4 + 2] * p.scale), (__bf16)(dq[db][4 * r4 + 3] * p.scale)};
        uint2 w;
        w.x = __builtin_bit_cast(unsigned, lo);
        w.y = __builtin_bit_cast(unsigned, hi);
        *reinterpret_cast<uint2*>(drow + 32 * db + 8 * r4 + 4 * hl) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
// Each wave owns 16 keys and works with 16x16x32 MFMAs, which keeps its
// state small: K^T and V^T of its keys as B operands (D/4 registers each)
// and the dK^T, dV^T accumulators (D/2 registers each).  LDS per stage: a Q
// tile and a dO tile (kDkvRows rows each, swizzle SW = 1), then the LSE and
// Delta of those rows (fp32).
constexpr int kDkvWaves = 4;

template <int D>
struct DkvStage {
  static constexpr int TILE = kDkvRows * 2 * D;
  static constexpr int STATS = 2 * kDkvRows * 4;
  // The third stage exists only at d = 256 (placeholders elsewhere).
  static constexpr int TILE3 = D == 256 ? TILE : 16;
  static constexpr int STATS3 = D == 256 ? STATS : 16;
};

template <int D, bool CAUSAL>
__device__ __forceinline__ void bwd_dkdv_body(const BwdParams& p, lds_char* qt0, lds_char* qt1,
                                              lds_char* qt2, lds_char* dt0, lds_char* dt1,
                                              lds_char* dt2, lds_char* st0, lds_char* st1,
                                              lds_char* st2) {
  using S = BwdShape<D>;
  constexpr int BM = kDkvRows, BNK = kDkvKeys, NW = kDkvWaves;
  constexpr int KT = D / 32;   // 16x16x32 k-steps over d
  constexpr int DB = D / 16;   // 16-row d blocks of dK^T, dV^T
  static_assert(BM == 32 && BNK == 16 * NW, "two 16-row blocks per tile, 16 keys per wave");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;     // MFMA column: key kw0 + n
  const int grp = lane >> 4;   // 16-lane group

  const int BG = p.B * p.Hkv;
  const int bg = blockIdx.x % BG;
  const int kblk = blockIdx.x / BG;               // low key blocks see the most queries
  const int b = bg / p.Hkv;
  const int g = bg - b * p.Hkv;
  const int k0 = kblk * BNK;
  const int kw0 = k0 + 16 * wave;                 // first key of this wave
  const int key = kw0 + n;
  const int off = p.Nk - p.Nq;
  const bool live = key < p.Nk;
  const size_t kvrow = ((size_t)bg * p.Nk + key) * D;

  // K^T and V^T of this lane's key as B operands: d = 32t + 8grp .. +7.
  bf16x8 kf[KT], vf[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    kf[t] = live ? *reinterpret_cast<const bf16x8*>(p.k + kvrow + 32 * t + 8 * grp) : bf16x8{};
    vf[t] = live ? *reinterpret_cast<const bf16x8*>(p.v + kvrow + 32 * t + 8 * grp) : bf16x8{};
  }

  // Query tiles: every query head of the group, rows from the first one that
  // sees key k0 (causal) to Nq.
  const int qstart = CAUSAL ? (max(0, k0 - off) / BM) * BM : 0;
  const int nqt = (p.Nq - qstart + BM - 1) / BM;
  const int steps = p.group * nqt;

  // Transposing reads of a 16-wide d block db: lane (grp, n) addresses row
  // 4grp + n/4 (+16 for the second row block), columns 16db + 4(n%4) .. +3,
  // and receives rows 4grp + 0..3 of column 16db + n: the queries that the
  // B-operand registers 0..3 (4..7) of its column hold.
  int toff[DB];
  {
    const int r = 4 * grp + (n >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = 2 * db + ((n & 3) >> 1);
      toff[db] = r * S::RB + ((c ^ bwd_xor<S::RB, 1>(r)) << 4) + 8 * (n & 1);
    }
  }

  f32x4 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x4{};
    dv[db] = f32x4{};
  }

  int doff[Dma<D, BM, NW>::LOADS];
  dma_offsets<D, BM, 1, NW>(wave, lane, doff);
  // Steps walk the query heads of the group, each over its row tiles
  // qstart, qstart + BM, ...: the tile to load next and the tile of the
  // current step advance by one each time (no division per step).
  //
  // At d = 256 (one wave per SIMD) every copy is issued two steps ahead into
  // three stages, and a step's barrier waits only for the previous step's
  // copies: +12% there, -2% to -4% at d = 64 and 128, which keep two stages.
  // Copies past the last tile are then still issued (zero rows, and the
  // stats of a valid tile), so that every step issues the same number.
  constexpr bool kThree = D == 256;
  int ld_h = g * p.group, ld_i0 = qstart;
  const int h_end = (g + 1) * p.group;
  auto load = [&](lds_char* qt, lds_char* dt, lds_char* st) {
    const bool past = kThree && ld_h >= h_end;
    const int hh = past ? h_end - 1 : ld_h;
    const int r0 = past ? p.Nq : ld_i0;
    const size_t hb = (size_t)(b * p.Hq + hh) * p.Nq;
    dma_tile<D, BM, NW>(rows_rsrc<D, BM>(p.q + hb * D, r0, p.Nq), doff, qt, wave);
    dma_tile<D, BM, NW>(rows_rsrc<D, BM>(p.dout + hb * D, r0, p.Nq), doff, dt, wave);
    if (wave == 0) {   // lanes 0-31: LSE of the BM rows, lanes 32-63: Delta
      const float* src = (lane < BM ? p.lse : p.delta - BM) + hb;
      __builtin_amdgcn_global_load_lds(src + min(ld_i0 + (lane & (BM - 1)), p.Nq - 1) + (lane & BM),
                                       st, 4, 0, 0);
    }
    ld_i0 += BM;
    if (ld_i0 >= p.Nq) {
      ld_i0 = qstart;
      ++ld_h;
    }
  };
  int cur_i0 = qstart;

  auto step = [&](const lds_char* qt, const lds_char* dt, const lds_char* st, lds_char* qw,
                  lds_char* dw, lds_char* sw, int s) {
    FA_STAGE_FENCE();
    if (kThree || s + 1 < steps) load(qw, dw, sw);
    FA_STAGE_FENCE();
    const int i0 = cur_i0;
    cur_i0 = cur_i0 + BM >= p.Nq ? qstart : cur_i0 + BM;
    const __attribute__((address_space(3))) f32x4* lse4 =
        (const __attribute__((address_space(3))) f32x4*)st;
    const __attribute__((address_space(3))) f32x4* del4 = lse4 + BM / 4;

    // S = Q K^T and dP = dO V^T for the two 16-row blocks: lane (grp, n)
    // gets rows 16qb + 4grp + r (r = 0..3) of key n.
    f32x4 sacc[2], dpacc[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      sacc[qb] = f32x4{};
      dpacc[qb] = f32x4{};
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        sacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            row_read<S::RB, 1>(qt, 16 * qb + n, 4 * t + grp), kf[t], sacc[qb], 0, 0, 0);
        dpacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            row_read<S::RB, 1>(dt, 16 * qb + n, 4 * t + grp), vf[t], dpacc[qb], 0, 0, 0);
      }
    }
    if ((i0 + 31 >= p.Nq) || (CAUSAL && kw0 + 15 > i0 + off)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ri = i0 + 16 * qb + 4 * grp + r;
          if (ri >= p.Nq || (CAUSAL && key > ri + off)) sacc[qb][r] = -INFINITY;
        }
    }
    // P = exp(S - LSE) (base 2) and dS = P (dP - Delta), as bf16 B operands;
    // register 4qb + r holds row 16qb + 4grp + r.
    bf16x8 pb, sb;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const f32x4 l4 = lse4[4 * qb + grp];
      const f32x4 d4 = del4[4 * qb + grp];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[qb][r], p.c, -l4[r] * kLog2e));
        pb[4 * qb + r] = (__bf16)pr;
        sb[4 * qb + r] = (__bf16)(pr * (dpacc[qb][r] - d4[r]));
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS, the transposed A operands read from
    // the dO and Q tiles.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dv[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          tr_read(dt, toff[db], toff[db] + 16 * S::RB), pb, dv[db], 0, 0, 0);
      dk[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          tr_read(qt, toff[db], toff[db] + 16 * S::RB), sb, dk[db], 0, 0, 0);
    }
    if constexpr (kThree) {
      // Only the copies issued in this step may be in flight: the Q and dO
      // tiles, and on wave 0 the stats.
      constexpr int L = 2 * Dma<D, BM, NW>::LOADS;
      if (wave == 0)
        wait_copies_in_flight<L + 1>();
      else
        wait_copies_in_flight<L>();
      step_barrier();
    } else {
      __syncthreads();
    }
  };

  load(qt0, dt0, st0);
  if constexpr (kThree) {
    // Tile s lives in stage s % 3; step s copies tile s + 2.
    load(qt1, dt1, st1);
    __syncthreads();
    lds_char* const qts[3] = {qt0, qt1, qt2};
    lds_char* const dts[3] = {dt0, dt1, dt2};
    lds_char* const sts[3] = {st0, st1, st2};
    for (int s0 = 0; s0 < steps; s0 += 3) {
      bwd_static_for<0, 3>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if (u == 0 || s0 + u < steps)
          step(qts[u], dts[u], sts[u], qts[(u + 2) % 3], dts[(u + 2) % 3], sts[(u + 2) % 3],
               s0 + u);
      });
    }
    // No copy into this workgroup's LDS may still be in flight when it ends.
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    __syncthreads();
    for (int s = 0; s < steps; s += 2) {
      step(qt0, dt0, st0, qt1, dt1, st1, s);
      if (s + 1 < steps) step(qt1, dt1, st1, qt0, dt0, st0, s + 1);
    }
  }

  // dK = scale * acc, dV = acc, bf16; lane (grp, n) holds d rows 16db +
  // 4grp + r of key n.
  if (live) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x2 klo = {(__bf16)(dk[db][0] * p.scale), (__bf16)(dk[db][1] * p.scale)};
      bf16x2 khi = {(__bf16)(dk[db][2] * p.scale), (__bf16)(dk[db][3] * p.scale)};
      bf16x2 vlo = {(__bf16)dv[db][0], (__bf16)dv[db][1]};
      bf16x2 vhi = {(__bf16)dv[db][2], (__bf16)dv[db][3]};
      uint2 wk, wv;
      wk.x = __builtin_bit_cast(unsigned, klo);
      wk.y = __builtin_bit_cast(unsigned, khi);
      wv.x = __builtin_bit_cast(unsigned, vlo);
      wv.y = __builtin_bit_cast(unsigned, vhi);
      *reinterpret_cast<uint2*>(p.dk + kvrow + 16 * db + 4 * grp) = wk;
      *reinterpret_cast<uint2*>(p.dv + kvrow + 16 * db + 4 * grp) = wv;
    }
  }
}

}  // namespace
}  // namespace fa

#define FA_BWD_DQ(D, CAUSAL, NAME, WPE)                                                    \
  extern "C" __global__ void __launch_bounds__(64 * fa::kBwdWaves, WPE) NAME(fa::BwdParams p) { \
    constexpr int T = fa::dq_keys<D>() * 2 * D;                                            \
    constexpr int T3 = D == 256 ? T : 16; /* third stage at d = 256 only */                \
    __shared__ __attribute__((aligned(1024))) char k0[T];                                  \
    __shared__ __attribute__((aligned(1024))) char k1[T];                                  \
    __shared__ __attribute__((aligned(1024))) char k2[T3];                                 \
    __shared__ __attribute__((aligned(1024))) char v0[T];                                  \
    __shared__ __attribute__((aligned(1024))) char v1[T];                                  \
    __shared__ __attribute__((aligned(1024))) char v2[T3];                                 \
    fa::bwd_dq_body<D, CAUSAL>(p, (fa::lds_char*)k0, (fa::lds_char*)k1, (fa::lds_char*)k2, \
                               (fa::lds_char*)v0, (fa::lds_char*)v1, (fa::lds_char*)v2);   \
  }

#define FA_BWD_DKDV(D, CAUSAL, NAME, WPE)                                                  \
  extern "C" __global__ void __launch_bounds__(64 * fa::kDkvWaves, WPE) NAME(fa::BwdParams p) { \
    using St = fa::DkvStage<D>;                                                            \
    __shared__ __attribute__((aligned(1024))) char q0[St::TILE];                           \
    __shared__ __attribute__((aligned(1024))) char q1[St::TILE];                           \
    __shared__ __attribute__((aligned(1024))) char q2[St::TILE3];                          \
    __shared__ __attribute__((aligned(1024))) char d0[St::TILE];                           \
    __shared__ __attribute__((aligned(1024))) char d1[St::TILE];                           \
    __shared__ __attribute__((aligned(1024))) char d2[St::TILE3];                          \
    __shared__ __attribute__((aligned(256))) char s0[St::STATS];                           \
    __shared__ __attribute__((aligned(256))) char s1[St::STATS];                           \
    __shared__ __attribute__((aligned(256))) char s2[St::STATS3];                          \
    fa::bwd_dkdv_body<D, CAUSAL>(p, (fa::lds_char*)q0, (fa::lds_char*)q1,                  \
                                 (fa::lds_char*)q2, (fa::lds_char*)d0,                     \
                                 (fa::lds_char*)d1, (fa::lds_char*)d2,                     \
                                 (fa::lds_char*)s0, (fa::lds_char*)s1,                     \
                                 (fa::lds_char*)s2);                                       \
  }

FA_BWD_DQ(32, false, fa_bwd_dq_d32_nomask, 2)
FA_BWD_DQ(32, true, fa_bwd_dq_d32_causal, 2)
FA_BWD_DQ(64, false, fa_bwd_dq_d64_nomask, 2)
FA_BWD_DQ(64, true, fa_bwd_dq_d64_causal, 2)
FA_BWD_DQ(128, false, fa_bwd_dq_d128_nomask, 2)
FA_BWD_DQ(128, true, fa_bwd_dq_d128_causal, 2)
FA_BWD_DQ(256, false, fa_bwd_dq_d256_nomask, 1)
FA_BWD_DQ(256, true, fa_bwd_dq_d256_causal, 1)
FA_BWD_DKDV(32, false, fa_bwd_dkdv_d32_nomask, 3)
FA_BWD_DKDV(32, true, fa_bwd_dkdv_d32_causal, 3)
FA_BWD_DKDV(64, false, fa_bwd_dkdv_d64_nomask, 3)
FA_BWD_DKDV(64, true, fa_bwd_dkdv_d64_causal, 3)
FA_BWD_DKDV(128, false, fa_bwd_dkdv_d128_nomask, 3)
FA_BWD_DKDV(128, true, fa_bwd_dkdv_d128_causal, 3)
FA_BWD_DKDV(256, false, fa_bwd_dkdv_d256_nomask, 1)
FA_BWD_DKDV(256, true, fa_bwd_dkdv_d256_causal, 1)

namespace fa {

bool bwd_supported_d(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

int bwd_dq_grid_blocks(int B, int Hq, int Nq) { return ((Nq + kDqRows - 1) / kDqRows) * B * Hq; }
int bwd_dkdv_grid_blocks(int B, int Hkv, int Nk) {
  return ((Nk + kDkvKeys - 1) / kDkvKeys) * B * Hkv;
}

const char* bwd_kernel_name(int d, bool causal, int stage) {
  static const char* const names[2][4][2] = {
      {{"fa_bwd_dq_d32_nomask", "fa_bwd_dq_d32_causal"},
       {"fa_bwd_dq_d64_nomask", "fa_bwd_dq_d64_causal"},
       {"fa_bwd_dq_d128_nomask", "fa_bwd_dq_d128_causal"},
       {"fa_bwd_dq_d256_nomask", "fa_bwd_dq_d256_causal"}},
      {{"fa_bwd_dkdv_d32_nomask", "fa_bwd_dkdv_d32_causal"},
       {"fa_bwd_dkdv_d64_nomask", "fa_bwd_dkdv_d64_causal"},
       {"fa_bwd_dkdv_d128_nomask", "fa_bwd_dkdv_d128_causal"},
       {"fa_bwd_dkdv_d256_nomask", "fa_bwd_dkdv_d256_causal"}}};
  if (stage != 0 && stage != 1) return nullptr;
  const int di = d == 32 ? 0 : d == 64 ? 1 : d == 128 ? 2 : d == 256 ? 3 : -1;
  if (di < 0) return nullptr;
  return names[stage][di][causal ? 1 : 0];
}

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t s) {
  const void* f1 = nullptr;
  const void* f2 = nullptr;
#define FA_PICK(D)                                                                       \
  case D:                                                                                \
    f1 = causal ? (const void*)fa_bwd_dq_d##D##_causal : (const void*)fa_bwd_dq_d##D##_nomask; \
    f2 = causal ? (const void*)fa_bwd_dkdv_d##D##_causal : (const void*)fa_bwd_dkdv_d##D##_nomask; \
    break;
  switch (d) {
    FA_PICK(32)
    FA_PICK(64)
    FA_PICK(128)
    FA_PICK(256)
    default: return hipErrorInvalidValue;
  }
#undef FA_PICK
  BwdParams arg = p;
  void* args[] = {&arg};
  const dim3 block(64 * kBwdWaves);
  // The dQ kernel writes Delta, which the dK/dV kernel reads: stream order.
  hipError_t e = hipLaunchKernel(f1, dim3(bwd_dq_grid_blocks(p.B, p.Hq, p.Nq)), block, args, 0, s);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(f2, dim3(bwd_dkdv_grid_blocks(p.B, p.Hkv, p.Nk)), block, args, 0, s);
}

}  // namespace fa
