// FP8 exact-attention forward for gfx950 (CDNA4 OCP fp8 e4m3 MFMA).
//
// Pages cited (short names):
//   [Evolution]  "FlashAttention evolution" (sandeep007734.github.io,
//                posts/flashattention-evolution)
//   [Comparison] "FlashAttention 1-4 generation comparison"
//                (phantomic12.github.io, inference-research)
//
// The same fused forward as fa_fwd.hip (tiling, online softmax, one query
// per lane through S^T = K Q^T, deferred normalisation), with both products
// in 8-bit floating point as FlashAttention-3 does on Hopper ([Evolution]
// §4; [Comparison] "Notes", FA-3 entry).  Q, K and V arrive as OCP fp8
// e4m3 values with one dequantisation factor each (real = fp8 * factor):
//   S^T = K Q^T          v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 x fp8, unit
//                        block scales), fp32 accumulate; the three factors
//                        and the softmax scale fold into the exponent FMA.
//   online softmax       base 2, running reference maximum and sum in
//                        fp32, probabilities against the reference without
//                        a per-tile row maximum: the reference only moves
//                        when a lane's tile sum reaches 2^8 (below).
//   O^T += V^T P^T       P^T rounded to fp8 e4m3 in the accumulator's own
//                        registers (4 per dword, v_cvt_pk_fp8_f32), V^T from
//                        gfx950's 8-bit transposing LDS read.
// The MFMA contracts lane half h, byte p of the A operand with lane half h,
// byte p of the B operand (any consistent k assignment gives the same
// product), so K and Q use contiguous d ranges, and V^T is read with the key
// order that the P^T registers hold.  O = v_factor * acc / l (bf16), LSE in
// natural log of the scaled scores.
//
// Schedule: 32 query rows per wave, one 64-key tile per step.  The P V
// product of a tile runs one step after its probabilities, so a step's
// MFMAs do not depend on its exponentials.  At d = 128 eight waves share a
// workgroup (two per SIMD), and the two waves of a SIMD issue the MFMAs and
// the exponentials in opposite orders, so one wave's softmax overlaps the
// other wave's products.  At d = 64 and 256 a workgroup has four waves and
// the compiler interleaves each wave's MFMAs with its own exponentials; at
// d = 64 three workgroups share a CU, at d = 256 (O^T alone takes 128
// registers) one.  K and V tiles are copied two steps ahead into three LDS
// buffers each, so the per-step barrier rarely waits for memory.

#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

// A lane's 32 probabilities of a tile summing below 2^8 bounds each of them
// below 2^8 < 448 (the e4m3 maximum).  Otherwise (the row's first tile, whose
// reference is still -1e30 and so gives inf, or a score that rose by several
// units) the tile's row maximum becomes the reference, the accumulator is
// rescaled and the tile's probabilities are recomputed, now all <= 1.  Any
// reference gives the same exact result ([Evolution] §5 and [Comparison]
// "Workarounds": conditional rescaling); this one only bounds the range,
// and the common path needs no row maximum at all.
constexpr float kF8SumLimit = 256.0f;

template <int D, int NW>
struct F8Shape {
  static constexpr int BN = 64;            // keys per tile (one PV k-step)
  static constexpr int BM = 32 * NW;       // query rows per workgroup
  static constexpr int RB = D;             // bytes per K or V row
  static constexpr int CPR = D / 16;       // 16-byte chunks per row
  static constexpr int KSTEPS = D >= 64 ? D / 64 : 1;   // 32x32x64 k-steps over d
  static constexpr int KB = BN / 32;       // 32-key blocks per tile
  static constexpr int DB = D / 32;        // 32-row d blocks of O^T
  static constexpr int TILE = BN * RB;
  static constexpr int BLKS = TILE / 1024;
  static constexpr int LOADS = (BLKS + NW - 1) / NW;
  static_assert(D == 32 || D % 64 == 0, "fp8 head dim");
};

// LDS tiles: 16-byte chunk c of row r at c ^ X(r).  Two read patterns meet
// there:
//  * the K operand (16-byte reads, 16 lanes per LDS pass): 16 consecutive
//    rows, one chunk each, so X must separate rows sharing a bank-line
//    position (a bijection on the row's line index);
//  * the V^T operand (8-bit transposing 8-byte reads, 32 lanes per pass):
//    rows {0..3, 8..11} + 4h, chunks 2db and 2db + 1, so the rows of one
//    line position must differ in X's bit 1.
// 256-byte rows (one per line): X is the bit permutation of r mod 16 that
// takes r's bits 2, 0, 1, 3 to X's bits 0, 1, 2, 3 -- a bijection on 16
// consecutive rows (K), and X / 2 differs across rows {0..3, 8..11} + 4h
// (V^T).  128-byte rows (two per line): X = i with its two low bits
// swapped, i = (r / 2) mod 8; 64-byte rows (four per line): X = (r / 4) mod
// 4.  All three touch every bank once per pass in either pattern (an
// earlier X = i put two lanes on each bank of the V^T reads, and the
// 128-byte rule on 256-byte rows two on each bank of the K reads).
// 32-byte rows (eight per line, two chunks): X = (r / 8) mod 2 keeps the K
// reads conflict-free; the V^T reads of rows {0..3} and {8..11} then share
// their banks (two lanes per bank), which no chunk permutation inside a
// 32-byte row can avoid.
template <int RB>
__device__ __forceinline__ int f8_xor(int r) {
  if constexpr (RB >= 256) {
    return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8);
  } else if constexpr (RB == 128) {
    const int i = (r >> 1) & 7;
    return ((i & 1) << 1) | ((i >> 1) & 1) | (i & 4);
  } else if constexpr (RB == 64) {
    return (r >> 2) & 3;
  } else {
    return (r >> 3) & 1;
  }
}

__device__ __forceinline__ float f8_half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float f8_half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource over the `rows` keys of one tile at `base` (fp8
// [key][D]): loads past those rows return zero without touching memory,
// which covers the key tail and the tiles past the end (rows = 0).
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f8_tile_rsrc(const uint8_t* base, int rows) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, rows * D, 0x00020000);
}
// A tile is copied with direct buffer -> LDS loads: wave w writes the 1 KB
// blocks i*NW + w, lane l the l-th 16-byte chunk of the block, which holds
// row P / CPR, swizzled chunk P % CPR of the tile (P = 64 * block + l).  The
// per-lane global offsets are fixed for the kernel, so the loads' only
// vector operand is never rewritten while a copy is in flight.
template <int D, int NW>
__device__ __forceinline__ void f8_load_offsets(int wave, int lane, int* voff) {
  using S = F8Shape<D, NW>;
#pragma unroll
  for (int i = 0; i < S::LOADS; ++i) {
    const int P = (i * NW + wave) * 64 + lane;
    const int row = P / S::CPR;
    voff[i] = row * D + (((P % S::CPR) ^ f8_xor<S::RB>(row)) << 4);
  }
}
template <int D, int NW>
__device__ __forceinline__ void f8_load_tile(__amdgpu_buffer_rsrc_t rs, lds_char* tile, int wave,
                                             const int* voff) {
  using S = F8Shape<D, NW>;
#pragma unroll
  for (int i = 0; i < S::LOADS; ++i) {
    const int blk = i * NW + wave;
    if (S::BLKS % NW != 0 && blk >= S::BLKS) break;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(tile + blk * 1024), 16, voff[i], 0, 0, 0);
  }
}

// Compile-time loop (every unrolled step's LDS buffers are then constants).
template <int I>
struct F8Int {
  static constexpr int value = I;
};
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(F8Int<I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ v8i f8_mfma_operand(v4i lo, v4i hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int D, int NW, bool CAUSAL>
__device__ __forceinline__ void fwd_fp8_body(const FwdF8Params& p, lds_char* kb0, lds_char* kb1,
                                             lds_char* kb2, lds_char* vb0, lds_char* vb1,
                                             lds_char* vb2) {
  using S = F8Shape<D, NW>;
  constexpr int BN = S::BN;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int n = lane & 31;

  // Grid order as in the bf16 forward: query block major (longest causal
  // blocks first), (batch, head) minor; non-causal grids with a head count
  // divisible by 8 run head major inside each XCD (workgroup w goes to XCD
  // w mod 8), so the XCD's workgroups stream the same K/V tiles together.
  // Measured: +2.4% at B=8 H=16 N=2048 non-causal; at the long causal
  // workload head-major order was 2.9% slower here, so causal grids keep
  // the block-major order.
  const int BH = p.B * p.Hq;
  const int nqb = (p.Nq + S::BM - 1) / S::BM;
  int bh, qi;
  if (!CAUSAL && BH % 8 == 0) {
    const int x = blockIdx.x % 8, i = blockIdx.x / 8;
    bh = x + 8 * (i / nqb);
    qi = i % nqb;
  } else {
    bh = blockIdx.x % BH;
    qi = blockIdx.x / BH;
  }
  const int qblk = CAUSAL ? (nqb - 1 - qi) : qi;
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int g = h / p.group;
  const int q0 = qblk * S::BM;
  const int qw = q0 + 32 * wave;
  const int row = qw + n;
  const int off = p.Nk - p.Nq;

  // Exponent factor scale * q_descale * k_descale * log2(e) and the V
  // factor: from the arguments, or from device memory when the descales
  // were produced on the device (the quantisation step writes them).
  float cexp = p.c, vds = p.v_descale;
  if (p.q_ds) {
    cexp = p.c * *p.q_ds * *p.k_ds;
    vds = *p.v_ds;
  }

  const uint8_t* kbase = p.k + (size_t)(b * p.Hkv + g) * p.Nk * D;
  const uint8_t* vbase = p.v + (size_t)(b * p.Hkv + g) * p.Nk * D;

  int nkt = (p.Nk + BN - 1) / BN;
  if (CAUSAL) nkt = min(nkt, (min(q0 + S::BM, p.Nq) - 1 + off) / BN + 1);

  // Q^T B operand: lane (hl, n) holds Q[row][64t + 32hl .. +31].  Rows past
  // Nq are zero.  At d = 32 the one k-step's upper half (hl = 1) is zero,
  // and those lanes' K operand repeats the row's 32 bytes: e4m3 has no
  // infinity, so each added product is a zero unless the K row holds a NaN,
  // which makes the score NaN in any case.
  v8i qf[S::KSTEPS];
#pragma unroll
  for (int t = 0; t < S::KSTEPS; ++t) {
    if (row < p.Nq && (D >= 64 || hl == 0)) {
      const uint8_t* src = p.q + ((size_t)bh * p.Nq + row) * D + 64 * t + 32 * hl;
      qf[t] = f8_mfma_operand(*reinterpret_cast<const v4i*>(src),
                              *reinterpret_cast<const v4i*>(src + 16));
    } else {
      qf[t] = v8i{};
    }
  }

  // K A-operand reads: row 32kb + n, chunks 4t + 2hl and +1 (at d = 32
  // chunks 0 and 1 for both lane halves).
  const int kx = f8_xor<S::RB>(n);
  const int kc0 = D >= 64 ? 2 * hl : 0;
  // V^T A-operand reads (8-bit transposing loads): source lane s of a
  // 16-lane group (hl, g1) addresses key row vrow + 16u and 8 bytes at
  // column 32db + 16g1 + 8(s&1); lane i of the group then receives column
  // 32db + 16g1 + i of the 8 rows its group's sources address, in source
  // order, which is the key order of the P^T registers 8u .. 8u+7.
  const int s16 = lane & 15;
  const int g1 = (lane >> 4) & 1;
  const int qsel = ((s16 & 7) >> 1) + 4 * (s16 >> 3);
  const int vrow = 8 * (qsel >> 2) + 4 * hl + (qsel & 3);
  const int vx = f8_xor<S::RB>(vrow);
  int voff[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db)
    voff[db] = vrow * S::RB + (((2 * db + g1) ^ vx) << 4) + 8 * (s16 & 1);

  f32x16 oacc[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db) oacc[db] = f32x16{};
  float m_run = -1e30f;
  float l_run[2] = {0.f, 0.f};

  auto s_tile = [&](const lds_char* kt, f32x16 (&sacc)[S::KB]) {
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int t = 0; t < S::KSTEPS; ++t) {
        const lds_char* rp = kt + (kb * 32 + n) * S::RB;
        const v4i lo = *(const __attribute__((address_space(3))) v4i*)(rp + (((4 * t + kc0) ^ kx) << 4));
        const v4i hi = *(const __attribute__((address_space(3))) v4i*)(rp + (((4 * t + kc0 + 1) ^ kx) << 4));
        sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f8_mfma_operand(lo, hi), qf[t],
                                                                  sacc[kb], 0, 0, 0, 127, 0, 127);
      }
    }
  };
  auto needs_mask = [&](int t) {
    const int t0 = t * BN;
    return (t0 + BN > p.Nk) || (CAUSAL && t0 + BN - 1 > qw + off);
  };
  auto mask_tile = [&](f32x16 (&sacc)[S::KB], int t) {
    const int lim = (CAUSAL ? min(p.Nk - 1, row + off) : p.Nk - 1) - t * BN - 4 * hl;
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = -INFINITY;
  };
  auto tile_max = [&](const f32x16 (&sacc)[S::KB]) {
    float x = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) x = fmaxf(fmaxf(x, sacc[kb][r]), sacc[kb][r + 1]);
    return f8_half_max(x) * cexp;
  };

  // P V of a tile: O^T += V^T P^T, the V^T operand from 8-bit transposing
  // reads of the tile's V buffer.
  auto pv = [&](const lds_char* vt, const v8i& pft) {
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
      v8i a;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(vt + voff[db] + 16 * u * S::RB));
        a[2 * u] = t[0];
        a[2 * u + 1] = t[1];
      }
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pft, oacc[db], 0, 0, 0, 127, 0, 127);
    }
  };

  int ldoff[S::LOADS];
  f8_load_offsets<D, NW>(wave, lane, ldoff);
  auto load = [&](const uint8_t* base, int t, lds_char* tile) {
    const int rows = t < nkt ? min(p.Nk - t * BN, BN) : 0;
    f8_load_tile<D, NW>(f8_tile_rsrc<D>(base + (size_t)t * BN * D, rows), tile, wave, ldoff);
  };

  // One step for tile j.  The P V product of a tile runs one step after its
  // probabilities: step j issues S^T of tile j+1 and P V of tile j-1 on the
  // MFMA pipe, and neither depends on the VALU work that turns tile j's
  // scores into fp8 probabilities.  The two waves that share a SIMD (waves w
  // and w+4 of the workgroup) take the two halves in opposite orders (wave
  // group G = 1: products, then probabilities; G = 0: probabilities, then
  // products), so that one wave's exponentials run while the other wave's
  // MFMAs do.  A scheduling barrier keeps each order as written.  In a
  // four-wave workgroup (d = 64 and 256) no wave of the same workgroup
  // shares the SIMD: both halves then form one scheduling region and the
  // compiler interleaves the wave's MFMAs with its own exponentials, under
  // LLVM's instruction-group strategy 0 (+1% to +2% over its default; +14% to
  // +15% over the fixed order at d = 256; at d = 64, +16% to +20% over eight
  // waves in the two orders, while at d = 128 the eight-wave order measured
  // 1% faster at the long prefill and the d = 128 sweep shape).
  //
  // Buffers: K_{j+1} and V_{j-1} are read here; K_{j+3} is loaded over K_j
  // (read in the previous step) and V_{j+1} over V_{j-2}.  Every copy is
  // thus issued two steps before its tile is read, and the step ends with a
  // workgroup barrier that waits only for the previous step's copies (the
  // two issued here may stay in flight).  The loads are unconditional
  // (tiles past the end read zero rows), which keeps that count exact.
  //
  // On entry sc holds S^T of tile j and pf the fp8 probabilities of tile
  // j-1 (unused when j = 0).
  v8i pf = v8i{};
  auto step = [&](const lds_char* kr, const lds_char* vprev, lds_char* kw, lds_char* vw,
                  f32x16 (&sc)[S::KB], f32x16 (&sn)[S::KB], int j, auto group) {
    if (needs_mask(j)) mask_tile(sc, j);
    FA_STAGE_FENCE();
    load(kbase, j + 3, kw);
    load(vbase, j + 1, vw);
    FA_STAGE_FENCE();

    // P^T = 2^(S*c - m) rounded to fp8: dword w holds keys of block w/4,
    // registers 4(w%4) .. +3, which the V^T reads follow.  The two
    // conversions of dword w overwrite both of its halves; passing the
    // previous tile's dword as the "old" operand keeps the same registers
    // and saves zeroing them.
    v8i pn = pf;
    float t0, t1;
    // The sums start from the first pair: a sum started at 0.f costs an
    // addition of zero, which the compiler keeps (it would turn -0 into +0).
    auto probs = [&]() {
      const float nm = -m_run;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r0 = 4 * (w & 3);
        const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[kb][r0 + 0], cexp, nm));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[kb][r0 + 1], cexp, nm));
        const float e2 = __builtin_amdgcn_exp2f(fmaf(sc[kb][r0 + 2], cexp, nm));
        const float e3 = __builtin_amdgcn_exp2f(fmaf(sc[kb][r0 + 3], cexp, nm));
        t0 = w == 0 ? e0 + e2 : t0 + (e0 + e2);
        t1 = w == 0 ? e1 + e3 : t1 + (e1 + e3);
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, pn[w], false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, x, true);
        pn[w] = x;
      }
    };
    auto products = [&]() {
      s_tile(kr, sn);
      if (j > 0) pv(vprev, pf);
    };
    if constexpr (NW == 4) {
      __builtin_amdgcn_iglp_opt(0);
      products();
      probs();
    } else if constexpr (decltype(group)::value) {
      products();
      __builtin_amdgcn_sched_barrier(0);
      probs();
    } else {
      probs();
      __builtin_amdgcn_sched_barrier(0);
      products();
    }
    // A second pass runs only after the reference moved (see kF8SumLimit);
    // the rescale of the accumulator then follows the P V product of tile
    // j-1, which was taken against the old reference.  The bit-pattern test
    // on the next tile's scores (a NaN) is never true for finite inputs;
    // reading them here keeps their MFMAs ahead of the branch.
    bool bad = !(t0 + t1 < kF8SumLimit);
#pragma unroll
    for (int kb = 0; kb < S::KB; ++kb) bad = bad || __builtin_bit_cast(int, sn[kb][15]) == -1;
    if (__builtin_expect(__any(bad), 0)) {
      const float m_new = fmaxf(m_run, tile_max(sc));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run[0] *= alpha;
      l_run[1] *= alpha;
#pragma unroll
      for (int db = 0; db < S::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
      probs();
    }
    l_run[0] += t0;
    l_run[1] += t1;
    pf = pn;
    // Step barrier: only this step's copies (a K and a V tile) may be in
    // flight past it.
    copies_in_flight_barrier<2 * S::LOADS>();
  };

  // The V buffers start as zeros: a copy through a resource of fewer rows
  // leaves the LDS rows past them as they were, and those rows meet
  // probability 0 in the P V product, which stays 0 only for finite values
  // (stale rows of earlier tiles are finite; LDS never written may not be).
  {
    using v4 = unsigned __attribute__((ext_vector_type(4)));
    for (int i = tid; i < S::TILE / 16; i += 64 * NW) {
      *(__attribute__((address_space(3))) v4*)(vb0 + 16 * i) = v4{};
      *(__attribute__((address_space(3))) v4*)(vb1 + 16 * i) = v4{};
      *(__attribute__((address_space(3))) v4*)(vb2 + 16 * i) = v4{};
    }
    __syncthreads();
  }
  f32x16 sa[S::KB], sb[S::KB];
  load(kbase, 0, kb0);
  load(vbase, 0, vb0);
  load(kbase, 1, kb1);
  load(kbase, 2, kb2);
  __syncthreads();
  s_tile(kb0, sa);
  __syncthreads();
  // Tile t lives in K buffer t % 3 and V buffer t % 3; six steps per
  // iteration keep every buffer choice (and the S^T register set, which
  // alternates) a compile-time constant.
  lds_char* const kbs[3] = {kb0, kb1, kb2};
  lds_char* const vbs[3] = {vb0, vb1, vb2};
  auto run = [&](auto group) {
    for (int j0 = 0; j0 < nkt; j0 += 6) {
      static_for<0, 6>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const int j = j0 + u;
        if (u == 0 || j < nkt) {
          auto& sc = (u % 2 == 0) ? sa : sb;
          auto& sn = (u % 2 == 0) ? sb : sa;
          step(kbs[(u + 1) % 3], vbs[(u + 2) % 3], kbs[u % 3], vbs[(u + 1) % 3], sc, sn, j, group);
        }
      });
    }
  };
  if (NW == 8 && ((wave >> 2) & 1))
    run(F8Int<1>{});
  else
    run(F8Int<0>{});
  // The copies of the last steps (tiles past the end) must land before the
  // workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(0);
  // P V of the last tile.  Each of its MFMAs reads operands from every lane,
  // so it must run with the whole wave active; the empty asm statements use
  // the accumulators here, which keeps the compiler from sinking the
  // products into the row-predicated store below.
  {
    const int last = nkt - 1;
    const lds_char* vl = last % 3 == 0 ? vb0 : last % 3 == 1 ? vb1 : vb2;
    pv(vl, pf);
  }
#pragma unroll
  for (int db = 0; db < S::DB; ++db) asm volatile("" : "+v"(oacc[db]));

  const float l_tot = f8_half_sum(l_run[0] + l_run[1]);
  if (row < p.Nq) {
    const float inv = vds / l_tot;
    uint16_t* orow = p.o + ((size_t)bh * p.Nq + row) * D;
#pragma unroll
    for (int db = 0; db < S::DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x2 lo = {(__bf16)(oacc[db][4 * r4 + 0] * inv), (__bf16)(oacc[db][4 * r4 + 1] * inv)};
        bf16x2 hi = {(__bf16)(oacc[db][4 * r4 + 2] * inv), (__bf16)(oacc[db][4 * r4 + 3] * inv)};
        uint2 w;
        w.x = __builtin_bit_cast(unsigned, lo);
        w.y = __builtin_bit_cast(unsigned, hi);
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * r4 + 4 * hl) = w;
      }
    if (hl == 0) p.lse[(size_t)bh * p.Nq + row] = (m_run + log2f(l_tot)) * kLn2;
  }
}


}  // namespace
}  // namespace fa

#define FA_FWD_FP8_KERNEL(NAME, D, NW, CAUSAL)                                          \
  extern "C" __global__ void __launch_bounds__(64 * NW, D == 256 ? 1 : 2) NAME(fa::FwdF8Params p) { \
    using Sh = fa::F8Shape<D, NW>;                                                     \
    __shared__ __attribute__((aligned(1024))) char k0[Sh::TILE];                       \
    __shared__ __attribute__((aligned(1024))) char k1[Sh::TILE];                       \
    __shared__ __attribute__((aligned(1024))) char k2[Sh::TILE];                       \
    __shared__ __attribute__((aligned(1024))) char v0[Sh::TILE];                       \
    __shared__ __attribute__((aligned(1024))) char v1[Sh::TILE];                       \
    __shared__ __attribute__((aligned(1024))) char v2[Sh::TILE];                       \
    fa::fwd_fp8_body<D, NW, CAUSAL>(p, (fa::lds_char*)k0, (fa::lds_char*)k1,           \
                                    (fa::lds_char*)k2, (fa::lds_char*)v0,              \
                                    (fa::lds_char*)v1, (fa::lds_char*)v2);             \
  }

FA_FWD_FP8_KERNEL(fa_fwd_fp8_d32_nomask, 32, 4, false)
FA_FWD_FP8_KERNEL(fa_fwd_fp8_d32_causal, 32, 4, true)
FA_FWD_FP8_KERNEL(fa_fwd_fp8_d64_nomask, 64, 4, false)
FA_FWD_FP8_KERNEL(fa_fwd_fp8_d64_causal, 64, 4, true)
FA_FWD_FP8_KERNEL(fa_fwd_fp8_d128_nomask, 128, 8, false)
FA_FWD_FP8_KERNEL(fa_fwd_fp8_d128_causal, 128, 8, true)
FA_FWD_FP8_KERNEL(fa_fwd_fp8_d256_nomask, 256, 4, false)
FA_FWD_FP8_KERNEL(fa_fwd_fp8_d256_causal, 256, 4, true)


namespace fa {

// Waves per workgroup: eight (two per SIMD) at d = 128, four at d = 32 (four
// workgroups per CU), 64 (three) and 256 (one).
static int fwd_fp8_waves(int d) { return d == 128 ? 8 : 4; }

int fwd_fp8_rows_per_block(int d) { return 32 * fwd_fp8_waves(d); }

const char* fwd_fp8_kernel_name(int d, bool causal) {
  switch (d) {
    case 32: return causal ? "fa_fwd_fp8_d32_causal" : "fa_fwd_fp8_d32_nomask";
    case 64: return causal ? "fa_fwd_fp8_d64_causal" : "fa_fwd_fp8_d64_nomask";
    case 128: return causal ? "fa_fwd_fp8_d128_causal" : "fa_fwd_fp8_d128_nomask";
    case 256: return causal ? "fa_fwd_fp8_d256_causal" : "fa_fwd_fp8_d256_nomask";
    default: return nullptr;
  }
}

hipError_t launch_fwd_fp8(const FwdF8Params& p, int d, bool causal, hipStream_t s) {
  const void* fn = nullptr;
  switch (d) {
    case 32: fn = causal ? (const void*)fa_fwd_fp8_d32_causal : (const void*)fa_fwd_fp8_d32_nomask; break;
    case 64: fn = causal ? (const void*)fa_fwd_fp8_d64_causal : (const void*)fa_fwd_fp8_d64_nomask; break;
    case 128: fn = causal ? (const void*)fa_fwd_fp8_d128_causal : (const void*)fa_fwd_fp8_d128_nomask; break;
    case 256: fn = causal ? (const void*)fa_fwd_fp8_d256_causal : (const void*)fa_fwd_fp8_d256_nomask; break;
    default: return hipErrorInvalidValue;
  }
  const int bm = fwd_fp8_rows_per_block(d);
  const dim3 grid((unsigned)(((p.Nq + bm - 1) / bm) * p.B * p.Hq));
  FwdF8Params arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, grid, dim3(64 * fwd_fp8_waves(d)), args, 0, s);
}

}  // namespace fa
