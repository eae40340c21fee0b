// Exact fused attention forward for gfx950 (CDNA4, wave64, bf16 MFMA).
//
// Pages cited (short names):
//   [Evolution]  "FlashAttention evolution" (sandeep007734.github.io,
//                posts/flashattention-evolution)
//   [Kruglikov]  "Flash Attention" (vladislavkruglikov.com,
//                articles/flash-attention)
//   [Comparison] "FlashAttention 1-4 generation comparison"
//                (phantomic12.github.io, inference-research)
//
// One workgroup owns BM = 32*NW query rows of one (batch, head); each wave64
// owns 32 whole rows and the K/V tile is shared read-only between the waves,
// so no cross-wave reduction exists ([Evolution] §3, Fig. 2: sliced-Q).
// The grid spans batch x head x query block ([Evolution] §3; [Comparison]
// workarounds), heaviest causal blocks first (LPT, [Comparison] workarounds).
//
// Per KV tile of BN keys ([Evolution] §1 invariant, [Kruglikov] "The IO
// problem": score/probability tiles live only in registers):
//   S^T = K Q^T          bf16 MFMA 32x32x16, fp32 accumulate.  Computing the
//                        transpose puts one query per lane, so the row max and
//                        row sum are in-lane except for one lane-half swap.
//   mask                 diagonal / tail tiles only.
//   online softmax       running max m (base-2 units, scale*log2e folded into
//                        one FMA), P = 2^(S*c - m) with v_exp_f32, running
//                        sum l; the accumulator is rescaled only when some
//                        row's maximum rose ([Evolution] §5, the exact case).
//   O^T += V^T P^T       bf16 MFMA; the P^T registers are already the MFMA B
//                        operand because V^T is stored in LDS with its keys
//                        permuted to match (the contraction order is free).
// Normalisation by 1/l happens once at the end ([Evolution] §2 and §3), and
// only O (bf16) and LSE (fp32) are written.
//
// K/V tiles are double-buffered in LDS: the global loads of tile j+1 are in
// flight while tile j is computed, then written to the other buffer (the
// CDNA counterpart of the Hopper asynchronous copies of [Evolution] §4).
// Both LDS tiles use an XOR swizzle on 16-byte chunks so that the MFMA
// operand reads of 16 consecutive rows hit distinct banks.

#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

template <int D, int BN, int NW>
struct FwdShape {
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int KSTEPS = D / 16;   // MFMA k-steps over d (S^T)
  static constexpr int KB = BN / 32;      // 32-key blocks per tile (S^T rows)
  static constexpr int DB = D / 32;       // 32-wide d blocks (O^T rows)
  static constexpr int KC = BN / 16;      // 16-key chunks (PV k-steps)
  static constexpr int RBK = D * 2;       // bytes per K row in LDS
  static constexpr int RBV = BN * 2;      // bytes per V^T row in LDS
  static constexpr int KT_BYTES = BN * RBK;
  static constexpr int VT_BYTES = D * RBV;
  static constexpr int STAGE = KT_BYTES + VT_BYTES;
  static constexpr int CPR = D / 8;       // 16-byte chunks per K/V row
  static constexpr int K_CHUNKS = BN * CPR;
  static constexpr int K_IT = (K_CHUNKS + NT - 1) / NT;
  static constexpr int V_ASSIGN = (BN / 4) * CPR;   // (4-key group, d chunk)
  static constexpr int V_IT = (V_ASSIGN + NT - 1) / NT;
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");
};

// Byte offset of 16-byte chunk c of row r in an LDS tile with RB-byte rows.
// The XOR term differs for any 16 consecutive rows, so 16 lanes reading the
// same logical chunk of consecutive rows touch 16 distinct bank groups.
template <int RB>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int NC = RB / 16;
  int x;
  if constexpr (RB >= 256) {
    x = r & 15;
  } else {
    x = (r / (256 / RB)) & (NC - 1);
  }
  return r * RB + ((c ^ x) << 4);
}

__device__ __forceinline__ float max_raw(float a, float b) { return a > b ? a : b; }

// Combine a value with the same lane of the other 32-lane half.
// The two results of the swap are the lane's own value and its partner's
// (lane l and lane l ^ 32), in an order that depends on the half.
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Position of key kk (0..BN-1) inside a V^T row.  Within every 16 keys the
// two middle bits are swapped: the PV B operand of lane half h, element
// 4a+b (taken straight from the S^T accumulator) is key 8a+4h+b, and it must
// meet V^T element 8h+4a+b of the A operand.
__device__ __forceinline__ int vt_pos(int kk) {
  const int g = (kk >> 2) & 3;
  return (kk & ~15) | ((((g & 1) << 1) | (g >> 1)) << 2) | (kk & 3);
}

template <int D, int BN, int NW, bool CAUSAL>
__device__ __forceinline__ void fwd_body(const FwdParams& p, char* smem) {
  using S = FwdShape<D, BN, NW>;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hl = lane >> 5;   // lane half: selects k sub-block of MFMA operands
  const int n = lane & 31;    // query column of S^T / O^T owned by this lane

  // Grid: query block major (descending when causal, so the longest
  // workgroups start first), (batch, head) minor.
  const int BH = p.B * p.Hq;
  const int nqb = (p.Nq + S::BM - 1) / S::BM;
  const int bh = blockIdx.x % BH;
  const int qi = blockIdx.x / BH;
  const int qblk = CAUSAL ? (nqb - 1 - qi) : qi;
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int g = h / p.group;
  const int q0 = qblk * S::BM;
  const int qw = q0 + 32 * wave;
  const int off = p.Nk - p.Nq;   // key j allowed for row i iff j <= i + off

  const uint16_t* qbase = p.q + (size_t)(b * p.Hq + h) * p.Nq * D;
  const uint16_t* kbase = p.k + (size_t)(b * p.Hkv + g) * p.Nk * D;
  const uint16_t* vbase = p.v + (size_t)(b * p.Hkv + g) * p.Nk * D;

  int nkt = (p.Nk + BN - 1) / BN;
  if (CAUSAL) {
    const int last_row = min(q0 + S::BM, p.Nq) - 1;
    nkt = min(nkt, (last_row + off) / BN + 1);
  }

  // Q rows of this wave as MFMA B operands: lane (h, n) holds
  // Q[qw+n][16t + 8h .. +7] for k-step t.  Rows past Nq are zero.
  bf16x8 qf[S::KSTEPS];
  {
    const int row = qw + n;
#pragma unroll
    for (int t = 0; t < S::KSTEPS; ++t) {
      if (row < p.Nq) {
        qf[t] = *reinterpret_cast<const bf16x8*>(qbase + (size_t)row * D + 16 * t + 8 * hl);
      } else {
        qf[t] = bf16x8{};
      }
    }
  }

  // Register staging of one K/V tile (global -> VGPR -> LDS).
  uint4 kst[S::K_IT];
  uint4 vst[S::V_IT][4];

  auto gload = [&](int j0) {
#pragma unroll
    for (int i = 0; i < S::K_IT; ++i) {
      const int ci = tid + i * S::NT;
      if (S::K_CHUNKS % S::NT == 0 || ci < S::K_CHUNKS) {
        const int row = ci / S::CPR, c = ci % S::CPR;
        const int key = j0 + row;
        kst[i] = key < p.Nk
                     ? *reinterpret_cast<const uint4*>(kbase + (size_t)key * D + c * 8)
                     : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < S::V_IT; ++i) {
      const int a = tid + i * S::NT;
      if (S::V_ASSIGN % S::NT == 0 || a < S::V_ASSIGN) {
        const int kg4 = a % (BN / 4), cd = a / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = j0 + 4 * kg4 + r;
          vst[i][r] = key < p.Nk
                          ? *reinterpret_cast<const uint4*>(vbase + (size_t)key * D + cd * 8)
                          : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  auto lstore = [&](char* st) {
    char* sk = st;
    char* sv = st + S::KT_BYTES;
#pragma unroll
    for (int i = 0; i < S::K_IT; ++i) {
      const int ci = tid + i * S::NT;
      if (S::K_CHUNKS % S::NT == 0 || ci < S::K_CHUNKS) {
        const int row = ci / S::CPR, c = ci % S::CPR;
        *reinterpret_cast<uint4*>(sk + swz<S::RBK>(row, c)) = kst[i];
      }
    }
    // V^T: each thread transposes a 4-key x 8-d block into 8 rows of 4 keys.
#pragma unroll
    for (int i = 0; i < S::V_IT; ++i) {
      const int a = tid + i * S::NT;
      if (S::V_ASSIGN % S::NT == 0 || a < S::V_ASSIGN) {
        const int kg4 = a % (BN / 4), cd = a / (BN / 4);
        const int pos = vt_pos(4 * kg4);
        const int chunk = pos >> 3, half = (pos >> 2) & 1;
        const unsigned* w0 = reinterpret_cast<const unsigned*>(&vst[i][0]);
        const unsigned* w1 = reinterpret_cast<const unsigned*>(&vst[i][1]);
        const unsigned* w2 = reinterpret_cast<const unsigned*>(&vst[i][2]);
        const unsigned* w3 = reinterpret_cast<const unsigned*>(&vst[i][3]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const unsigned lo = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
          const unsigned hi = __builtin_amdgcn_perm(w3[e >> 1], w2[e >> 1], sel);
          *reinterpret_cast<uint2*>(sv + swz<S::RBV>(cd * 8 + e, chunk) + half * 8) =
              make_uint2(lo, hi);
        }
      }
    }
  };

  f32x16 oacc[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db) oacc[db] = f32x16{};
  float m_run = -1e30f;   // finite, so 2^(m_old - m_new) is never inf - inf
  float l_run = 0.f;      // partial row sum over this lane half's keys
  const int row = qw + n;

  gload(0);
  lstore(smem);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int j0 = j * BN;
    const bool more = j + 1 < nkt;
    if (more) gload(j0 + BN);

    bool active = qw < p.Nq;
    if (CAUSAL) active = active && (j0 <= qw + 31 + off);
    if (active) {
      const char* sk = smem + (j & 1) * S::STAGE;
      const char* sv = sk + S::KT_BYTES;

      // S^T = K Q^T
      f32x16 sacc[S::KB];
#pragma unroll
      for (int kb = 0; kb < S::KB; ++kb) {
        sacc[kb] = f32x16{};
#pragma unroll
        for (int t = 0; t < S::KSTEPS; ++t) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(sk + swz<S::RBK>(32 * kb + n, 2 * t + hl));
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], sacc[kb], 0, 0, 0);
        }
      }

      // Mask keys past Nk and, when causal, past the diagonal.
      const bool need_mask = (j0 + BN > p.Nk) || (CAUSAL && j0 + BN - 1 > qw + off);
      if (need_mask) {
        const int lim = CAUSAL ? min(p.Nk - 1, row + off) : p.Nk - 1;
#pragma unroll
        for (int kb = 0; kb < S::KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * kb + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (key > lim) sacc[kb][r] = -INFINITY;
          }
        }
      }

      // Online softmax in base-2 units.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = max_raw(mx, sacc[kb][r]);
      mx = half_max(mx);
      const float m_new = max_raw(m_run, mx * p.c);
      if (__any(m_new > m_run)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < S::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_run = m_new;
      }
      const float nm = -m_run;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < S::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], p.c, nm));
          sacc[kb][r] = e;
          ls += e;
        }
      l_run += ls;

      // P^T as bf16 B operands: chunk kc = registers 8*(kc%2).. of block kc/2.
      bf16x8 pb[S::KC];
#pragma unroll
      for (int kc = 0; kc < S::KC; ++kc)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[kc][i] = (__bf16)sacc[kc >> 1][8 * (kc & 1) + i];

      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < S::DB; ++db)
#pragma unroll
        for (int kc = 0; kc < S::KC; ++kc) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(sv + swz<S::RBV>(32 * db + n, 2 * kc + hl));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc], oacc[db], 0, 0, 0);
        }
    }

    if (more) lstore(smem + ((j + 1) & 1) * S::STAGE);
    __syncthreads();
  }

  // Epilogue: O = acc / l (bf16, round to nearest even), LSE in natural log.
  const float l_tot = half_sum(l_run);
  if (row < p.Nq) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = p.o + ((size_t)(b * p.Hq + h) * p.Nq + row) * D;
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
    if (hl == 0) p.lse[(size_t)(b * p.Hq + h) * p.Nq + row] = (m_run + log2f(l_tot)) * kLn2;
  }
}

}  // namespace
}  // namespace fa

// Kernel symbols carry plain C names so that a profiler trace names exactly
// which variant ran.
#define FA_FWD_KERNEL(NAME, D, BN, NW, CAUSAL, WAVES_PER_EU)                          \
  extern "C" __global__ void __launch_bounds__(64 * NW, WAVES_PER_EU) NAME(           \
      fa::FwdParams p) {                                                              \
    __shared__ __attribute__((aligned(16))) char smem[2 * fa::FwdShape<D, BN, NW>::STAGE]; \
    fa::fwd_body<D, BN, NW, CAUSAL>(p, smem);                                         \
  }

FA_FWD_KERNEL(fa_fwd_d32_nomask, 32, 64, 4, false, 2)
FA_FWD_KERNEL(fa_fwd_d32_causal, 32, 64, 4, true, 2)
FA_FWD_KERNEL(fa_fwd_d64_nomask, 64, 64, 4, false, 2)
FA_FWD_KERNEL(fa_fwd_d64_causal, 64, 64, 4, true, 2)
FA_FWD_KERNEL(fa_fwd_d128_nomask, 128, 64, 4, false, 2)
FA_FWD_KERNEL(fa_fwd_d128_causal, 128, 64, 4, true, 2)
FA_FWD_KERNEL(fa_fwd_d256_nomask, 256, 32, 4, false, 1)
FA_FWD_KERNEL(fa_fwd_d256_causal, 256, 32, 4, true, 1)

namespace fa {

FwdTile fwd_tile(int d) {
  switch (d) {
    case 32: return {128, 64, 4};
    case 64: return {128, 64, 4};
    case 128: return {128, 64, 4};
    case 256: return {128, 32, 4};
    default: return {0, 0, 0};
  }
}

const char* fwd_kernel_name(int d, bool causal) {
  switch (d) {
    case 32: return causal ? "fa_fwd_d32_causal" : "fa_fwd_d32_nomask";
    case 64: return causal ? "fa_fwd_d64_causal" : "fa_fwd_d64_nomask";
    case 128: return causal ? "fa_fwd_d128_causal" : "fa_fwd_d128_nomask";
    case 256: return causal ? "fa_fwd_d256_causal" : "fa_fwd_d256_nomask";
    default: return nullptr;
  }
}

hipError_t launch_fwd(const FwdParams& p, int d, bool causal, hipStream_t s) {
  const FwdTile t = fwd_tile(d);
  const int nqb = (p.Nq + t.bm - 1) / t.bm;
  const dim3 grid((unsigned)(nqb * p.B * p.Hq));
  const dim3 block((unsigned)(64 * t.waves));
  const void* fn = nullptr;
  switch (d) {
    case 32: fn = causal ? (const void*)fa_fwd_d32_causal : (const void*)fa_fwd_d32_nomask; break;
    case 64: fn = causal ? (const void*)fa_fwd_d64_causal : (const void*)fa_fwd_d64_nomask; break;
    case 128: fn = causal ? (const void*)fa_fwd_d128_causal : (const void*)fa_fwd_d128_nomask; break;
    case 256: fn = causal ? (const void*)fa_fwd_d256_causal : (const void*)fa_fwd_d256_nomask; break;
    default: return hipErrorInvalidValue;
  }
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, grid, block, args, 0, s);
}

}  // namespace fa
