// FP8 input step for gfx950: incoherent processing and per-tensor e4m3
// quantisation of Q, K (rotated) and V (not rotated).
//
// Pages cited (short names):
//   [Evolution]  "FlashAttention evolution" (sandeep007734.github.io,
//                posts/flashattention-evolution)
//   [Comparison] "FlashAttention 1-4 generation comparison"
//                (phantomic12.github.io, inference-research)
//
// FlashAttention-3's fp8 mode multiplies Q and K along the head dimension by
// one random orthogonal matrix, a Hadamard matrix with random signs, before
// quantising ([Comparison] "Notes", FA-3 entry; [Evolution] §4): Q Kᵀ is
// unchanged and an outlier channel is spread over all d channels, so the
// per-tensor scale loses less range.  With R = diag(signs) H_d / sqrt(d)
// (H_d the Sylvester Hadamard matrix) this step produces
//   u        = (x ∘ signs) · H_d          fast Walsh-Hadamard transform, fp32
//   descale  = max|u| / (448 sqrt(d))     so that code · descale ≈ x · R
//   code     = e4m3(448 · u / max|u|)     round to nearest even, ±448 clamp
// and without signs u = x, descale = max|x| / 448.  The 1/sqrt(d) of R only
// enters the reported descale: the code of an element depends on u / max|u|,
// which the normalisation does not change.
//
// Two HBM-bound passes (the tensor-wide maximum sits between them):
//   fa_fp8_absmax_d*    each workgroup transforms a grid-strided share of the
//                       rows and writes its largest |u| to the workspace;
//   fa_fp8_quant_d*     each workgroup reduces the workspace (all of them
//                       alike, so no ordering between workgroups is needed),
//                       transforms its rows again and stores the codes;
//                       workgroup 0 writes the descale.
// Recomputing the transform costs one more read of x (2 bytes per element)
// instead of writing and reading an fp32 copy (8).
//
// Row layout: a row of d bf16 values is d/16 lanes x 32 bytes, so one wave
// holds 64/(d/16) rows; lane j of a row holds elements 16j .. 16j+15.  The
// transform's four low index bits are butterflies inside a lane (one add or
// subtract per element each), the others butterflies between lanes j and
// j ^ m, exchanged with DPP moves inside the 16-lane rows of the wave (a row
// of d = 32 is an eighth of a DPP row, of d = 64 a quarter, of d = 128 half
// of one, of d = 256 a whole one, where distance 8 is the row rotation by 8
// lanes).  Sixteen
// elements per lane keep one more stage inside the lane than eight would.
// With rotation, d = 128 moves its three high bits into the lanes through
// an LDS transpose instead (below).

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantMaxBlocks = 1024;

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

template <int D>
struct QShape {
  static constexpr int L = D / 16;          // lanes per row
  static constexpr int RPW = 64 / L;        // rows per wave
  static constexpr int RPB = RPW * (kQuantThreads / 64);   // rows per workgroup pass
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "rotation head dims");
};

// Sign-bit masks of this lane's 16 elements (0 without rotation).
__device__ __forceinline__ void sign_masks(const int8_t* signs, int j, unsigned (&neg)[16]) {
#pragma unroll
  for (int s = 0; s < 16; ++s) neg[s] = (signs && signs[16 * j + s] < 0) ? 0x80000000u : 0u;
}

// x from lane i ^ M within the 16-lane DPP row, as VALU moves (no LDS):
// M = 1, 2 are quad permutations; M = 4 is the quad permutation i ^ 3
// followed by the half-row mirror (i ^ 7); M = 8 is the row rotation by 8
// lanes (i + 8 mod 16 = i ^ 8).
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  const int v = __float_as_int(x);
  constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kQuadXor3 = 0x1B;
  constexpr int kHalfMirror = 0x141;
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_mov_dpp(v, kQuadXor1, 0xF, 0xF, true);
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_mov_dpp(v, kQuadXor2, 0xF, 0xF, true);
  } else if constexpr (M == 4) {
    r = __builtin_amdgcn_mov_dpp(v, kQuadXor3, 0xF, 0xF, true);
    r = __builtin_amdgcn_mov_dpp(r, kHalfMirror, 0xF, 0xF, true);
  } else {
    static_assert(M == 8, "lane distance within a 16-lane row");
    constexpr int kRowRotate8 = 0x128;
    r = __builtin_amdgcn_mov_dpp(v, kRowRotate8, 0xF, 0xF, true);
  }
  return __int_as_float(r);
}

// One butterfly stage between lanes j and j ^ M: the lane with bit M clear
// keeps a + b, its partner a - b, i.e. partner's value + (+-1) * own value
// (one exact FMA: the product by +-1 does not round).
template <int M>
__device__ __forceinline__ void lane_butterfly(float (&v)[16], int j) {
  const float sgn = (j & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int s = 0; s < 16; ++s) v[s] = fmaf(sgn, v[s], lane_xor<M>(v[s]));
}

// This lane's 32 bytes of row `row` (zeros past the last row).
struct Row16 {
  u16x8 lo, hi;
};
template <int D>
__device__ __forceinline__ Row16 load_row(const uint16_t* x, int row, int rows, int j) {
  Row16 w = {};
  if (row < rows) {
    const u16x8* src = reinterpret_cast<const u16x8*>(x + (size_t)row * D + 16 * j);
    w.lo = src[0];
    w.hi = src[1];
  }
  return w;
}

// The lane's 16 bf16 values as fp32, with the signs applied.
__device__ __forceinline__ void to_f32(Row16 w, const unsigned (&neg)[16], float (&v)[16]) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    v[s] = __uint_as_float(((unsigned)w.lo[s] << 16) ^ neg[s]);
    v[s + 8] = __uint_as_float(((unsigned)w.hi[s] << 16) ^ neg[s + 8]);
  }
}

// Butterflies over the bits of `bits` (a set of register index bits):
// register s with the bit clear keeps a + b, its partner s + h gets a - b.
template <int BITS>
__device__ __forceinline__ void inlane_butterflies(float (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
    if ((BITS & h) == 0) continue;
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if ((s & h) == 0) {
        const float a = v[s], b = v[s + h];
        v[s] = a + b;
        v[s + h] = a - b;
      }
  }
}

// The lane's 16 values as fp32 and, when `rotate`, with the signs applied
// and the Walsh-Hadamard transform of the row: index bits 0..3 in the lane,
// the higher bits (one at d = 32, two at d = 64, four at d = 256; d = 128 takes this path
// only without rotation) between the row's lanes through DPP moves.
template <int D>
__device__ __forceinline__ void transform(Row16 w, const unsigned (&neg)[16], bool rotate, int j,
                                          float (&v)[16]) {
  to_f32(w, neg, v);
  if (!rotate) return;
  inlane_butterflies<15>(v);
  lane_butterfly<1>(v, j);
  if constexpr (QShape<D>::L >= 4) lane_butterfly<2>(v, j);
  if constexpr (QShape<D>::L >= 8) lane_butterfly<4>(v, j);
  if constexpr (QShape<D>::L >= 16) lane_butterfly<8>(v, j);
}

// d = 128 with rotation: the transform runs entirely inside lanes, with one
// transpose through LDS per pass.  In row-major order lane j of a row holds
// elements 16j + c (c = 0..15, index bits 0..3); in column order it holds
// elements 16k + c for its two columns c = 2j, 2j + 1 and k = 0..7 (index
// bits 4..6), in registers 2k + (c & 1).  Each wave has its own region per
// row group: 8 rows of 576 bytes (512 used).  The 16-byte chunk q of group k
// (elements 16k + 4q .. +3) of row rw sits at chunk q ^ ((k >> 2) | 2 (rw &
// 1)) of the group's 64 bytes, so that the row-major 16-byte accesses (16
// lanes per LDS pass: two rows) and the column 8-byte accesses (32 lanes
// per pass: four rows) each touch all 64 banks once.
constexpr int kTRowBytes = 576;
constexpr int kTRegion = 8 * kTRowBytes;

__device__ __forceinline__ int tchunk(int rw, int k, int q) {
  return rw * kTRowBytes + k * 64 + ((q ^ ((k >> 2) | ((rw & 1) << 1))) << 4);
}

// Row-major registers (v[c], lane j) -> LDS -> column registers (t[2k + c&1]).
__device__ __forceinline__ void rows_to_columns(lds_char* reg, int rw, int j, const float (&v)[16],
                                                float (&t)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *(__attribute__((address_space(3))) f32x4*)(reg + tchunk(rw, j, q)) =
        f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const f32x2 x =
        *(const __attribute__((address_space(3))) f32x2*)(reg + tchunk(rw, k, j >> 1) + 8 * (j & 1));
    t[2 * k] = x[0];
    t[2 * k + 1] = x[1];
  }
}

// Column registers -> LDS -> row-major registers.
__device__ __forceinline__ void columns_to_rows(lds_char* reg, int rw, int j, const float (&t)[16],
                                                float (&v)[16]) {
#pragma unroll
  for (int k = 0; k < 8; ++k)
    *(__attribute__((address_space(3))) f32x2*)(reg + tchunk(rw, k, j >> 1) + 8 * (j & 1)) =
        f32x2{t[2 * k], t[2 * k + 1]};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 x = *(const __attribute__((address_space(3))) f32x4*)(reg + tchunk(rw, j, q));
    v[4 * q] = x[0];
    v[4 * q + 1] = x[1];
    v[4 * q + 2] = x[2];
    v[4 * q + 3] = x[3];
  }
}

// Sign-bit masks of the lane's elements in column order (d = 128).
__device__ __forceinline__ void sign_masks_cols(const int8_t* signs, int j, unsigned (&neg)[16]) {
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      neg[2 * k + h] = (signs && signs[16 * k + 2 * j + h] < 0) ? 0x80000000u : 0u;
}

// Rows are visited in steps of kQuantUnroll row groups per workgroup, whose
// loads are all issued before the first transform (more bytes in flight per
// wave).
constexpr int kQuantUnroll = 2;

__device__ __forceinline__ float block_max(float x, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

template <int D>
__device__ __forceinline__ void absmax_body(const QuantParams& p) {
  using S = QShape<D>;
  __shared__ float red[kQuantThreads / 64];
  const int lane = threadIdx.x & 63;
  const int j = lane % S::L;
  const int r_in = (threadIdx.x >> 6) * S::RPW + lane / S::L;
  unsigned neg[16];
  sign_masks(p.signs, j, neg);
  float mx = 0.f;
  const int stride = gridDim.x * S::RPB;
  if constexpr (D == 128) {
    if (p.signs) {
      // Row-major loads, bits 0..3 in the lane, transpose, bits 4..6 in the lane.
      __shared__ __attribute__((aligned(16))) char tb[kQuantThreads / 64][kQuantUnroll][kTRegion];
      const int wave = threadIdx.x >> 6, rw = lane / S::L;
      for (int r0 = blockIdx.x * S::RPB; r0 < p.rows; r0 += kQuantUnroll * stride) {
        Row16 w[kQuantUnroll];
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u)
          w[u] = load_row<D>(p.x, r0 + u * stride + r_in, p.rows, j);
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) {
          float v[16], t[16];
          to_f32(w[u], neg, v);
          inlane_butterflies<15>(v);
          rows_to_columns((lds_char*)tb[wave][u], rw, j, v, t);
          inlane_butterflies<14>(t);
#pragma unroll
          for (int s = 0; s < 16; ++s) mx = fmaxf(mx, fabsf(t[s]));
        }
      }
      mx = block_max(mx, red);
      if (threadIdx.x == 0) p.partial[blockIdx.x] = mx;
      return;
    }
  }
  for (int r0 = blockIdx.x * S::RPB; r0 < p.rows; r0 += kQuantUnroll * stride) {
    Row16 w[kQuantUnroll];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) w[u] = load_row<D>(p.x, r0 + u * stride + r_in, p.rows, j);
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      float v[16];
      transform<D>(w[u], neg, p.signs != nullptr, j, v);
#pragma unroll
      for (int s = 0; s < 16; ++s) mx = fmaxf(mx, fabsf(v[s]));
    }
  }
  mx = block_max(mx, red);
  if (threadIdx.x == 0) p.partial[blockIdx.x] = mx;
}

template <int D>
__device__ __forceinline__ void quant_body(const QuantParams& p) {
  using S = QShape<D>;
  __shared__ float red[kQuantThreads / 64];
  float mx = 0.f;
  for (int i = threadIdx.x; i < p.nblocks; i += kQuantThreads) mx = fmaxf(mx, p.partial[i]);
  const float amax = block_max(mx, red);
  const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0)
    *p.descale = amax > 0.f ? amax / (448.0f * p.norm) : 1.0f;

  const int lane = threadIdx.x & 63;
  const int j = lane % S::L;
  const int r_in = (threadIdx.x >> 6) * S::RPW + lane / S::L;
  const int stride = gridDim.x * S::RPB;
  // Codes of one row group: byte t of the lane's 16-byte group is element
  // 16j + t.  The two conversions of a dword overwrite both halves, so its
  // "old" operand is only a register to write into: the first source, dead
  // afterwards.
  auto store_codes = [&](int row, const float (&v)[16]) {
    float c[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) c[s] = fminf(fmaxf(v[s] * inv, -448.0f), 448.0f);
    unsigned o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[q] = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * q], c[4 * q + 1], __float_as_int(c[4 * q]), false);
      o[q] = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * q + 2], c[4 * q + 3], o[q], true);
    }
    if (row < p.rows)
      *reinterpret_cast<uint4*>(p.codes + (size_t)row * D + 16 * j) = make_uint4(o[0], o[1], o[2], o[3]);
  };
  if constexpr (D == 128) {
    if (p.signs) {
      // Column-order loads (4 bytes: elements 16k + 2j, 16k + 2j + 1), bits
      // 4..6 in the lane, transpose, bits 0..3 in the lane, row-major store.
      __shared__ __attribute__((aligned(16))) char tb[kQuantThreads / 64][kQuantUnroll][kTRegion];
      const int wave = threadIdx.x >> 6, rw = lane / S::L;
      unsigned negc[16];
      sign_masks_cols(p.signs, j, negc);
      for (int r0 = blockIdx.x * S::RPB; r0 < p.rows; r0 += kQuantUnroll * stride) {
        unsigned w[kQuantUnroll][8];
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) {
          const int row = r0 + u * stride + r_in;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            w[u][k] = row < p.rows
                          ? *reinterpret_cast<const unsigned*>(p.x + (size_t)row * D + 16 * k + 2 * j)
                          : 0u;
        }
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) {
          float t[16], v[16];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            t[2 * k] = __uint_as_float((w[u][k] << 16) ^ negc[2 * k]);
            t[2 * k + 1] = __uint_as_float((w[u][k] & 0xFFFF0000u) ^ negc[2 * k + 1]);
          }
          inlane_butterflies<14>(t);
          columns_to_rows((lds_char*)tb[wave][u], rw, j, t, v);
          inlane_butterflies<15>(v);
          store_codes(r0 + u * stride + r_in, v);
        }
      }
      return;
    }
  }
  unsigned neg[16];
  sign_masks(p.signs, j, neg);
  for (int r0 = blockIdx.x * S::RPB; r0 < p.rows; r0 += kQuantUnroll * stride) {
    Row16 w[kQuantUnroll];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) w[u] = load_row<D>(p.x, r0 + u * stride + r_in, p.rows, j);
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      float v[16];
      transform<D>(w[u], neg, p.signs != nullptr, j, v);
      store_codes(r0 + u * stride + r_in, v);
    }
  }
}

}  // namespace
}  // namespace fa

#define FA_FP8_QUANT_KERNELS(D)                                                              \
  extern "C" __global__ void __launch_bounds__(fa::kQuantThreads) fa_fp8_absmax_d##D(      \
      fa::QuantParams p) {                                                                 \
    fa::absmax_body<D>(p);                                                                 \
  }                                                                                        \
  extern "C" __global__ void __launch_bounds__(fa::kQuantThreads) fa_fp8_quant_d##D(       \
      fa::QuantParams p) {                                                                 \
    fa::quant_body<D>(p);                                                                  \
  }

FA_FP8_QUANT_KERNELS(32)
FA_FP8_QUANT_KERNELS(64)
FA_FP8_QUANT_KERNELS(128)
FA_FP8_QUANT_KERNELS(256)

namespace fa {

int quant_blocks(int rows, int d) {
  const int rpb = (64 / (d / 16)) * (kQuantThreads / 64);
  const long long need = ((long long)rows + rpb - 1) / rpb;
  return (int)(need < kQuantMaxBlocks ? need : kQuantMaxBlocks);
}

const char* quant_kernel_name(int d, int stage) {
  if (d == 32) return stage == 0 ? "fa_fp8_absmax_d32" : "fa_fp8_quant_d32";
  if (d == 64) return stage == 0 ? "fa_fp8_absmax_d64" : "fa_fp8_quant_d64";
  if (d == 128) return stage == 0 ? "fa_fp8_absmax_d128" : "fa_fp8_quant_d128";
  if (d == 256) return stage == 0 ? "fa_fp8_absmax_d256" : "fa_fp8_quant_d256";
  return nullptr;
}

hipError_t launch_quant(const QuantParams& p, int d, hipStream_t s) {
  const void *k0, *k1;
  switch (d) {
    case 32: k0 = (const void*)fa_fp8_absmax_d32; k1 = (const void*)fa_fp8_quant_d32; break;
    case 64: k0 = (const void*)fa_fp8_absmax_d64; k1 = (const void*)fa_fp8_quant_d64; break;
    case 128: k0 = (const void*)fa_fp8_absmax_d128; k1 = (const void*)fa_fp8_quant_d128; break;
    case 256: k0 = (const void*)fa_fp8_absmax_d256; k1 = (const void*)fa_fp8_quant_d256; break;
    default: return hipErrorInvalidValue;
  }
  QuantParams arg = p;
  void* args[] = {&arg};
  hipError_t e = hipLaunchKernel(k0, dim3(p.nblocks), dim3(kQuantThreads), args, 0, s);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(k1, dim3(p.nblocks), dim3(kQuantThreads), args, 0, s);
}

}  // namespace fa
