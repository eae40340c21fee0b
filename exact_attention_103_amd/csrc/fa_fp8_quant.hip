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
// of d = 128 is half a DPP row).  Sixteen elements per lane keep one more
// stage inside the lane than eight would, and drop the lane distance 8,
// whose exchange takes two DPP moves.

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantMaxBlocks = 1024;

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

template <int D>
struct QShape {
  static constexpr int L = D / 16;          // lanes per row
  static constexpr int RPW = 64 / L;        // rows per wave
  static constexpr int RPB = RPW * (kQuantThreads / 64);   // rows per workgroup pass
  static_assert(D == 64 || D == 128, "rotation head dims");
};

// Sign-bit masks of this lane's 16 elements (0 without rotation).
__device__ __forceinline__ void sign_masks(const int8_t* signs, int j, unsigned (&neg)[16]) {
#pragma unroll
  for (int s = 0; s < 16; ++s) neg[s] = (signs && signs[16 * j + s] < 0) ? 0x80000000u : 0u;
}

// x from lane i ^ M within the 16-lane DPP row, as VALU moves (no LDS):
// M = 1, 2 are quad permutations; M = 4 is the quad permutation i ^ 3
// followed by the half-row mirror (i ^ 7).
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
  } else {
    static_assert(M == 4, "lane distance within an 8-lane group");
    r = __builtin_amdgcn_mov_dpp(v, kQuadXor3, 0xF, 0xF, true);
    r = __builtin_amdgcn_mov_dpp(r, kHalfMirror, 0xF, 0xF, true);
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

// The lane's 16 values as fp32 and, when `rotate`, with the signs applied
// and the Walsh-Hadamard transform of the row.
template <int D>
__device__ __forceinline__ void transform(Row16 w, const unsigned (&neg)[16], bool rotate, int j,
                                          float (&v)[16]) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    v[s] = __uint_as_float(((unsigned)w.lo[s] << 16) ^ neg[s]);
    v[s + 8] = __uint_as_float(((unsigned)w.hi[s] << 16) ^ neg[s + 8]);
  }
  if (!rotate) return;
  // Butterflies over index bits 0..3 (inside the lane).
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if ((s & h) == 0) {
        const float a = v[s], b = v[s + h];
        v[s] = a + b;
        v[s + h] = a - b;
      }
  // Butterflies over index bits 4.. (lane bit m of the row).
  lane_butterfly<1>(v, j);
  lane_butterfly<2>(v, j);
  if constexpr (QShape<D>::L == 8) lane_butterfly<4>(v, j);
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
  unsigned neg[16];
  sign_masks(p.signs, j, neg);
  const int stride = gridDim.x * S::RPB;
  for (int r0 = blockIdx.x * S::RPB; r0 < p.rows; r0 += kQuantUnroll * stride) {
    Row16 w[kQuantUnroll];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) w[u] = load_row<D>(p.x, r0 + u * stride + r_in, p.rows, j);
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const int row = r0 + u * stride + r_in;
      float v[16];
      transform<D>(w[u], neg, p.signs != nullptr, j, v);
      float c[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) c[s] = fminf(fmaxf(v[s] * inv, -448.0f), 448.0f);
      // Byte t of the 16-byte group is element 16j + t.  The two conversions
      // of a dword overwrite both halves, so its "old" operand is only a
      // register to write into: the first source, dead afterwards.
      unsigned o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o[q] = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * q], c[4 * q + 1], __float_as_int(c[4 * q]), false);
        o[q] = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * q + 2], c[4 * q + 3], o[q], true);
      }
      if (row < p.rows)
        *reinterpret_cast<uint4*>(p.codes + (size_t)row * D + 16 * j) = make_uint4(o[0], o[1], o[2], o[3]);
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

FA_FP8_QUANT_KERNELS(64)
FA_FP8_QUANT_KERNELS(128)

namespace fa {

int quant_blocks(int rows, int d) {
  const int rpb = (64 / (d / 16)) * (kQuantThreads / 64);
  const long long need = ((long long)rows + rpb - 1) / rpb;
  return (int)(need < kQuantMaxBlocks ? need : kQuantMaxBlocks);
}

const char* quant_kernel_name(int d, int stage) {
  if (d == 64) return stage == 0 ? "fa_fp8_absmax_d64" : "fa_fp8_quant_d64";
  if (d == 128) return stage == 0 ? "fa_fp8_absmax_d128" : "fa_fp8_quant_d128";
  return nullptr;
}

hipError_t launch_quant(const QuantParams& p, int d, hipStream_t s) {
  const void* k0 = d == 64 ? (const void*)fa_fp8_absmax_d64 : (const void*)fa_fp8_absmax_d128;
  const void* k1 = d == 64 ? (const void*)fa_fp8_quant_d64 : (const void*)fa_fp8_quant_d128;
  QuantParams arg = p;
  void* args[] = {&arg};
  hipError_t e = hipLaunchKernel(k0, dim3(p.nblocks), dim3(kQuantThreads), args, 0, s);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(k1, dim3(p.nblocks), dim3(kQuantThreads), args, 0, s);
}

}  // namespace fa
