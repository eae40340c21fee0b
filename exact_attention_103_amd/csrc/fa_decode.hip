// Split-KV decode (Flash-Decoding) for gfx950.
//
// Pages cited (short names):
//   [Evolution]  "FlashAttention evolution" (sandeep007734.github.io,
//                posts/flashattention-evolution)
//
// Decode has one query row per sequence, so query-side parallelism gives
// almost no work; the key/value sequence is cut into chunks instead and each
// chunk becomes an independent workgroup ([Evolution] §6).  A workgroup owns
// (batch b, KV head, chunk s) and all GT query heads that read that KV head,
// so every K/V byte of the cache is read from HBM once.  It writes the
// chunk's normalised partial output and LSE; a second kernel merges the
// chunks with the log-sum-exp identity ([Evolution] §6, final reduction).
//
// The path is bandwidth bound (about 4 flop per K/V byte at GT = 4), so the
// scores and the PV product use v_dot2_f32_bf16 on packed bf16 pairs rather
// than MFMA, and the design goal is many 16-byte loads in flight:
//   * LPK = d/8 lanes hold one key row (16 bytes each), so one wave-wide load
//     instruction reads 64*16 contiguous bytes (64/LPK whole key rows);
//   * each wave keeps U such loads of K and U of V in flight per iteration;
//   * a dot product is reduced over its LPK lanes with DPP row operations.
// Each group of LPK lanes keeps its own online-softmax state (running max m
// in base-2 units, running sum l, unnormalised accumulator) over the keys it
// saw; at the end of the chunk the lane groups of a wave are merged with
// shuffles and the waves through LDS, with the same identity the merge
// kernel uses.

#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecUnroll = 8;   // wave-wide K loads (and V loads) in flight per iteration

__device__ __forceinline__ float max_raw(float a, float b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of LPK consecutive lanes; every lane of a group ends with
// the group total.  Pairs, quads, halves of a 16-lane row, whole rows, then
// the two rows of a 32-lane half.
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LPK >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (LPK >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (LPK >= 8) x += dpp<0x141>(x);   // row_half_mirror
  if constexpr (LPK >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (LPK >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

template <int D, int GT>
struct DecShape {
  static constexpr int LPK = D / 8;            // lanes per key row
  static constexpr int KPI = 64 / LPK;         // key rows per wave-wide load
  static constexpr int U = kDecUnroll;
  static constexpr int KEYS_WAVE = U * KPI;    // keys per wave per iteration
  static constexpr int KEYS_ITER = kDecWaves * KEYS_WAVE;
  static constexpr int NPART = kDecWaves;       // partial states merged through LDS
  static constexpr int LDS_ACC = NPART * GT * D; // floats
  static_assert(U % 2 == 0, "PV consumes key pairs");
};

template <int D, int GT>
__device__ __forceinline__ void decode_split_body(const DecodeParams& p, float* lds) {
  using S = DecShape<D, GT>;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ks = lane / S::LPK;   // key slot inside one wave-wide load
  const int c = lane % S::LPK;    // 16-byte chunk of the row: d = 8c .. 8c+7

  // Workgroup -> (b, kv head, split, head group); head group innermost so
  // workgroups that share K/V bytes run next to each other.
  const int HG = p.group / GT;
  int id = blockIdx.x;
  const int hg = id % HG;  id /= HG;
  const int s = id % p.splits;  id /= p.splits;
  const int kvh = id % p.Hkv;
  const int b = id / p.Hkv;
  const int h0 = kvh * p.group + hg * GT;   // first query head of this workgroup

  const int kbeg = s * p.chunk;
  const int kend = min(kbeg + p.chunk, p.Nk);

  // Queries: 8 bf16 per lane per head, as 4 packed pairs.
  unsigned qw[GT][4];
#pragma unroll
  for (int gq = 0; gq < GT; ++gq) {
    const uint4 t = *reinterpret_cast<const uint4*>(
        p.q + ((size_t)(b * p.Hq + h0 + gq)) * D + 8 * c);
    qw[gq][0] = t.x; qw[gq][1] = t.y; qw[gq][2] = t.z; qw[gq][3] = t.w;
  }

  float m[GT], l[GT], acc[GT][8];
#pragma unroll
  for (int gq = 0; gq < GT; ++gq) {
    m[gq] = -1e30f;
    l[gq] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[gq][e] = 0.f;
  }

  const size_t kvoff = ((size_t)(b * p.Hkv + kvh)) * p.Nk * D;
  const uint16_t* kb = p.k + kvoff;
  const uint16_t* vb = p.v + kvoff;

  for (int base = kbeg + wave * S::KEYS_WAVE; base < kend; base += S::KEYS_ITER) {
    uint4 kv[S::U], vv[S::U];
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int key = base + u * S::KPI + ks;
      if (key < kend) {
        kv[u] = *reinterpret_cast<const uint4*>(kb + (size_t)key * D + 8 * c);
        vv[u] = *reinterpret_cast<const uint4*>(vb + (size_t)key * D + 8 * c);
      } else {
        kv[u] = make_uint4(0, 0, 0, 0);
        vv[u] = make_uint4(0, 0, 0, 0);
      }
    }

    // Scores in base-2 units; keys past the chunk end are -inf.
    float sc[S::U][GT];
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const bool ok = base + u * S::KPI + ks < kend;
#pragma unroll
      for (int gq = 0; gq < GT; ++gq) {
        float t = dot2(kv[u].x, qw[gq][0], 0.f);
        t = dot2(kv[u].y, qw[gq][1], t);
        t = dot2(kv[u].z, qw[gq][2], t);
        t = dot2(kv[u].w, qw[gq][3], t);
        t = group_sum<S::LPK>(t);
        sc[u][gq] = ok ? t * p.c : -INFINITY;
      }
    }

    // Online softmax update of this lane group's state.
#pragma unroll
    for (int gq = 0; gq < GT; ++gq) {
      float mx = sc[0][gq];
#pragma unroll
      for (int u = 1; u < S::U; ++u) mx = max_raw(mx, sc[u][gq]);
      const float m_new = max_raw(m[gq], mx);
      const float alpha = __builtin_amdgcn_exp2f(m[gq] - m_new);
      m[gq] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int u = 0; u < S::U; ++u) {
        sc[u][gq] = __builtin_amdgcn_exp2f(sc[u][gq] - m_new);
        ls += sc[u][gq];
      }
      l[gq] = l[gq] * alpha + ls;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[gq][e] *= alpha;
    }

    // acc += P V over key pairs: (V[u][d], V[u+1][d]) . (p[u], p[u+1]).
#pragma unroll
    for (int u = 0; u < S::U; u += 2) {
      const unsigned a[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
      const unsigned bq[4] = {vv[u + 1].x, vv[u + 1].y, vv[u + 1].z, vv[u + 1].w};
      unsigned x[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        x[2 * w] = __builtin_amdgcn_perm(bq[w], a[w], 0x05040100u);
        x[2 * w + 1] = __builtin_amdgcn_perm(bq[w], a[w], 0x07060302u);
      }
#pragma unroll
      for (int gq = 0; gq < GT; ++gq) {
        const unsigned pp = pack_bf16(sc[u][gq], sc[u + 1][gq]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[gq][e] = dot2(x[e], pp, acc[gq][e]);
      }
    }
  }

  // Merge the lane groups of each wave (same chunk c, different key slot)
  // with shuffles, then the waves through LDS.
#pragma unroll
  for (int x = S::LPK; x < 64; x *= 2) {
#pragma unroll
    for (int gq = 0; gq < GT; ++gq) {
      const float mo = __shfl_xor(m[gq], x);
      const float lo = __shfl_xor(l[gq], x);
      const float mn = max_raw(m[gq], mo);
      const float ws = __builtin_amdgcn_exp2f(m[gq] - mn);
      const float wo = __builtin_amdgcn_exp2f(mo - mn);
      m[gq] = mn;
      l[gq] = ws * l[gq] + wo * lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[gq][e] = ws * acc[gq][e] + wo * __shfl_xor(acc[gq][e], x);
    }
  }
  float* sm_m = lds;                              // [NPART][GT]
  float* sm_l = sm_m + S::NPART * GT;             // [NPART][GT]
  float* sm_acc = sm_l + S::NPART * GT;           // [NPART][GT][D]
  if (ks == 0) {
    if (c == 0) {
#pragma unroll
      for (int gq = 0; gq < GT; ++gq) {
        sm_m[wave * GT + gq] = m[gq];
        sm_l[wave * GT + gq] = l[gq];
      }
    }
#pragma unroll
    for (int gq = 0; gq < GT; ++gq) {
      float4* dst = reinterpret_cast<float4*>(sm_acc + ((size_t)wave * GT + gq) * D + 8 * c);
      dst[0] = make_float4(acc[gq][0], acc[gq][1], acc[gq][2], acc[gq][3]);
      dst[1] = make_float4(acc[gq][4], acc[gq][5], acc[gq][6], acc[gq][7]);
    }
  }
  __syncthreads();

  for (int o = tid; o < GT * D; o += kDecThreads) {
    const int gq = o / D, dd = o % D;
    float M = -1e30f;
    for (int i = 0; i < S::NPART; ++i) M = max_raw(M, sm_m[i * GT + gq]);
    float W = 0.f, O = 0.f;
    for (int i = 0; i < S::NPART; ++i) {
      const float w = __builtin_amdgcn_exp2f(sm_m[i * GT + gq] - M);
      W += w * sm_l[i * GT + gq];
      O += w * sm_acc[((size_t)i * GT + gq) * D + dd];
    }
    const int hq = h0 + gq;
    const size_t ps = ((size_t)(b * p.Hq + hq)) * p.splits + s;
    if (W > 0.f) {
      p.o_part[ps * D + dd] = O / W;
      if (dd == 0) p.lse_part[ps] = (M + log2f(W)) * kLn2;
    } else {   // empty chunk: weight 0 in the merge
      p.o_part[ps * D + dd] = 0.f;
      if (dd == 0) p.lse_part[ps] = -INFINITY;
    }
  }
}

// Merge: one workgroup of kMergeThreads per (b, query head).  The split
// LSEs are read in parallel and reduced through LDS; then thread t sums the
// splits s = t / D, t / D + SP, ... for output column t % D with independent
// loads, and the SP partial sums per column are added in a fixed order.
constexpr int kMergeThreads = 256;

template <int D>
__device__ __forceinline__ void decode_merge_body(const DecodeParams& p) {
  constexpr int SP = kMergeThreads / D;       // split phases per column
  __shared__ float red[kMergeThreads];
  __shared__ float part[kMergeThreads];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int S = p.splits;
  const float* lp = p.lse_part + (size_t)bh * S;
  const float* op = p.o_part + (size_t)bh * S * D;

  float mx = -INFINITY;
  for (int s = tid; s < S; s += kMergeThreads) mx = max_raw(mx, lp[s]);
  red[tid] = mx;
  __syncthreads();
  for (int w = kMergeThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = max_raw(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];   // finite: chunk 0 always holds at least one key
  __syncthreads();

  const int dd = tid % D, ph = tid / D;
  float O = 0.f, W = 0.f;
#pragma unroll 8
  for (int s = ph; s < S; s += SP) {
    const float ls = lp[s];
    const float w = ls == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((ls - M) * kLog2e);
    W += w;
    O += w * op[(size_t)s * D + dd];
  }
  part[tid] = O;
  red[tid] = W;
  __syncthreads();
  if (ph == 0) {
    float Ot = 0.f, Wt = 0.f;
#pragma unroll
    for (int q = 0; q < SP; ++q) {
      Ot += part[q * D + dd];
      Wt += red[q * D + dd];
    }
    bf16x2 v = {(__bf16)(Ot / Wt), (__bf16)0.f};
    p.o[(size_t)bh * D + dd] = __builtin_bit_cast(unsigned, v) & 0xFFFFu;
    if (dd == 0) p.lse[bh] = M + logf(Wt);
  }
}

}  // namespace
}  // namespace fa

#define FA_DEC_SPLIT(D, GT)                                                           \
  extern "C" __global__ void __launch_bounds__(fa::kDecThreads)                       \
      fa_decode_split_d##D##_g##GT(fa::DecodeParams p) {                             \
    __shared__ __attribute__((aligned(16)))                                           \
        float lds[2 * fa::DecShape<D, GT>::NPART * GT + fa::DecShape<D, GT>::LDS_ACC]; \
    fa::decode_split_body<D, GT>(p, lds);                                             \
  }

#define FA_DEC_MERGE(D)                                                               \
  extern "C" __global__ void __launch_bounds__(fa::kMergeThreads) fa_decode_merge_d##D( \
      fa::DecodeParams p) {                                                           \
    fa::decode_merge_body<D>(p);                                                      \
  }

#define FA_DEC_ALL(D) \
  FA_DEC_SPLIT(D, 1) FA_DEC_SPLIT(D, 2) FA_DEC_SPLIT(D, 4) FA_DEC_SPLIT(D, 8) FA_DEC_MERGE(D)

FA_DEC_ALL(32)
FA_DEC_ALL(64)
FA_DEC_ALL(128)
FA_DEC_ALL(256)

namespace fa {

int decode_group_tile(int group) {
  if (group % 8 == 0) return 8;
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

namespace {

const void* split_fn(int d, int gt) {
#define FA_CASE(D)                                                   \
  case D:                                                            \
    switch (gt) {                                                    \
      case 1: return (const void*)fa_decode_split_d##D##_g1;         \
      case 2: return (const void*)fa_decode_split_d##D##_g2;         \
      case 4: return (const void*)fa_decode_split_d##D##_g4;         \
      case 8: return (const void*)fa_decode_split_d##D##_g8;         \
    }                                                                \
    return nullptr;
  switch (d) {
    FA_CASE(32)
    FA_CASE(64)
    FA_CASE(128)
    FA_CASE(256)
  }
#undef FA_CASE
  return nullptr;
}

const void* merge_fn(int d) {
  switch (d) {
    case 32: return (const void*)fa_decode_merge_d32;
    case 64: return (const void*)fa_decode_merge_d64;
    case 128: return (const void*)fa_decode_merge_d128;
    case 256: return (const void*)fa_decode_merge_d256;
  }
  return nullptr;
}

}  // namespace

const char* decode_kernel_name(int d, int group, int stage) {
  static const char* const split_names[4][4] = {
      {"fa_decode_split_d32_g1", "fa_decode_split_d32_g2", "fa_decode_split_d32_g4", "fa_decode_split_d32_g8"},
      {"fa_decode_split_d64_g1", "fa_decode_split_d64_g2", "fa_decode_split_d64_g4", "fa_decode_split_d64_g8"},
      {"fa_decode_split_d128_g1", "fa_decode_split_d128_g2", "fa_decode_split_d128_g4", "fa_decode_split_d128_g8"},
      {"fa_decode_split_d256_g1", "fa_decode_split_d256_g2", "fa_decode_split_d256_g4", "fa_decode_split_d256_g8"}};
  static const char* const merge_names[4] = {"fa_decode_merge_d32", "fa_decode_merge_d64",
                                             "fa_decode_merge_d128", "fa_decode_merge_d256"};
  int di;
  switch (d) {
    case 32: di = 0; break;
    case 64: di = 1; break;
    case 128: di = 2; break;
    case 256: di = 3; break;
    default: return nullptr;
  }
  if (group <= 0) return nullptr;
  if (stage == 1) return merge_names[di];
  if (stage != 0) return nullptr;
  const int gt = decode_group_tile(group);
  const int gi = gt == 1 ? 0 : gt == 2 ? 1 : gt == 4 ? 2 : 3;
  return split_names[di][gi];
}

hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t s) {
  const int gt = decode_group_tile(p.group);
  const void* f1 = split_fn(d, gt);
  const void* f2 = merge_fn(d);
  if (!f1 || !f2) return hipErrorInvalidValue;
  DecodeParams arg = p;
  void* args[] = {&arg};
  const unsigned n1 = (unsigned)(p.B * p.Hkv * p.splits * (p.group / gt));
  hipError_t e = hipLaunchKernel(f1, dim3(n1), dim3(kDecThreads), args, 0, s);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(f2, dim3((unsigned)(p.B * p.Hq)), dim3(kMergeThreads), args, 0, s);
}

}  // namespace fa
