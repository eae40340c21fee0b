// Split-KV decode (Flash-Decoding) for gfx950.
//
// Pages cited (short names):
//   [Evolution]  "FlashAttention evolution" (sandeep007734.github.io,
//                posts/flashattention-evolution)
//
// Decode has one query row per sequence, so query-side parallelism gives
// almost no work; the key/value sequence is cut into chunks instead and each
// chunk becomes an independent workgroup ([Evolution] §6).  A workgroup owns
// (batch b, KV head, chunk s) and the GT query heads that read that KV head
// (up to 16), so every K/V byte of the cache is read from HBM once.  It
// writes the chunk's normalised partial output and LSE; a second kernel
// merges the chunks with the log-sum-exp identity ([Evolution] §6, final
// reduction).
//
// The path is bandwidth bound (about 4 flop per K/V byte at GT = 4); the
// arithmetic runs on the matrix cores so that the VALU stays light and the
// waves can keep many loads in flight:
//   * each wave streams its own 16-key tiles (tiles wave, wave+4, ... of the
//     chunk), two tiles ahead;
//   * K goes HBM -> VGPRs directly in the layout of the A operand of
//     S^T = K Q^T (v_mfma_f32_16x16x32_bf16; columns = the GT query heads);
//   * V goes HBM -> LDS with direct-to-LDS loads and feeds O^T += V^T P^T
//     (v_mfma_f32_16x16x16_bf16) through the transposing LDS read; the P^T
//     operand is the S^T accumulator converted to bf16 in place.
// Online softmax per query head in base-2 units (running max, running sum,
// unnormalised accumulator), with the accumulator rescaled only when a
// maximum rises by more than 2^8.  At the end of the chunk the four waves'
// states are merged through LDS with the same identity the merge kernel uses.

#include "fa_internal.h"

#include <limits.h>
#include <math.h>

namespace fa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecTile = 16;                 // keys per wave tile
constexpr float kDecRescaleThreshold = 8.0f;

__device__ __forceinline__ float max_raw(float a, float b) { return a > b ? a : b; }

template <int D>
struct DecShape {
  static constexpr int RB = D * 2;                       // bytes per V row in LDS
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int VTILE = kDecTile * RB;            // bytes of one V tile
  static constexpr int VLOADS = kDecTile * CPR / 64;     // 1 KB wave loads per V tile
  static constexpr int KSTEPS = D / 32;                  // S^T k-steps
  static constexpr int NDB = D / 16;                     // 16-row d blocks of O^T
  static_assert(VLOADS >= 1, "tile shape");
};

// V tile swizzle: 16-byte chunk c of row r sits at c ^ X(r).  The PV operand
// reads take chunks 2db, 2db+1 of all 16 rows; X spreads them so that every
// bank group is hit exactly twice (scaled for rows shorter than 256 bytes).
template <int RB>
__device__ __forceinline__ int dv_xor(int r) {
  if constexpr (RB >= 256) return 2 * (r & 7);
  else if constexpr (RB == 128) return 2 * ((r >> 1) & 3);
  else return 2 * ((r >> 2) & 1);
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// SERVE = false: one query row per sequence, every sequence Nk keys.
// SERVE = true (serving-shaped decode): Nq query rows per sequence and a
// per-sequence key count seqlens[b] <= Nk (Nk is then the cache capacity, the
// row stride of the K/V cache).  The MFMA columns are (query head, row)
// pairs, GT * Nq <= 16 of them; with causal masking row i of sequence b sits
// at position seqlens[b] - Nq + i and sees keys j <= that position.
template <int D, int GT, bool SERVE>
__device__ __forceinline__ void decode_split_body(const DecodeParams& p, lds_char* vs0,
                                                  lds_char* vs1, float* mlds) {
  using S = DecShape<D>;
  static_assert(GT >= 1 && GT <= 16, "query heads per workgroup");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;   // MFMA column: query head h0 + col (or a (head, row) pair)
  const int grp = lane >> 4;   // 16-lane group: k sub-block / row block
  const int nq = SERVE ? p.nq : 1;
  const int cols = GT * nq;                    // live MFMA columns
  const int chd = SERVE ? col / nq : col;      // column -> query head within the tile
  const int crow = SERVE ? col - chd * nq : 0; // column -> query row

  // Workgroup -> (b, kv head, split, head group); head group innermost so
  // workgroups that share K/V bytes run next to each other.
  const int HG = p.group / GT;
  int id = blockIdx.x;
  const int hg = id % HG;  id /= HG;
  const int s = id % p.splits;  id /= p.splits;
  const int kvh = id % p.Hkv;
  const int b = id / p.Hkv;
  const int h0 = kvh * p.group + hg * GT;   // first query head of this workgroup

  int len = p.Nk, chunk = p.chunk;
  if (SERVE) {
    if (p.seqlens) len = min(max(__builtin_amdgcn_readfirstlane(p.seqlens[b]), 0), p.Nk);
    chunk = ((len + p.splits - 1) / p.splits + kDecodeChunkAlign - 1) / kDecodeChunkAlign *
            kDecodeChunkAlign;
  }
  // Causal limit of this lane's column (SERVE only): keys j <= lim.
  const int lim = (SERVE && p.causal) ? len - nq + crow : INT_MAX;
  const int kbeg = s * chunk;
  const int kend = min(kbeg + chunk, len);
  const int ntiles = kend > kbeg ? (kend - kbeg + kDecTile - 1) / kDecTile : 0;
  const int my = ntiles > wave ? (ntiles - wave + kDecWaves - 1) / kDecWaves : 0;

  // Q^T as the B operand: lane (grp, col) holds Q[h0+col][32t + 8grp .. +7].
  bf16x8 qf[S::KSTEPS];
#pragma unroll
  for (int t = 0; t < S::KSTEPS; ++t) {
    qf[t] = col < cols ? *reinterpret_cast<const bf16x8*>(
                             p.q + ((size_t)(b * p.Hq + h0 + chd) * nq + crow) * D + 32 * t +
                             8 * grp)
                       : bf16x8{};
  }

  const size_t kvoff = ((size_t)(b * p.Hkv + kvh)) * p.Nk * D;
  const uint16_t* kb = p.k + kvoff;
  const uint16_t* vb = p.v + kvoff;
  lds_char* v0 = vs0 + wave * S::VTILE;
  lds_char* v1 = vs1 + wave * S::VTILE;

  // Transposing-read offsets: lane j of group grp addresses row 4*grp + j/4,
  // columns 16db + 4*(j&3), so it receives V[4grp + k][16db + j] for k = 0..3.
  const int vrow = 4 * grp + (col >> 2);
  const int vx = dv_xor<S::RB>(vrow) >> 1;
  const int voff = vrow * S::RB + 16 * ((col & 3) >> 1) + 8 * (col & 1);

  // Issue the loads of this wave's i-th tile: K rows into registers (A
  // operand layout: lane (grp, col) takes key col, d = 32t + 8grp ..), V rows
  // into LDS.  Keys past the chunk end re-read its last key (masked later).
  // Every K/V byte is read once, so both loads are nontemporal (the `nt`
  // cache policy): a 1 GiB streaming read measured 6.8 TB/s with it against
  // 6.2 without.
  auto issue = [&](int i, bf16x8 (&kf)[S::KSTEPS], lds_char* vt) {
    FA_STAGE_WAIT();
    const int tb = kbeg + kDecTile * (wave + kDecWaves * i);
    const int key = min(tb + col, kend - 1);
#pragma unroll
    for (int t = 0; t < S::KSTEPS; ++t)
      kf[t] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                             kb + (size_t)key * D + 32 * t + 8 * grp)));
#pragma unroll
    for (int L = 0; L < S::VLOADS; ++L) {
      const int P = L * 64 + lane;
      const int row = P / S::CPR;
      const int c = (P % S::CPR) ^ dv_xor<S::RB>(row);
      const int vkey = min(tb + row, kend - 1);
      __builtin_amdgcn_global_load_lds(vb + (size_t)vkey * D + c * 8, vt + L * 1024, 16, 0,
                                       kCachePolicyNT);
    }
    FA_STAGE_WAIT();
  };

  float m = -1e30f;   // running max (base 2) of query h0+col, same in all lane groups
  float l = 0.f;      // running sum over this lane group's keys
  f32x4 oacc[S::NDB];
#pragma unroll
  for (int db = 0; db < S::NDB; ++db) oacc[db] = f32x4{};

  auto process = [&](int i, const bf16x8 (&kf)[S::KSTEPS], const lds_char* vt) {
    const int tb = kbeg + kDecTile * (wave + kDecWaves * i);
    // S^T: lane (grp, col) gets keys tb + 4grp + r (r = 0..3) of query col.
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int t = 0; t < S::KSTEPS; ++t)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t], qf[t], sacc, 0, 0, 0);
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sv[r] = (tb + 4 * grp + r < kend && (!SERVE || tb + 4 * grp + r <= lim))
                  ? sacc[r] * p.c
                  : -INFINITY;
    const float mx = group4_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    const float m_new = fmaxf(m, mx);
    if (__any(m_new > m + kDecRescaleThreshold)) {
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][r] *= alpha;
      m = m_new;
    }
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(sv[r] - m);
    l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const s16x4 pb = __builtin_bit_cast(s16x4, (bf16x4_t){(__bf16)pr[0], (__bf16)pr[1],
                                                          (__bf16)pr[2], (__bf16)pr[3]});
    // O^T += V^T P^T over the 16 keys of the tile.
#pragma unroll
    for (int db = 0; db < S::NDB; ++db) {
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vt + voff + 32 * (db ^ vx)));
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[db], 0, 0, 0);
    }
  };

  bf16x8 kf0[S::KSTEPS], kf1[S::KSTEPS];
  if (my > 0) issue(0, kf0, v0);
  if (my > 1) issue(1, kf1, v1);
  for (int i = 0; i < my; i += 2) {
    process(i, kf0, v0);
    if (i + 2 < my) issue(i + 2, kf0, v0);
    if (i + 1 < my) {
      process(i + 1, kf1, v1);
      if (i + 3 < my) issue(i + 3, kf1, v1);
    }
  }

  // Merge the four waves' states through LDS: lane (grp, col) owns O^T rows
  // 16db + 4grp + r of query col.  The accumulator rows are padded by 4
  // floats, so the 16 columns of one 16-byte write land 4 banks apart (with
  // rows of exactly D floats they all hit the same 4 banks).
  const float lt = group4_sum(l);
  constexpr int AR = D + 4;                      // floats per accumulator row
  float* sm_m = mlds;                            // [4][16]
  float* sm_l = sm_m + kDecWaves * 16;           // [4][16]
  float* sm_acc = sm_l + kDecWaves * 16;         // [4][16][AR]
  if (grp == 0) {
    sm_m[wave * 16 + col] = m;
    sm_l[wave * 16 + col] = lt;
  }
#pragma unroll
  for (int db = 0; db < S::NDB; ++db)
    *reinterpret_cast<float4*>(sm_acc + ((size_t)wave * 16 + col) * AR + 16 * db + 4 * grp) =
        make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
  __syncthreads();

  for (int o = tid; o < cols * D; o += kDecThreads) {
    const int gq = o / D, dd = o % D;
    const int gh = SERVE ? gq / nq : gq;
    const int gr = SERVE ? gq - gh * nq : 0;
    float M = -1e30f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = max_raw(M, sm_m[w * 16 + gq]);
    float W = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(sm_m[w * 16 + gq] - M);
      W += wt * sm_l[w * 16 + gq];
      O += wt * sm_acc[((size_t)w * 16 + gq) * AR + dd];
    }
    const size_t ps = ((size_t)(b * p.Hq + h0 + gh) * nq + gr) * p.splits + s;
    if (W > 0.f) {
      p.o_part[ps * D + dd] = O / W;
      if (dd == 0) p.lse_part[ps] = (M + log2f(W)) * kLn2;
    } else {   // empty chunk: weight 0 in the merge
      p.o_part[ps * D + dd] = 0.f;
      if (dd == 0) p.lse_part[ps] = -INFINITY;
    }
  }
}

// Merge: one workgroup of kMergeThreads per (b, query head).  Thread t owns
// output column t % D and the splits s = t / D, t / D + SP, ...; it loads
// their LSEs and partial outputs in batches of kMergeBatch independent
// loads.  The first batch is issued before the maximum LSE is known: every
// wave finds that maximum itself (strided loads and a shuffle reduction), so
// the partial outputs cost no second round trip.  The SP partial sums per
// column are then added through LDS in a fixed order.
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 8;

template <int D>
__device__ __forceinline__ void decode_merge_body(const DecodeParams& p) {
  constexpr int SP = kMergeThreads / D;       // split phases per column
  constexpr int U = kMergeBatch;
  __shared__ float red[kMergeThreads];
  __shared__ float part[kMergeThreads];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int S = p.splits;
  const float* lp = p.lse_part + (size_t)bh * S;
  const float* op = p.o_part + (size_t)bh * S * D;
  const int dd = tid % D, ph = tid / D;

  float ls[U], ov[U];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * SP;
      ls[u] = s < S ? lp[s] : -INFINITY;
      ov[u] = s < S ? op[(size_t)s * D + dd] : 0.f;
    }
  };
  load_batch(ph);

  float M = -INFINITY;
  for (int s = tid & 63; s < S; s += 64) M = max_raw(M, lp[s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = max_raw(M, __shfl_xor(M, off));
  // M is finite unless every chunk of the row is empty (Wt = 0 below).

  float O = 0.f, W = 0.f;
  for (int s0 = ph;;) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = ls[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((ls[u] - M) * kLog2e);
      W += w;
      O += w * ov[u];
    }
    s0 += U * SP;
    if (s0 >= S) break;
    load_batch(s0);
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
    // A row with no allowed key at all (only possible in the serving form)
    // gets O = 0 and LSE = -inf.
    bf16x2 v = {(__bf16)(Wt > 0.f ? Ot / Wt : 0.f), (__bf16)0.f};
    p.o[(size_t)bh * D + dd] = __builtin_bit_cast(unsigned, v) & 0xFFFFu;
    if (dd == 0) p.lse[bh] = Wt > 0.f ? M + logf(Wt) : -INFINITY;
  }
}

}  // namespace
}  // namespace fa

#define FA_DEC_SPLIT_K(NAME, D, GT, SERVE)                                               \
  extern "C" __global__ void __launch_bounds__(fa::kDecThreads, 2) NAME(fa::DecodeParams p) { \
    __shared__ __attribute__((aligned(1024))) char vs0[fa::kDecWaves * fa::DecShape<D>::VTILE]; \
    __shared__ __attribute__((aligned(1024))) char vs1[fa::kDecWaves * fa::DecShape<D>::VTILE]; \
    __shared__ __attribute__((aligned(16))) float mlds[fa::kDecWaves * 16 * (2 + D + 4)]; \
    fa::decode_split_body<D, GT, SERVE>(p, (fa::lds_char*)vs0, (fa::lds_char*)vs1, mlds); \
  }
#define FA_DEC_SPLIT(D, GT)                                          \
  FA_DEC_SPLIT_K(fa_decode_split_d##D##_g##GT, D, GT, false)         \
  FA_DEC_SPLIT_K(fa_decode_serve_split_d##D##_g##GT, D, GT, true)

#define FA_DEC_MERGE(D)                                                               \
  extern "C" __global__ void __launch_bounds__(fa::kMergeThreads) fa_decode_merge_d##D( \
      fa::DecodeParams p) {                                                           \
    fa::decode_merge_body<D>(p);                                                      \
  }

#define FA_DEC_ALL(D)                                                                  \
  FA_DEC_SPLIT(D, 1) FA_DEC_SPLIT(D, 2) FA_DEC_SPLIT(D, 4) FA_DEC_SPLIT(D, 8)          \
  FA_DEC_SPLIT(D, 16) FA_DEC_MERGE(D)

FA_DEC_ALL(32)
FA_DEC_ALL(64)
FA_DEC_ALL(128)
FA_DEC_ALL(256)

namespace fa {

int decode_group_tile(int group) {
  if (group % 16 == 0) return 16;
  if (group % 8 == 0) return 8;
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

int decode_serve_group_tile(int group, int nq) {
  for (int gt = 16; gt > 1; gt >>= 1)
    if (group % gt == 0 && gt * nq <= 16) return gt;
  return 1;
}

namespace {

const void* split_fn(int d, int gt, bool serve) {
#define FA_CASE(D)                                                                            \
  case D:                                                                                     \
    switch (gt) {                                                                             \
      case 1: return serve ? (const void*)fa_decode_serve_split_d##D##_g1                     \
                           : (const void*)fa_decode_split_d##D##_g1;                          \
      case 2: return serve ? (const void*)fa_decode_serve_split_d##D##_g2                     \
                           : (const void*)fa_decode_split_d##D##_g2;                          \
      case 4: return serve ? (const void*)fa_decode_serve_split_d##D##_g4                     \
                           : (const void*)fa_decode_split_d##D##_g4;                          \
      case 8: return serve ? (const void*)fa_decode_serve_split_d##D##_g8                     \
                           : (const void*)fa_decode_split_d##D##_g8;                          \
      case 16: return serve ? (const void*)fa_decode_serve_split_d##D##_g16                   \
                            : (const void*)fa_decode_split_d##D##_g16;                        \
    }                                                                                         \
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
  static const char* const split_names[4][5] = {
      {"fa_decode_split_d32_g1", "fa_decode_split_d32_g2", "fa_decode_split_d32_g4",
       "fa_decode_split_d32_g8", "fa_decode_split_d32_g16"},
      {"fa_decode_split_d64_g1", "fa_decode_split_d64_g2", "fa_decode_split_d64_g4",
       "fa_decode_split_d64_g8", "fa_decode_split_d64_g16"},
      {"fa_decode_split_d128_g1", "fa_decode_split_d128_g2", "fa_decode_split_d128_g4",
       "fa_decode_split_d128_g8", "fa_decode_split_d128_g16"},
      {"fa_decode_split_d256_g1", "fa_decode_split_d256_g2", "fa_decode_split_d256_g4",
       "fa_decode_split_d256_g8", "fa_decode_split_d256_g16"}};
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
  const int gi = gt == 1 ? 0 : gt == 2 ? 1 : gt == 4 ? 2 : gt == 8 ? 3 : 4;
  return split_names[di][gi];
}

const char* decode_serve_kernel_name(int d, int group, int nq) {
  static const char* const names[4][5] = {
      {"fa_decode_serve_split_d32_g1", "fa_decode_serve_split_d32_g2",
       "fa_decode_serve_split_d32_g4", "fa_decode_serve_split_d32_g8",
       "fa_decode_serve_split_d32_g16"},
      {"fa_decode_serve_split_d64_g1", "fa_decode_serve_split_d64_g2",
       "fa_decode_serve_split_d64_g4", "fa_decode_serve_split_d64_g8",
       "fa_decode_serve_split_d64_g16"},
      {"fa_decode_serve_split_d128_g1", "fa_decode_serve_split_d128_g2",
       "fa_decode_serve_split_d128_g4", "fa_decode_serve_split_d128_g8",
       "fa_decode_serve_split_d128_g16"},
      {"fa_decode_serve_split_d256_g1", "fa_decode_serve_split_d256_g2",
       "fa_decode_serve_split_d256_g4", "fa_decode_serve_split_d256_g8",
       "fa_decode_serve_split_d256_g16"}};
  const int di = d == 32 ? 0 : d == 64 ? 1 : d == 128 ? 2 : d == 256 ? 3 : -1;
  if (di < 0 || group <= 0 || nq < 1 || nq > 16) return nullptr;
  const int gt = decode_serve_group_tile(group, nq);
  const int gi = gt == 1 ? 0 : gt == 2 ? 1 : gt == 4 ? 2 : gt == 8 ? 3 : 4;
  return names[di][gi];
}

hipError_t launch_decode_serve(const DecodeParams& p, int d, hipStream_t s) {
  const int gt = decode_serve_group_tile(p.group, p.nq);
  const void* f1 = split_fn(d, gt, true);
  const void* f2 = merge_fn(d);
  if (!f1 || !f2) return hipErrorInvalidValue;
  DecodeParams arg = p;
  void* args[] = {&arg};
  const unsigned n1 = (unsigned)(p.B * p.Hkv * p.splits * (p.group / gt));
  hipError_t e = hipLaunchKernel(f1, dim3(n1), dim3(kDecThreads), args, 0, s);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(f2, dim3((unsigned)(p.B * p.Hq * p.nq)), dim3(kMergeThreads), args, 0, s);
}

hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t s) {
  const int gt = decode_group_tile(p.group);
  const void* f1 = split_fn(d, gt, false);
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
