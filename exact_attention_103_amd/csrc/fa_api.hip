// C-ABI layer of libfa.so: argument validation, dispatch and error text.
// Every check runs on the host before the first HIP call, so an invalid call
// enqueues nothing and writes nothing (the declarations in include/fa.h give
// the full contract).

#include "fa.h"
#include "fa_internal.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

namespace {

thread_local char g_hip_error[256] = "";

int hip_fail(hipError_t e) {
  snprintf(g_hip_error, sizeof(g_hip_error), "%s: %s", hipGetErrorName(e),
           hipGetErrorString(e));
  return FA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_d(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

// Product of positive factors, or -1 when it exceeds 2^62.
int64_t checked_product(std::initializer_list<int64_t> xs) {
  const int64_t lim = int64_t(1) << 62;
  int64_t r = 1;
  for (int64_t x : xs) {
    if (x <= 0) return -1;
    if (r > lim / x) return -1;
    r *= x;
  }
  return r;
}

struct Span {
  uintptr_t lo, hi;
};

Span span(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + static_cast<uintptr_t>(bytes)};
}

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

int max_splits(int Nk) { return Nk <= 0 ? 0 : (Nk + fa::kDecodeChunkAlign - 1) / fa::kDecodeChunkAlign; }

int split_chunk(int Nk, int S) {
  const int c = (Nk + S - 1) / S;
  return (c + fa::kDecodeChunkAlign - 1) / fa::kDecodeChunkAlign * fa::kDecodeChunkAlign;
}

// Shared by fa_fwd_fp8 (descales as values) and fa_fwd_fp8_devscale
// (descales in device memory: qdp, kdp, vdp non-null, value factors 1).
int fwd_fp8_common(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, float q_descale,
                   float k_descale, float v_descale, const float* qdp, const float* kdp,
                   const float* vdp, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (causal && Nq > Nk) return FA_ERR_SHAPE;
  if (!supported_d(d)) return FA_ERR_HEAD_DIM;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  for (const float* dp : {qdp, kdp, vdp})
    if (dp && (reinterpret_cast<uintptr_t>(dp) & 3u) != 0) return FA_ERR_ALIGN;
  const int64_t q_bytes = checked_product({B, Hq, Nq, d});
  const int64_t kv_bytes = checked_product({B, Hkv, Nk, d});
  const int64_t o_bytes = checked_product({B, Hq, Nq, d, 2});
  const int64_t lse_bytes = checked_product({B, Hq, Nq, 4});
  const int bm = fa::fwd_fp8_rows_per_block(d);
  const int64_t grid = checked_product({(Nq + bm - 1) / bm, B, Hq});
  if (q_bytes < 0 || kv_bytes < 0 || o_bytes < 0 || lse_bytes < 0 || grid < 0 ||
      grid > INT32_MAX)
    return FA_ERR_TOO_LARGE;
  const Span ins[6] = {span(q, q_bytes), span(k, kv_bytes), span(v, kv_bytes),
                       qdp ? span(qdp, 4) : Span{0, 0}, kdp ? span(kdp, 4) : Span{0, 0},
                       vdp ? span(vdp, 4) : Span{0, 0}};
  const Span so = span(o, o_bytes), sl = span(lse, lse_bytes);
  for (const Span& in : ins)
    if (overlaps(so, in) || overlaps(sl, in)) return FA_ERR_ALIAS;
  if (overlaps(so, sl)) return FA_ERR_ALIAS;

  fa::FwdF8Params p;
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.group = Hq / Hkv;
  // Same association as the kernel's (scale * log2 e) * q_ds * k_ds, so that
  // value and device descales give identical results.
  p.c = scale * fa::kLog2e * q_descale * k_descale;
  p.v_descale = v_descale;
  p.q_ds = qdp;
  p.k_ds = kdp;
  p.v_ds = vdp;
  if (!isfinite(p.c) || !(p.c > 0.f)) return FA_ERR_SCALE;
  const hipError_t e = fa::launch_fwd_fp8(p, d, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

}  // namespace

// Shared with the allocation-free decode (fa_noalloc.hip).
namespace fa {

int decode_check(const void* q, const void* k_cache, const void* v_cache, const void* o,
                 const float* lse, int B, int Hq, int Hkv, int Nk, int d, float scale,
                 int num_splits, int* splits) {
  if (!q || !k_cache || !v_cache || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nk <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (!supported_d(d)) return FA_ERR_HEAD_DIM;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  if (num_splits < 0 || num_splits > max_splits(Nk)) return FA_ERR_SPLITS;
  const int S = num_splits == 0 ? fa_decode_num_splits(B, Hq, Hkv, Nk, d) : num_splits;
  if (S < 0) return S;
  if (fa_decode_workspace_size(B, Hq, d, S) == 0) return FA_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      !aligned16(lse))
    return FA_ERR_ALIGN;

  const int group = Hq / Hkv;
  const int64_t q_bytes = checked_product({B, Hq, d, 2});
  const int64_t kv_bytes = checked_product({B, Hkv, Nk, d, 2});
  const int64_t lse_bytes = checked_product({B, Hq, 4});
  const int64_t grid = checked_product({B, Hkv, S, group / decode_group_tile(group)});
  if (q_bytes < 0 || kv_bytes < 0 || lse_bytes < 0 || grid < 0 || grid > INT32_MAX)
    return FA_ERR_TOO_LARGE;

  const Span sq = span(q, q_bytes), sk = span(k_cache, kv_bytes), sv = span(v_cache, kv_bytes);
  const Span so = span(o, q_bytes), sl = span(lse, lse_bytes);
  const Span ins[3] = {sq, sk, sv};
  for (const Span& in : ins)
    if (overlaps(so, in) || overlaps(sl, in)) return FA_ERR_ALIAS;
  if (overlaps(so, sl)) return FA_ERR_ALIAS;
  *splits = S;
  return FA_OK;
}

int hip_status(hipError_t e) { return hip_fail(e); }

}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
           int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (causal && Nq > Nk) return FA_ERR_SHAPE;
  if (!supported_d(d)) return FA_ERR_HEAD_DIM;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;

  const int64_t q_bytes = checked_product({B, Hq, Nq, d, 2});
  const int64_t kv_bytes = checked_product({B, Hkv, Nk, d, 2});
  const int64_t lse_bytes = checked_product({B, Hq, Nq, 4});
  const fa::FwdTile t = fa::fwd_tile(d, causal != 0, Nq, Nk);
  const int64_t grid = checked_product({(Nq + t.bm - 1) / t.bm, B, Hq});
  if (q_bytes < 0 || kv_bytes < 0 || lse_bytes < 0 || grid < 0 || grid > INT32_MAX)
    return FA_ERR_TOO_LARGE;

  const Span sq = span(q, q_bytes), sk = span(k, kv_bytes), sv = span(v, kv_bytes);
  const Span so = span(o, q_bytes), sl = span(lse, lse_bytes);
  if (overlaps(so, sq) || overlaps(so, sk) || overlaps(so, sv) || overlaps(sl, sq) ||
      overlaps(sl, sk) || overlaps(sl, sv) || overlaps(so, sl))
    return FA_ERR_ALIAS;

  fa::FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.group = Hq / Hkv;
  p.c = scale * fa::kLog2e;
  const hipError_t e = fa::launch_fwd(p, d, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B,
               int Hq, int Hkv, int Nq, int Nk, int d, float scale, float q_descale,
               float k_descale, float v_descale, int causal, void* stream) {
  if (!scale_ok(q_descale) || !scale_ok(k_descale) || !scale_ok(v_descale)) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    return FA_ERR_SCALE;
  }
  return fwd_fp8_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, q_descale, k_descale,
                        v_descale, nullptr, nullptr, nullptr, causal, stream);
}

int fa_fwd_fp8_devscale(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                        const float* q_descale, const float* k_descale,
                        const float* v_descale, int causal, void* stream) {
  if (!q_descale || !k_descale || !v_descale) return FA_ERR_NULL;
  return fwd_fp8_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, 1.f, 1.f, 1.f, q_descale,
                        k_descale, v_descale, causal, stream);
}

size_t fa_fp8_quantize_workspace_size(int rows, int d) {
  if (rows <= 0 || !supported_d(d)) return 0;
  return 4 * (size_t)fa::quant_blocks(rows, d);
}

int fa_fp8_quantize(const void* x, void* codes, float* descale, const void* signs, int rows,
                    int d, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !codes || !descale) return FA_ERR_NULL;
  if (rows <= 0) return FA_ERR_SHAPE;
  if (!supported_d(d)) return FA_ERR_HEAD_DIM;
  if (!aligned16(x) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(descale) & 3u) != 0)
    return FA_ERR_ALIGN;
  const int64_t x_bytes = checked_product({rows, d, 2});
  const int64_t c_bytes = checked_product({rows, d});
  if (x_bytes < 0 || c_bytes < 0) return FA_ERR_TOO_LARGE;
  const size_t need = fa_fp8_quantize_workspace_size(rows, d);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  const Span sx = span(x, x_bytes), sc = span(codes, c_bytes), sd = span(descale, 4);
  const Span sw = span(workspace, static_cast<int64_t>(need));
  const Span ss = signs ? span(signs, d) : Span{0, 0};
  const Span outs[3] = {sc, sd, sw};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], sx) || overlaps(outs[i], ss)) return FA_ERR_ALIAS;
    for (int k2 = i + 1; k2 < 3; ++k2)
      if (overlaps(outs[i], outs[k2])) return FA_ERR_ALIAS;
  }

  fa::QuantParams p;
  p.x = static_cast<const uint16_t*>(x);
  p.signs = static_cast<const int8_t*>(signs);
  p.codes = static_cast<uint8_t*>(codes);
  p.descale = descale;
  p.partial = static_cast<float*>(workspace);
  p.rows = rows;
  p.nblocks = fa::quant_blocks(rows, d);
  p.norm = signs ? sqrtf(static_cast<float>(d)) : 1.0f;
  const hipError_t e = fa::launch_quant(p, d, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

const char* fa_fp8_quantize_kernel_name(int d, int stage) {
  if (stage != 0 && stage != 1) return nullptr;
  return fa::quant_kernel_name(d, stage);
}

const char* fa_fwd_fp8_kernel_name(int d, int causal) {
  if (causal != 0 && causal != 1) return nullptr;
  return fa::fwd_fp8_kernel_name(d, causal != 0);
}

int fa_decode_max_splits(int Nk) { return max_splits(Nk); }

size_t fa_decode_workspace_size(int B, int Hq, int d, int num_splits) {
  if (!supported_d(d)) return 0;
  const int64_t n = checked_product({B, Hq, num_splits, d + 1, 4});
  return n < 0 ? 0 : static_cast<size_t>(n);
}

int fa_decode_num_splits(int B, int Hq, int Hkv, int Nk, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nk <= 0 || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (!supported_d(d)) return FA_ERR_HEAD_DIM;
  const int group = Hq / Hkv;
  const int64_t per_split = checked_product({B, Hkv, group / fa::decode_group_tile(group)});
  if (per_split < 0) return FA_ERR_TOO_LARGE;
  // About 1024 workgroups (4 per CU on 256 CUs), chunks of >= 256 keys.
  int64_t s = (1024 + per_split - 1) / per_split;
  const int64_t by_len = Nk / 256 > 0 ? Nk / 256 : 1;
  if (s > by_len) s = by_len;
  if (s > max_splits(Nk)) s = max_splits(Nk);
  if (s < 1) s = 1;
  return static_cast<int>(s);
}


int fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache, void* o,
                      float* lse, int B, int Hq, int Hkv, int Nk, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  int S = 0;
  const int rc = fa::decode_check(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nk, d, scale,
                                  num_splits, &S);
  if (rc != FA_OK) return rc;
  const size_t need = fa_decode_workspace_size(B, Hq, d, S);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  const int64_t q_bytes = static_cast<int64_t>(B) * Hq * d * 2;
  const int64_t kv_bytes = static_cast<int64_t>(B) * Hkv * Nk * d * 2;
  const Span sw = span(workspace, static_cast<int64_t>(need));
  const Span others[5] = {span(q, q_bytes), span(k_cache, kv_bytes), span(v_cache, kv_bytes),
                          span(o, q_bytes), span(lse, static_cast<int64_t>(B) * Hq * 4)};
  for (const Span& t : others)
    if (overlaps(sw, t)) return FA_ERR_ALIAS;

  fa::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.o_part = static_cast<float*>(workspace);
  p.lse_part = p.o_part + static_cast<size_t>(B) * Hq * S * d;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nk = Nk;
  p.group = Hq / Hkv;
  p.splits = S;
  p.chunk = split_chunk(Nk, S);
  p.c = scale * fa::kLog2e;
  p.seqlens = nullptr;
  p.nq = 1;
  p.causal = 0;
  const hipError_t e = fa::launch_decode(p, d, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

size_t fa_decode_serve_workspace_size(int B, int Hq, int Nq, int d, int num_splits) {
  if (!supported_d(d) || Nq < 1 || Nq > 16) return 0;
  const int64_t n = checked_product({B, Hq, Nq, num_splits, d + 1, 4});
  return n < 0 ? 0 : static_cast<size_t>(n);
}

int fa_decode_serve_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nk <= 0 || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (Nq < 1 || Nq > 16) return FA_ERR_SHAPE;
  if (!supported_d(d)) return FA_ERR_HEAD_DIM;
  const int group = Hq / Hkv;
  const int64_t per_split =
      checked_product({B, Hkv, group / fa::decode_serve_group_tile(group, Nq)});
  if (per_split < 0) return FA_ERR_TOO_LARGE;
  int64_t s = (1024 + per_split - 1) / per_split;
  const int64_t by_len = Nk / 256 > 0 ? Nk / 256 : 1;
  if (s > by_len) s = by_len;
  if (s > max_splits(Nk)) s = max_splits(Nk);
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

int fa_decode_serve(const void* q, const void* k_cache, const void* v_cache, const int* seqlens,
                    void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                    float scale, int causal, int num_splits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nk <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0 || Nq < 1 || Nq > 16) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!supported_d(d)) return FA_ERR_HEAD_DIM;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  if (num_splits < 0 || num_splits > max_splits(Nk)) return FA_ERR_SPLITS;
  const int S = num_splits == 0 ? fa_decode_serve_num_splits(B, Hq, Hkv, Nq, Nk, d) : num_splits;
  if (S < 0) return S;
  const size_t need = fa_decode_serve_workspace_size(B, Hq, Nq, d, S);
  if (need == 0) return FA_ERR_TOO_LARGE;
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      !aligned16(lse) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0)
    return FA_ERR_ALIGN;

  const int group = Hq / Hkv;
  const int64_t q_bytes = checked_product({B, Hq, Nq, d, 2});
  const int64_t kv_bytes = checked_product({B, Hkv, Nk, d, 2});
  const int64_t lse_bytes = checked_product({B, Hq, Nq, 4});
  const int64_t grid = checked_product({B, Hkv, S, group / fa::decode_serve_group_tile(group, Nq)});
  const int64_t grid2 = checked_product({B, Hq, Nq});
  if (q_bytes < 0 || kv_bytes < 0 || lse_bytes < 0 || grid < 0 || grid > INT32_MAX ||
      grid2 < 0 || grid2 > INT32_MAX)
    return FA_ERR_TOO_LARGE;

  const Span ins[4] = {span(q, q_bytes), span(k_cache, kv_bytes), span(v_cache, kv_bytes),
                       span(seqlens, seqlens ? static_cast<int64_t>(B) * 4 : 0)};
  const Span outs[3] = {span(o, q_bytes), span(lse, lse_bytes),
                        span(workspace, static_cast<int64_t>(need))};
  for (int i = 0; i < 3; ++i) {
    for (const Span& in : ins)
      if (overlaps(outs[i], in)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outs[j])) return FA_ERR_ALIAS;
  }

  fa::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_cache);
  p.v = static_cast<const uint16_t*>(v_cache);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.o_part = static_cast<float*>(workspace);
  p.lse_part = p.o_part + static_cast<size_t>(B) * Hq * Nq * S * d;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nk = Nk;
  p.group = group;
  p.splits = S;
  p.chunk = split_chunk(Nk, S);
  p.c = scale * fa::kLog2e;
  p.seqlens = seqlens;
  p.nq = Nq;
  p.causal = causal;
  const hipError_t e = fa::launch_decode_serve(p, d, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

size_t fa_bwd_workspace_size(int B, int Hq, int Nq) {
  const int64_t n = checked_product({B, Hq, Nq, 4});
  return n < 0 ? 0 : static_cast<size_t>(n);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
           int Nk, int d, float scale, int causal, void* workspace, size_t workspace_bytes,
           void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (causal && Nq > Nk) return FA_ERR_SHAPE;
  if (!fa::bwd_supported_d(d)) return FA_ERR_HEAD_DIM;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  const size_t need = fa_bwd_workspace_size(B, Hq, Nq);
  if (need == 0) return FA_ERR_TOO_LARGE;
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(workspace))
    return FA_ERR_ALIGN;

  const int64_t q_bytes = checked_product({B, Hq, Nq, d, 2});
  const int64_t kv_bytes = checked_product({B, Hkv, Nk, d, 2});
  const int64_t lse_bytes = checked_product({B, Hq, Nq, 4});
  const int64_t g1 = checked_product({(Nq + 127) / 128, B, Hq});
  const int64_t g2 = checked_product({(Nk + 63) / 64, B, Hkv});
  if (q_bytes < 0 || kv_bytes < 0 || lse_bytes < 0 || g1 < 0 || g1 > INT32_MAX || g2 < 0 ||
      g2 > INT32_MAX)
    return FA_ERR_TOO_LARGE;

  const Span ins[6] = {span(q, q_bytes), span(k, kv_bytes), span(v, kv_bytes),
                       span(o, q_bytes), span(dout, q_bytes), span(lse, lse_bytes)};
  const Span outs[4] = {span(dq, q_bytes), span(dk, kv_bytes), span(dv, kv_bytes),
                        span(workspace, static_cast<int64_t>(need))};
  for (int i = 0; i < 4; ++i) {
    for (const Span& in : ins)
      if (overlaps(outs[i], in)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return FA_ERR_ALIAS;
  }

  fa::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.delta = static_cast<float*>(workspace);
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.group = Hq / Hkv;
  p.c = scale * fa::kLog2e;
  p.scale = scale;
  const hipError_t e = fa::launch_bwd(p, d, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : hip_fail(e);
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape (sizes must be > 0, Hq a multiple of Hkv, causal needs Nq <= Nk)";
    case FA_ERR_HEAD_DIM: return "unsupported head dimension (32, 64, 128 or 256)";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "workspace is NULL or too small";
    case FA_ERR_SPLITS: return "num_splits out of range";
    case FA_ERR_HIP: return "HIP launch failed";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_TOO_LARGE: return "sizes exceed the supported range";
    case FA_ERR_SCRATCH: return "the split partials exceed the fixed scratch of the allocation-free decode";
    default: return "unknown status";
  }
}

const char* fa_last_hip_error(void) { return g_hip_error; }

int fa_build_is_serial(void) {
#ifdef FA_SERIAL_PIPELINE
  return 1;
#else
  return 0;
#endif
}

const char* fa_fwd_kernel_name(int d, int causal, int Nq, int Nk) {
  if (causal != 0 && causal != 1) return nullptr;
  if (Nq <= 0 || Nk <= 0) return nullptr;
  return fa::fwd_kernel_name(d, causal != 0, Nq, Nk);
}

const char* fa_decode_kernel_name(int d, int hq_per_kv, int stage) {
  return fa::decode_kernel_name(d, hq_per_kv, stage);
}

const char* fa_decode_serve_kernel_name(int d, int hq_per_kv, int Nq, int stage) {
  if (stage == 1) return fa::decode_kernel_name(d, hq_per_kv, 1);
  if (stage != 0) return nullptr;
  return fa::decode_serve_kernel_name(d, hq_per_kv, Nq);
}

const char* fa_bwd_kernel_name(int d, int causal, int stage) {
  if (causal != 0 && causal != 1) return nullptr;
  return fa::bwd_kernel_name(d, causal != 0, stage);
}

}  // extern "C"
