// Internal declarations shared by the kernels and the C-ABI layer of libfa.so.
// Everything here is device-side plumbing for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy operand of __builtin_amdgcn_global_load_lds for a
// nontemporal (streaming) load: the `nt` bit of gfx950's global loads.
constexpr int kCachePolicyNT = 2;

// Race-check build (compiled with -DFA_SERIAL_PIPELINE into a second
// library).  Around every staged copy into LDS, FA_STAGE_FENCE waits for all
// of the wave's outstanding memory operations and then for every wave of the
// workgroup, on both sides of the copy; FA_STAGE_WAIT does the same for
// copies into a wave's own LDS buffers, without the workgroup barrier.  No
// copy then overlaps a read of the buffer it targets, nor any compute.  The
// arithmetic and its order do not change, so that build must reproduce the
// pipelined one bit for bit: a difference is a race between a staged copy
// and the reads of its buffer.  FA_STAGE_FENCE is only placed where every
// wave of the workgroup arrives.
#ifdef FA_SERIAL_PIPELINE
#define FA_STAGE_FENCE()                 \
  do {                                   \
    __builtin_amdgcn_s_waitcnt(0);       \
    __syncthreads();                     \
  } while (0)
#define FA_STAGE_WAIT() __builtin_amdgcn_s_waitcnt(0)
#else
#define FA_STAGE_FENCE() \
  do {                   \
  } while (0)
#define FA_STAGE_WAIT() \
  do {                  \
  } while (0)
#endif

// Step barrier of kernels that issue their LDS copies two steps ahead: the
// wave waits until at most N of its vector-memory operations are in flight
// (the copies it issued in this step, which may land later) and its LDS
// operations are done, then every wave of the workgroup meets.  A plain
// __syncthreads would also wait for this step's copies.  The signal fences
// keep the compiler from moving memory operations across the barrier.  The
// immediate is gfx9's s_waitcnt encoding: vmcnt in bits 3:0 and 15:14,
// expcnt (7: no wait) in bits 6:4, lgkmcnt (0) in bits 11:8.
template <int N>
__device__ __forceinline__ void wait_copies_in_flight() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
template <int N>
__device__ __forceinline__ void copies_in_flight_barrier() {
  wait_copies_in_flight<N>();
  step_barrier();
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Arguments of one forward launch.  Tensors are [B][H][N][d] bf16 (raw
// 16-bit words), LSE fp32.  c = scale * log2(e): scores are kept in base-2
// units so that the exponential is a single v_exp_f32.
struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk;
  int group;     // Hq / Hkv
  float c;       // scale * log2(e)
};

// Arguments of one fp8 forward launch: q, k, v are OCP fp8 e4m3 bytes
// [B][H][N][d] (real value = byte value * its descale factor); o bf16, lse
// fp32.  c = scale * q_descale * k_descale * log2(e).
struct FwdF8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk;
  int group;
  float c;           // scale * q_descale * k_descale * log2(e), or scale * log2(e)
  float v_descale;   //   when the descales come from device memory (q_ds != null)
  const float* q_ds;
  const float* k_ds;
  const float* v_ds;
};

// Arguments of one fp8 quantisation (two launches over the same rows).
// signs: ±1 per head-dim channel (int8, negative = -1) or null for no
// rotation; partial: one float per workgroup of the first launch; norm:
// sqrt(d) with rotation, else 1 (divides the reported descale).
struct QuantParams {
  const uint16_t* x;
  const int8_t* signs;
  uint8_t* codes;
  float* descale;
  float* partial;
  int rows;
  int nblocks;
  float norm;
};

// Arguments of one split-KV decode (split kernel + merge kernel).
struct DecodeParams {
  const uint16_t* q;      // [B][Hq][d]
  const uint16_t* k;      // [B][Hkv][Nk][d]
  const uint16_t* v;
  uint16_t* o;            // [B][Hq][d]
  float* lse;             // [B][Hq]
  float* o_part;          // [B][Hq][S][d]   chunk-normalised partial outputs
  float* lse_part;        // [B][Hq][S]      chunk LSE (natural log), -inf if empty
  int B, Hq, Hkv, Nk;
  int group;              // Hq / Hkv
  int splits;             // S
  int chunk;              // keys per split (multiple of 64); per sequence when serving
  float c;                // scale * log2(e)
  // Serving-shaped decode only (fa_decode_serve): Nq query rows per
  // sequence (q, o, lse, o_part, lse_part gain an [Nq] axis after the head),
  // per-sequence key counts seqlens[b] <= Nk (Nk = cache capacity; NULL = all
  // Nk), and bottom-right causal masking among the Nq rows.
  const int* seqlens;
  int nq;
  int causal;
};

// Arguments of one backward call (dQ kernel, then dK/dV kernel).  Tensors
// are [B][H][N][d] bf16; lse and delta are [B][Hq][Nq] fp32.
struct BwdParams {
  const uint16_t* q;      // [B][Hq][Nq][d]
  const uint16_t* k;      // [B][Hkv][Nk][d]
  const uint16_t* v;
  const uint16_t* o;      // forward output
  const uint16_t* dout;   // gradient of the loss with respect to o
  const float* lse;       // forward LSE, natural log
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;           // rowsum(dout * o): written by the dQ kernel, read by dK/dV
  int B, Hq, Hkv, Nq, Nk;
  int group;              // Hq / Hkv
  float c;                // scale * log2(e)
  float scale;
};

// Host-side launchers (defined next to their kernels).  They assume the
// arguments were validated and return the hipError_t of the launch.
hipError_t launch_fwd(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t s);
hipError_t launch_decode_serve(const DecodeParams& p, int d, hipStream_t s);
const char* decode_serve_kernel_name(int d, int group, int nq);
int decode_serve_group_tile(int group, int nq);
const char* fwd_kernel_name(int d, bool causal, int Nq, int Nk);
const char* decode_kernel_name(int d, int group, int stage);
hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_fwd_fp8(const FwdF8Params& p, int d, bool causal, hipStream_t s);
int quant_blocks(int rows, int d);
const char* quant_kernel_name(int d, int stage);
hipError_t launch_quant(const QuantParams& p, int d, hipStream_t s);
const char* fwd_fp8_kernel_name(int d, bool causal);
int fwd_fp8_rows_per_block(int d);
const char* bwd_kernel_name(int d, bool causal, int stage);
bool bwd_supported_d(int d);
int bwd_dq_grid_blocks(int B, int Hq, int Nq);
int bwd_dkdv_grid_blocks(int B, int Hkv, int Nk);

// Tile shape of the forward kernel that runs for a problem (BM query rows
// per workgroup, BN keys per tile, waves per workgroup).
struct FwdTile { int bm, bn, waves; };
FwdTile fwd_tile(int d, bool causal, int Nq, int Nk);

// Query heads handled by one decode split workgroup: the largest of 16, 8,
// 4, 2, 1 that divides the number of query heads per KV head.
int decode_group_tile(int group);

// Keys per decode split are rounded up to this multiple.
constexpr int kDecodeChunkAlign = 64;

// Every check fa_decode_splitkv makes except those on the workspace (nulls,
// shapes, head dim, scale, split range, alignment, size limits, overlaps
// among the tensors), with no HIP call; on FA_OK *splits is the split count
// after the 0 -> heuristic substitution.
int decode_check(const void* q, const void* k_cache, const void* v_cache, const void* o,
                 const float* lse, int B, int Hq, int Hkv, int Nk, int d, float scale,
                 int num_splits, int* splits);

// Records the text of a HIP error for fa_last_hip_error and returns
// FA_ERR_HIP.
int hip_status(hipError_t e);

}  // namespace fa
