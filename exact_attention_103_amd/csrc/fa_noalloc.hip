// Allocation-free split-KV decode: fa_decode_splitkv with its partial
// outputs and partial LSEs in a fixed device array of this library instead
// of a caller workspace, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops).
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, from module load until the
// process ends.  In host code the name `scratch` is only a host-side
// stand-in, so the device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever handed to a kernel.

#include "fa.h"
#include "fa_internal.h"

#include <mutex>

namespace {

static_assert(FA_DECODE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[FA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};

DeviceScratch g_scratch[kMaxDevices];

// Device address of the current device's copy of `scratch` (looked up on
// the first call per device), or the HIP error of that lookup.  A stream of
// another device is refused: its kernels would reach this array through
// another GPU's address.
hipError_t device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (stream != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != dev) return hipErrorInvalidDevice;
  }
  DeviceScratch& s = g_scratch[dev];
  std::call_once(s.once, [&s]() {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s.err == hipSuccess && p == nullptr) s.err = hipErrorInvalidSymbol;
    if (s.err == hipSuccess) s.ptr = p;
  });
  *out = s.ptr;
  return s.err;
}

}  // namespace

extern "C" int fa_decode_splitkv_noalloc(const void* q, const void* k_cache,
                                         const void* v_cache, void* o, float* lse, int B,
                                         int Hq, int Hkv, int Nk, int d, float scale,
                                         int num_splits, void* stream) {
  // Every argument check first (none of them calls HIP), then the one limit
  // of this entry point.
  int S = 0;
  const int rc = fa::decode_check(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nk, d, scale,
                                  num_splits, &S);
  if (rc != FA_OK) return rc;
  if (fa_decode_workspace_size(B, Hq, d, S) > FA_DECODE_NOALLOC_SCRATCH_BYTES)
    return FA_ERR_SCRATCH;

  void* ws = nullptr;
  const hipError_t e = device_scratch(static_cast<hipStream_t>(stream), &ws);
  if (e != hipSuccess) return fa::hip_status(e);
  // Every partial slot (empty chunks included) is written by the split
  // kernel before the merge reads it, so nothing needs clearing.
  return fa_decode_splitkv(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nk, d, scale, S, ws,
                           FA_DECODE_NOALLOC_SCRATCH_BYTES, stream);
}
