// Allocation-free latent-cache decode: the step of mla_decode_latentcache
// with its workspace in a library-owned device array instead of a caller
// buffer.  It serves callers that cannot call hipMalloc (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array lives in this file's device code object, one copy per GPU that
// loads the library, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it names a stand-in, not device
// memory): on the first call on a device, with that device current, its
// device address is looked up once with hipGetSymbolAddress and cached per
// device, and only that address is used afterwards.
//
// Every call on a GPU shares that GPU's array, and the array keeps what the
// last call left in it.  The decode kernels write every workspace word they
// read within the same step (projection outputs, split partials, split
// records and plans), so nothing has to start at zero.  Calls that overlap
// on one GPU (other streams, other threads) race on the array.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/mla.h"

namespace {

static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

// Device address of this device's array (looked up on the first call on
// the device); NULL with *err set when the lookup fails.
void* scratch_on(int dev, hipError_t* err) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  *err = hipSuccess;
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

// argument checks and error reporting of the C-ABI layer (mla_api.cpp)
extern "C" int mla_internal_decode_latent_check(const mla_dims* d, const mla_weights* w, const void* x,
                                                int B, int P, int L_cap, const void* latent_cache,
                                                const float* rc, const float* rs, int rope_rows,
                                                const void* out);
extern "C" int mla_internal_fail(int code, const char* msg);

extern "C" int mla_decode_latentcache_noalloc(const mla_dims* dims, const mla_weights* w,
                                              const void* x, int B, int P, int L_cap,
                                              void* latent_cache, const float* rope_cos,
                                              const float* rope_sin, int rope_rows, void* out,
                                              void* stream) {
  // every argument check, then the size check, before any HIP call
  int r = mla_internal_decode_latent_check(dims, w, x, B, P, L_cap, latent_cache, rope_cos, rope_sin,
                                           rope_rows, out);
  if (r) return r;
  const size_t need = mla_decode_workspace_size(dims, B, L_cap);
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "allocation-free decode: B=%d, L_cap=%d need %zu bytes of scratch, above the %u-byte "
             "array; use mla_decode_latentcache with a caller workspace",
             B, L_cap, need, (unsigned)MLA_NOALLOC_SCRATCH_BYTES);
    return mla_internal_fail(MLA_ERR_WORKSPACE, msg);
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mla_internal_fail(MLA_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return mla_internal_fail(MLA_ERR_UNSUPPORTED, "device index above 63");
  if (stream) {
    // the array used is the current device's; the stream must run there
    int sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return mla_internal_fail(MLA_ERR_HIP, hipGetErrorString(e));
    if (sdev != dev)
      return mla_internal_fail(MLA_ERR_UNSUPPORTED, "stream belongs to a device other than the current one");
  }
  void* ws = scratch_on(dev, &e);
  if (!ws) return mla_internal_fail(MLA_ERR_HIP, hipGetErrorString(e));
  return mla_decode_latentcache(dims, w, x, B, P, L_cap, latent_cache, rope_cos, rope_sin, rope_rows,
                                out, ws, (size_t)MLA_NOALLOC_SCRATCH_BYTES, stream);
}
