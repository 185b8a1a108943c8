// bd_attn_packed_noalloc: bd_attn_packed for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops).
//
// The attention's scratch (the longest-first row order and the split-prefix
// partials) lives in one file-scope device array instead of a caller
// workspace.  Host code never uses the array's name as an address: on the
// first call on each device, with that device current, the device address
// is looked up with hipGetSymbolAddress and kept per device; kernels get
// that address.  Nothing in the array needs clearing between calls (the row
// order and the partials are written before they are read), and every call
// on one GPU shares it, so calls that overlap on one GPU (two streams) race.
#include <mutex>

#include "bd_common.h"

static __device__ __align__(256) char scratch[BD_NOALLOC_SCRATCH_BYTES];

namespace bd {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device); BD_OK or an error status with the message set.
int scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return attn_launch_status(e, "bd_attn_packed_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("bd_attn_packed_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    return BD_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return attn_launch_status(e, "bd_attn_packed_noalloc: hipGetSymbolAddress");
    if (!p || ((uintptr_t)p & 255u) != 0) {
      set_error("bd_attn_packed_noalloc: scratch address %p is not 256-byte aligned", p);
      return BD_ERR_HIP;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return BD_OK;
}

}  // namespace
}  // namespace bd

using namespace bd;

extern "C" int bd_attn_packed_noalloc(int dtype, int B, int Hq, int Hkv, int d, int q, int bl,
                                      const int32_t *row_ids, int n_rows, const void *q_ptr,
                                      const int64_t q_strides[3], const void *pk, const void *pv,
                                      const int64_t p_strides[3], int p_cap, const int32_t *p_len,
                                      int p_max, const void *wk, const void *wv,
                                      const int64_t w_strides[3], float sm_scale, void *out,
                                      const int64_t out_strides[3], float *lse, void *stream) {
  static const char *fn = "bd_attn_packed_noalloc";
  const PrefixArg pa{row_ids, n_rows, pk, pv, p_strides, p_cap, p_len, p_max};
  AttnArgs a;
  AttnPlan plan;
  bool launch;
  const int st = attn_setup(fn, dtype, B, Hq, Hkv, d, q, bl, BD_MASK_BLOCK_CAUSAL, q_ptr, q_strides,
                            pa, nullptr, wk, wv, w_strides, sm_scale, out, out_strides, lse, a, plan,
                            &launch);
  if (st != BD_OK || !launch) return st;
  if (plan.ws_bytes > (size_t)BD_NOALLOC_SCRATCH_BYTES) {
    set_error("%s: this call needs %zu bytes of scratch, more than the %zu the library holds",
              fn, plan.ws_bytes, (size_t)BD_NOALLOC_SCRATCH_BYTES);
    return BD_ERR_WORKSPACE;
  }
  if (plan.ws_bytes > 0) {
    void *ws = nullptr;
    const int e = scratch_address(&ws);
    if (e != BD_OK) return e;
    attn_bind_workspace(a, plan, (char *)ws);
  }
  return attn_launch_status(launch_attn(a, (hipStream_t)stream), fn);
}
