// xt_op_bwd_noalloc: xt_op_bwd with its workspace taken from a static device
// array of this library instead of the caller, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array `scratch` below is XT_NOALLOC_SCRATCH_BYTES of device memory
// that every GPU the library runs on holds from the first call until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the device symbol): the first call on a
// device resolves the device address with hipGetSymbolAddress, with that
// device current, and keeps it per device; every kernel argument and size
// below uses that address.
//
// What the kernels put in the workspace (parameter-gradient partial rows,
// split-K partial products, the attention row term, the embedding sort keys
// and segment sums) is written before it is read within one call, so nothing
// has to start at zero and nothing is cleared.  All calls on one GPU share
// its array: two calls whose kernels overlap on that GPU (different streams,
// or different host threads without ordering) race on it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "../../include/xt.h"
#include "internal.h"

namespace {

constexpr size_t SCRATCH_BYTES = XT_NOALLOC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_mu;
void* g_ptr[MAX_DEVICES];          // device address of `scratch` per device, once resolved

// Device address of this device's `scratch`, resolved on the first call with
// the device current.
xt_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return xt::set_error(XT_ERR_HIP, "xt_op_bwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES)
    return xt::set_error(XT_ERR_UNSUPPORTED, "xt_op_bwd_noalloc: device %d is beyond the %d this library tracks", dev,
                         MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return xt::set_error(XT_ERR_HIP, "xt_op_bwd_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return XT_OK;
}

}  // namespace

extern "C" xt_status xt_op_bwd_noalloc(xt_op op, const xt_params* prm, const xt_tensor* dout, const xt_tensor* in,
                                       int n_in, const xt_tensor* saved, int n_saved, const xt_tensor* din, int n_din,
                                       uint32_t accumulate, void* stream) {
  if (!prm) return xt::set_error(XT_ERR_INVALID_ARG, "null params");
  if (!in || n_in < 1) return xt::set_error(XT_ERR_INVALID_ARG, "null or empty input list");
  const size_t need = xt_workspace_bytes(op, 1, prm, in, n_in);
  // A matmul splits its contraction less when given less workspace (same
  // product, one f32 partial per slice): it runs within the array whatever
  // its size.  Every other op needs its whole workspace.
  const size_t use = op == XT_OP_MATMUL ? std::min(need, SCRATCH_BYTES) : need;
  if (use > SCRATCH_BYTES)
    return xt::set_error(XT_ERR_WORKSPACE,
                         "xt_op_bwd_noalloc: this backward needs %zu bytes of workspace, beyond the static %zu-byte "
                         "scratch array; call xt_op_bwd with a caller workspace instead",
                         need, SCRATCH_BYTES);
  void* ws = nullptr;
  if (use) {
    const xt_status st = scratch_ptr(&ws);
    if (st != XT_OK) return st;
  }
  return xt_op_bwd(op, prm, dout, in, n_in, saved, n_saved, din, n_din, accumulate, use ? ws : nullptr, use, stream);
}
