// twell_ffn_forward for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): the
// forward's workspaces live in one statically sized device array of the
// library instead of caller memory.
//
// `scratch` is a file-scope device array; every GPU the library runs on holds
// its own copy at its own address until the process ends. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol): on a device's first call its device address is looked up once
// with hipGetSymbolAddress, with that device current, and kept per device;
// the kernels receive that address as their workspace pointer, exactly as
// they receive a caller's workspace from twell_ffn_forward. No call here
// allocates, frees or creates a stream: everything is enqueued on the
// caller's stream in order.
#include <mutex>

#include "twell_host.h"
#include "twell_internal.h"
#include "twell_kernels.h"

namespace twell {
namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;  // TWELL_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == TWELL_NOALLOC_SCRATCH_BYTES, "header and library disagree on the scratch size");
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if ((err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace
}  // namespace twell

extern "C" twell_status twell_ffn_forward_noalloc(const twell_dims* dims, twell_dtype dtype, const void* x,
                                                   const void* w_gate_t, const float* t, const twell_pack* pack,
                                                   const void* w_up_t, const void* w_down, float* y, float* a_save,
                                                   void* stream) {
  twell_sizes z;
  twell_status st = twell_query_sizes(dims, dtype, &z);
  if (st != TWELL_OK) return st;
  // forward workspace first, then (small batches) the gate's g
  const size_t off_gate = twell::align256(z.ws_fwd);
  const size_t need = off_gate + z.ws_gate;
  if (need > twell::kScratchBytes)
    return twell::set_error(TWELL_ERR_WORKSPACE,
                            "twell_ffn_forward_noalloc: this shape needs more workspace than the library's static "
                            "scratch of TWELL_NOALLOC_SCRATCH_BYTES (128 MiB); use twell_ffn_forward with a "
                            "caller workspace");
  // every argument is checked before any HIP call (stand-in workspace address)
  void* fake = reinterpret_cast<void*>(uintptr_t(256));
  st = twell::ffn_forward_call(dims, dtype, x, w_gate_t, t, pack, w_up_t, w_down, y, a_save, fake, z.ws_fwd,
                               z.ws_gate ? fake : nullptr, z.ws_gate, false, true, stream);
  if (st != TWELL_OK || dims->n_tokens == 0) return st;
  void* base = nullptr;
  const hipError_t err = twell::scratch_address(&base);
  if (err != hipSuccess) {
    return twell::set_error(TWELL_ERR_HIP, (std::string("twell_ffn_forward_noalloc: scratch address: ") +
                                            hipGetErrorString(err)).c_str());
  }
  char* b = static_cast<char*>(base);
  return twell::ffn_forward_call(dims, dtype, x, w_gate_t, t, pack, w_up_t, w_down, y, a_save, b, z.ws_fwd,
                                 z.ws_gate ? b + off_gate : nullptr, z.ws_gate, false, false, stream);
}
