// hybrid_layer_decode_noalloc: the decode step of hybrid_layer_decode with its
// workspace in a file-scope device array instead of caller memory, for
// callers that cannot allocate (code under graph capture, tight serving
// loops).
//
// The array `scratch` is one per device (each device holds its own copy while
// the library is loaded).  Host code never passes the array's name to a
// kernel: its device address is taken once per device with
// hipGetSymbolAddress while that device is current, and kept in g_dev[] with
// the configuration of the last call on the device.  The workspace contract
// of hybrid_layer_decode (zero-filled when first used, and again whenever it
// serves another configuration) is kept by clearing the bytes the call needs
// with a fill kernel on the first call and whenever the configuration differs
// from the previous call's on that device; the decode kernels leave their
// counters at zero when they finish.

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "csa.h"
#include "kernels.h"

namespace {

// 32 MiB: the decode workspace of a Pro-shaped CSA layer (4 sequences of
// 262,144 entries, k = 1024, 128 heads) or a Flash-shaped HCA layer (8
// sequences of 8,192 entries, 64 heads) fits
constexpr size_t kScratchBytes = (size_t)32 << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// what a call's workspace layout depends on
struct Config {
  csa_layer_desc d;
  int B, E_cap;
  int paged;  // a paged cache runs other kernels (the fold apart from the scan)
  bool operator==(const Config& o) const { return std::memcmp(this, &o, sizeof(Config)) == 0; }
};

struct DevScratch {
  void* ptr = nullptr;  // device address of `scratch` on this device
  bool have_cfg = false;
  Config cfg;
};

std::mutex g_mu;
DevScratch g_dev[csa::kMaxDevices];

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = uint4{0, 0, 0, 0};
}

}  // namespace

extern "C" {

size_t hybrid_layer_noalloc_scratch_bytes(void) { return kScratchBytes; }

csa_status hybrid_layer_decode_noalloc(const csa_layer_desc* desc, csa_layer_state* state,
                                       const csa_decode_io* io, void* stream) {
  // every argument check first: an error enqueues nothing
  const csa_status chk = csa::decode_check(desc, state, io);
  if (chk != CSA_OK) return chk;
  const size_t need = hybrid_layer_workspace(desc, state->B, 1, state->E_cap);
  if (need > kScratchBytes)
    return (csa_status)csa::set_error(CSA_ERR_WORKSPACE,
                                      "hybrid_layer_decode_noalloc: this call needs %zu bytes of workspace, "
                                      "more than its %zu-byte scratch array",
                                      need, kScratchBytes);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= csa::kMaxDevices)
    return (csa_status)csa::set_error(CSA_ERR_DEVICE, "hybrid_layer_decode_noalloc: no usable current device");
  std::lock_guard<std::mutex> lk(g_mu);
  DevScratch& ds = g_dev[dev];
  if (ds.ptr == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return (csa_status)csa::set_error(CSA_ERR_DEVICE, "hybrid_layer_decode_noalloc: hipGetSymbolAddress: %s",
                                        hipGetErrorString(e));
    ds.ptr = p;
  }
  Config cfg;
  std::memset(&cfg, 0, sizeof(cfg));
  cfg.d = *desc;
  cfg.B = state->B;
  cfg.E_cap = state->E_cap;
  cfg.paged = state->block_table != nullptr;
  if (!ds.have_cfg || !(ds.cfg == cfg)) {
    // another configuration places other data where this one's counters
    // live: clear what this call uses (stream-ordered before it)
    const size_t n16 = (need + 15) / 16;
    const unsigned grid = (unsigned)((n16 + 255) / 256 < 2048 ? (n16 + 255) / 256 : 2048);
    hipLaunchKernelGGL(scratch_clear_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<uint4*>(ds.ptr), n16);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return (csa_status)csa::set_error(CSA_ERR_DEVICE, "hybrid_layer_decode_noalloc: clearing the scratch: %s",
                                        hipGetErrorString(e));
    ds.cfg = cfg;
    ds.have_cfg = true;
  }
  const csa_status st = hybrid_layer_decode(desc, state, io, ds.ptr, kScratchBytes, stream);
  if (st != CSA_OK) ds.have_cfg = false;  // a failed call may leave counters set: clear next time
  return st;
}

}  // extern "C"
