// rsa_score_blocks_noalloc: the scoring call with its workspace in a static
// device array, for callers that cannot allocate device memory (HIP graph
// capture, serving loops, harnesses that forbid it).
//
// The array below is a file-scope __device__ object: every GPU the library
// runs on holds its own copy (kNoallocScratchBytes) until the process ends.
// Host code never passes the array's name to a kernel (on the host that name
// is only a stand-in, not a device address); the device address is looked up
// once per device with hipGetSymbolAddress, on the first call made with that
// device current, and that pointer is what the kernels receive.
// Every call on a device shares the array, and the scoring kernels write all
// of their workspace before reading it, so nothing needs clearing between
// calls; calls that overlap in time on one device (two streams, two host
// threads) race on the array.
#include <mutex>

#include "rsa.h"
#include "kernels.h"

namespace {

__device__ __align__(256) unsigned char scratch[RSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (nullptr on failure).
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = ptr;
  }
  return g_ptr[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" rsa_status rsa_score_blocks_noalloc(const rsa_problem* p, const void* q, const void* k,
                                               const uint8_t* head_active, float* scores, hipStream_t stream) {
  if (p == nullptr || q == nullptr || k == nullptr || scores == nullptr) return RSA_ERR_NULL;
  // the problem checks and the launches are those of rsa_score_blocks, with
  // the static array as the workspace
  const size_t need = rsa_workspace_bytes(p, RSA_OP_SCORE);
  if (need == 0) {
    // invalid problem: let the regular entry point name the error (it
    // validates before touching the workspace)
    return rsa_score_blocks(p, q, k, head_active, scores, nullptr, 0, stream);
  }
  if (need > RSA_NOALLOC_SCRATCH_BYTES) return RSA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(scores)) return RSA_ERR_ALIGN;
  void* ws = scratch_ptr();
  if (ws == nullptr) return RSA_ERR_HIP;
  return rsa_score_blocks(p, q, k, head_active, scores, ws, need, stream);
}
