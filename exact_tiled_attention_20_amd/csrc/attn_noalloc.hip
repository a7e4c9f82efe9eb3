// attn_bwd_noalloc: the backward without a caller-supplied workspace, for
// callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The workspace attn_bwd takes (two float32 (B, H, Np) arrays, Np = N rounded
// up to a multiple of 4: D_i = dO_i . O_i and lse_i * log2(e)) lives instead in a fixed file-scope device array,
// `scratch`, of kScratchBytes per GPU. Each GPU that runs the library holds its
// own copy until the process ends. Host code never uses the array's name as
// a device address: the address is resolved once per device with
// hipGetSymbolAddress (with that device current) and cached. This entry point
// calls no allocating routine.
//
// Every call on one GPU shares that GPU's array and leaves its contents behind.
// Nothing in it needs to start at zero: the first backward kernel writes every
// element the later ones read. Calls that overlap in time on one GPU (two host
// threads, or two streams without ordering between them) race on the array.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/attn.h"
#include "api_internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
std::atomic<void*> g_ptr[kMaxDevices];

// Device address of this GPU's scratch array, resolved on first use with the
// device current. Returns nullptr if the runtime cannot provide it.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_mu);
  p = g_ptr[dev].load(std::memory_order_relaxed);
  if (p != nullptr) return p;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || addr == nullptr) return nullptr;
  g_ptr[dev].store(addr, std::memory_order_release);
  return addr;
}

}  // namespace

extern "C" {

size_t attn_bwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

attn_status attn_bwd_noalloc(const attn_params* p, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* d_o, void* dq,
                             void* dk, void* dv, void* stream) {
  // Parameter and pointer errors are reported exactly as attn_bwd reports
  // them, before any HIP call; then the size limit.
  const attn_status st =
      attn::bwd_validate_without_workspace(p, q, k, v, o, lse, d_o, dq, dk, dv);
  if (st != ATTN_OK) return st;
  const size_t need = attn_bwd_workspace_bytes(p);
  if (need > kScratchBytes) return ATTN_ERR_TOO_LARGE;
  // No workspace needed (no query rows, or an empty problem): attn_bwd takes
  // none either.
  if (need == 0) return attn_bwd(p, q, k, v, o, lse, d_o, dq, dk, dv, nullptr, 0, stream);
  int dev = -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (s != nullptr) {
    if (hipStreamGetDevice(s, &dev) != hipSuccess) return ATTN_ERR_LAUNCH;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return ATTN_ERR_LAUNCH;
  }
  void* ws = scratch_on(dev);
  if (ws == nullptr) return ATTN_ERR_LAUNCH;
  return attn_bwd(p, q, k, v, o, lse, d_o, dq, dk, dv, ws, kScratchBytes, stream);
}

}  // extern "C"
