// ua_forward_noalloc: the planned path (one pass, or split-KV partitions and
// the LSE reduce) with the split-KV workspace in a library-owned static device
// array instead of caller memory, for callers that cannot allocate device
// memory.  No hipMalloc, hipFree or allocating library call is made.
//
// The array lives in this file's device code: each GPU the library runs on
// holds one copy (UA_NOALLOC_SCRATCH_BYTES) until the process ends.  Host code
// never uses the array's name as an address (on the host it is only a stand-in
// for the symbol): its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept per device; kernels
// receive that address exactly as they receive a caller's workspace.
//
// Nothing in the array needs to start at zero: the partition kernel writes
// every (m, l) entry of the plan and every acc row whose l is non-zero, and
// the reduce reads nothing else.  Every call on a GPU shares that GPU's array,
// so two calls that overlap in time on one GPU (different streams, or
// different host threads) race on it.

#include <mutex>

#include "ua_internal.h"

namespace {

constexpr uint64_t kScratchBytes = UA_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch` per device (null: not yet)
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up on the first
// call for that device.
ua_status scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return UA_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return UA_EHIP;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return UA_OK;
}

}  // namespace

extern "C" ua_status ua_forward_noalloc(const ua_problem* prob, const ua_plan_t* plan,
                                        const ua_args* args, void* stream) {
  if (!prob || !plan || !args) return UA_EINVAL;
  if (plan->path == UA_PATH_2D) return ua_forward_2d(prob, plan, args, stream);
  // Host checks first: an invalid call touches no device.
  ua_status st = ua::check_split_call(prob, plan, args);
  if (st != UA_OK) return st;
  if (prob->total_q == 0 || prob->num_seqs == 0) return UA_OK;
  if (plan->workspace_bytes > kScratchBytes) return UA_ESCRATCH;
  // The array is per device: the stream must belong to the current device.
  if (stream != nullptr) {
    hipDevice_t sdev;
    int cur = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess ||
        hipGetDevice(&cur) != hipSuccess)
      return UA_EHIP;
    if ((int)sdev != cur) return UA_EINVAL;
  }
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != UA_OK) return st;
  st = ua_forward_splitkv(prob, plan, args, ws, kScratchBytes, stream);
  if (st != UA_OK) return st;
  return ua_reduce(prob, plan, args, ws, kScratchBytes, stream);
}
