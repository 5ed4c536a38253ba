// Decode without a caller workspace: sparse_attn_decode_paged_noalloc runs
// the same range teams and merge as sparse_attn_decode_paged, with their
// partial results in a static device array instead of a caller buffer, for
// callers that cannot allocate (stream capture into a HIP graph, serving
// loops, harnesses that forbid device allocation).
//
// Each device holds its own copy of the array for the life of the process.
// Its device address is looked up once per device, with that device
// current, on the first call there (after the arguments have passed); the
// kernels receive that address, never the array's host-side name. Calls
// that overlap on one device share the array and race. The partial results
// need no clearing: a range without a valid slot writes its LSE only, and
// the merge never reads its O.
#include <atomic>
#include <cstdio>
#include <mutex>

#include "sparse_attn.h"
#include "sa_internal.h"

namespace {

constexpr size_t kScratchBytes = SA_DECODE_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address; nullptr and a message on failure.
void* scratch_lookup(char* msg, size_t msg_len) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(msg, msg_len, "no current device: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, msg_len, "device %d beyond the %d the scratch table covers", dev, kMaxDevices);
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(msg, msg_len, "scratch address lookup on device %d failed: %s", dev,
               hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" sa_status sparse_attn_decode_paged_noalloc(
    const sa_attn_desc* desc, const sa_page_desc* pages, const void* q, const uint8_t* pool,
    int32_t num_dst_pages, const int32_t* idx, const int32_t* topk_len, int32_t batch,
    float* out, float* lse, hipStream_t stream) {
  sa::api_clear_error();
  return sa::decode_paged_ws(desc, pages, q, pool, num_dst_pages, idx, topk_len, batch, nullptr,
                             kScratchBytes, out, lse, stream, SA_ENTRY_DECODE_PAGED_NOALLOC,
                             scratch_lookup);
}
