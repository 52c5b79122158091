// pa_decode_noalloc: pa_decode for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The decode's scratch -- the merge counters and the partition
// states -- lives in one file-scope device array that each GPU holds for the
// life of the process, instead of a caller-provided workspace.
//
// The array's name is a host-side stand-in in host code, not a device address.
// Its address on each device comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is handed to kernels.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "pa_internal.h"

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // the array's address on each device, once known

// Address of the scratch array on the current device.
pa_status scratch_address(const char* fn, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return pa::fail(PA_ERR_HIP, "%s: no current device (or device id %d out of range)", fn, dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pa::fail(PA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                      hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

// Zeroes n 32-bit words (a kernel, not hipMemsetAsync, so a captured graph replays it
// as a kernel node).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

extern "C" {

pa_status pa_decode_noalloc(const pa_cache* cache, const void* q, int32_t num_seqs,
                            int32_t num_heads, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, float scale, void* out, void* stream) {
  const char* fn = "pa_decode_noalloc";
  pa::clear_error();
  pa_status st = pa::check_cache(cache, fn);
  if (st != PA_OK) return st;
  if (num_seqs > 0 && (!block_tables || !context_lens))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: block_tables / context_lens NULL", fn);
  const size_t need =
      pa_decode_workspace_size(num_seqs, num_heads, cache->head_dim, max_context_len);
  if (need > kScratchBytes)
    return pa::fail(PA_ERR_WORKSPACE,
                    "%s: %d sequences x %d heads up to %d tokens need %zu bytes of scratch; the "
                    "library holds %zu (PA_NOALLOC_SCRATCH_BYTES): use pa_decode with a workspace",
                    fn, num_seqs, num_heads, max_context_len, need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(fn, &ws);
    if (st != PA_OK) return st;
    // every check pa_decode makes, before anything is enqueued
    st = pa::decode_check(cache, q, num_seqs, num_heads, max_blocks_per_seq, max_context_len, scale,
                          out, ws, need);
    if (st != PA_OK) return st;
    // the merge counters and the claim counter start at zero (they lead the scratch, as
    // they lead a workspace)
    const int64_t words = static_cast<int64_t>(num_seqs) * num_heads + 1;
    zero_words_kernel<<<dim3(static_cast<uint32_t>((words + 255) / 256)), dim3(256), 0,
                        static_cast<hipStream_t>(stream)>>>(static_cast<uint32_t*>(ws), words);
    st = pa::launch_status(fn);
    if (st != PA_OK) return st;
  }
  return pa::decode_run(fn, cache, q, num_seqs, num_heads, block_tables, max_blocks_per_seq,
                        context_lens, max_context_len, scale, out, ws, need, nullptr, nullptr,
                        nullptr, true, true, 0, nullptr, nullptr, stream);
}

}  // extern "C"
