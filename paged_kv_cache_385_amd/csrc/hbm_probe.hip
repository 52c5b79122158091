// Streaming-read probes: how fast gfx950's memory system delivers bytes that are
// read once and never reused, with nothing computed on them.  They give the
// decode kernel a measured ceiling beside the nominal HBM peak: decode attention
// is bound by reading the cached history ("PagedAttention 实战", section
// "Decode：逐 token 生成输出"), and a kernel that only reads the same bytes in
// the same pattern shows what that pattern can reach on the device.
//
//   probe_contiguous_kernel  one buffer, front to back
//   probe_tiles_kernel       a list of (block, head) tiles of a K pool and a V pool,
//                            in the given order (the tile gather of a decode pass)
//
// Both use 16-byte non-temporal loads (the decode kernel's streaming loads) and
// fold the data into one word per thread, stored only if it equals a value the
// caller's data never produces, so no load can be dropped.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_internal.h"
#include "../../include/pa_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 4;               // 16-byte loads in flight per thread
constexpr uint32_t kNever = 0x9E3779B9u; // folded value that triggers the sink store

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kThreads) void probe_contiguous_kernel(const u32x4* __restrict__ p,
                                                                    int64_t n_vec,
                                                                    uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n_vec; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
  }
  for (; i < n_vec; i += stride) acc ^= fold(__builtin_nontemporal_load(p + i));
  if (acc == kNever) sink[0] = acc;
}

// Each tile is read by 2^lanes_log2 lanes of 16 bytes (64 lanes for 1 KiB, 256 for 4 KiB);
// a workgroup reads 256 >> lanes_log2 tiles of each pool per load instruction, tiles
// t, t + step, ... of the list (step = that count x the grid), two tiles in flight.
__global__ __launch_bounds__(kThreads) void probe_tiles_kernel(const char* __restrict__ k_base,
                                                               const char* __restrict__ v_base,
                                                               const int32_t* __restrict__ tiles,
                                                               int32_t num_tiles, int32_t lanes_log2,
                                                               uint32_t* __restrict__ sink) {
  const int64_t tile_bytes = int64_t{16} << lanes_log2;
  const int32_t per_wg = kThreads >> lanes_log2;
  const int64_t lane_off = static_cast<int64_t>(threadIdx.x & ((1 << lanes_log2) - 1)) * 16;
  const int32_t step = static_cast<int32_t>(gridDim.x) * per_wg;
  uint32_t acc = 0;
  int32_t t = blockIdx.x * per_wg + (threadIdx.x >> lanes_log2);
  for (; t + step < num_tiles; t += 2 * step) {
    const int64_t a = static_cast<int64_t>(tiles[t]) * tile_bytes + lane_off;
    const int64_t b = static_cast<int64_t>(tiles[t + step]) * tile_bytes + lane_off;
    const u32x4 ka = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_base + a));
    const u32x4 va = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_base + a));
    const u32x4 kb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_base + b));
    const u32x4 vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_base + b));
    acc ^= fold(ka) ^ fold(va) ^ fold(kb) ^ fold(vb);
  }
  if (t < num_tiles) {
    const int64_t a = static_cast<int64_t>(tiles[t]) * tile_bytes + lane_off;
    acc ^= fold(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_base + a)));
    acc ^= fold(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_base + a)));
  }
  if (acc == kNever) sink[0] = acc;
}

}  // namespace

extern "C" {

pa_status pa_probe_read_contiguous(const void* buf, size_t bytes, int32_t workgroups_per_cu,
                                   uint32_t* sink, void* stream) {
  const char* fn = "pa_probe_read_contiguous";
  pa::clear_error();
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15u) || bytes % 16 || bytes == 0)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: buf NULL, misaligned or not a multiple of 16 bytes", fn);
  if (workgroups_per_cu < 1 || workgroups_per_cu > 64)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: workgroups_per_cu %d (1 .. 64)", fn, workgroups_per_cu);
  const int64_t grid = static_cast<int64_t>(pa::device_cus()) * workgroups_per_cu;
  probe_contiguous_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0,
                            static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(buf), static_cast<int64_t>(bytes / 16), sink);
  return pa::launch_status(fn);
}

pa_status pa_probe_read_tiles(const void* k_base, const void* v_base, size_t pool_bytes,
                              int32_t tile_bytes, const int32_t* tiles, const int32_t* tiles_host,
                              int32_t num_tiles, int32_t workgroups_per_cu, uint32_t* sink,
                              void* stream) {
  const char* fn = "pa_probe_read_tiles";
  pa::clear_error();
  if (!k_base || !v_base || !tiles || !tiles_host || !sink || num_tiles < 1 ||
      (reinterpret_cast<uintptr_t>(k_base) & 15u) || (reinterpret_cast<uintptr_t>(v_base) & 15u))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL or misaligned argument, or no tiles", fn);
  if (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: tile_bytes %d (1024, 2048 or 4096)", fn, tile_bytes);
  if (workgroups_per_cu < 1 || workgroups_per_cu > 64)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: workgroups_per_cu %d (1 .. 64)", fn, workgroups_per_cu);
  const int32_t lanes_log2 = tile_bytes == 1024 ? 6 : tile_bytes == 2048 ? 7 : 8;
  const int64_t n_pool = static_cast<int64_t>(pool_bytes / static_cast<size_t>(tile_bytes));
  for (int32_t i = 0; i < num_tiles; ++i)
    if (tiles_host[i] < 0 || tiles_host[i] >= n_pool)
      return pa::fail(PA_ERR_INVALID_ARG, "%s: tile %d = %d outside the pools' %lld tiles", fn, i,
                      tiles_host[i], static_cast<long long>(n_pool));
  const int64_t grid = static_cast<int64_t>(pa::device_cus()) * workgroups_per_cu;
  probe_tiles_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream)>>>(
      static_cast<const char*>(k_base), static_cast<const char*>(v_base), tiles, num_tiles,
      lanes_log2, sink);
  return pa::launch_status(fn);
}

}  // extern "C"
