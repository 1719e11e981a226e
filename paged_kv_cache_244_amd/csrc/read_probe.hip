// A plain HBM read kernel: the bandwidth ceiling that decode attention is
// measured against.  Decode reads every cached key and value once per step and
// does little arithmetic per byte ("Only 20.4% of your KV cache held actual
// tokens" (blog.teqners.com), section "Why the KV cache is the thing that
// limits your batch"), so its time is bounded below by the bytes it reads over
// the bandwidth this kernel reaches on the same device.
//
// The buffer is a sequence of 4 KiB tiles, the size of one (block, KV head) of
// K or V at 16 tokens x 128 dims in fp16.  Tiles are read in order, or in the
// order of a device index array (a permutation gives the scattered 4 KiB reads
// of a paged pool).  One 256-thread workgroup reads a tile with one 16-byte
// non-temporal load per thread, kProbeUnroll tiles in flight; the XOR of all
// words decides a store that never happens for zeros, so no load can be
// dropped by the compiler.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "errors.h"
#include "launch.h"
#include "pagedkv.h"

namespace {

using pkv::fail;

constexpr int kProbeThreads = 256;     // 16-byte chunks per 4 KiB tile
constexpr int kProbeUnroll = 8;        // tiles in flight per workgroup

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ src,
                                                                   const int32_t* __restrict__ order,
                                                                   int64_t num_tiles,
                                                                   uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t step = static_cast<int64_t>(gridDim.x) * kProbeUnroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kProbeUnroll; base < num_tiles;
       base += step) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t i = base + u;
      int64_t tile = -1;
      if (i < num_tiles) tile = order ? static_cast<int64_t>(order[i]) : i;
      if (static_cast<uint64_t>(tile) < static_cast<uint64_t>(num_tiles))
        v[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(src + tile * kProbeThreads + threadIdx.x));
      else
        v[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" int pkv_read_probe(const void* src, int64_t num_tiles, const int32_t* tile_order,
                              uint32_t* sink, int32_t workgroups, void* stream) {
  pkv::TimedCall timed;   // consumes the events of pkv_time_next_call
  if (num_tiles < 0 || workgroups <= 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_read_probe: num_tiles %lld, workgroups %d",
                static_cast<long long>(num_tiles), workgroups);
  if (num_tiles == 0) return PKV_OK;
  if (!src || !sink) return fail(PKV_ERR_INVALID_ARG, "pkv_read_probe: NULL pointer");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_read_probe: src must be 16-byte aligned");
  pkv::launch_kernel(read_probe_kernel, dim3(static_cast<unsigned>(workgroups)),
                     dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), tile_order, num_tiles, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_read_probe launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

// Events for pkv_time_next_call: created here (not recorded), so that a caller
// need not record an event on a stream merely to bring it into existence.
extern "C" int pkv_event_create(void** event) {
  if (!event) return fail(PKV_ERR_INVALID_ARG, "pkv_event_create: NULL");
  hipEvent_t e = nullptr;
  const hipError_t rc = hipEventCreate(&e);
  if (rc != hipSuccess) return fail(PKV_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(rc));
  *event = e;
  return PKV_OK;
}

extern "C" int pkv_event_destroy(void* event) {
  if (!event) return PKV_OK;
  const hipError_t rc = hipEventDestroy(static_cast<hipEvent_t>(event));
  if (rc != hipSuccess) return fail(PKV_ERR_HIP, "hipEventDestroy: %s", hipGetErrorString(rc));
  return PKV_OK;
}

extern "C" int pkv_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return fail(PKV_ERR_INVALID_ARG, "pkv_event_elapsed_ms: NULL");
  hipError_t rc = hipEventSynchronize(static_cast<hipEvent_t>(stop));
  if (rc == hipSuccess)
    rc = hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop));
  if (rc != hipSuccess) return fail(PKV_ERR_HIP, "pkv_event_elapsed_ms: %s", hipGetErrorString(rc));
  return PKV_OK;
}
