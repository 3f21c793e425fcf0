// A plain streaming read of a buffer: the bandwidth reference the benchmark
// compares the library's read-bound kernels with (include/mla_measure.h).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device.h"
#include "launch.h"
#include "mla_measure.h"
#include "mla_post.h"

namespace {

using mla_dev::launch;

typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int RTHREADS = 512;
constexpr int RUNROLL = 16;  // 16-byte loads in flight per thread
constexpr int RPER_CU = 8;   // workgroups per CU

// Workgroup b reads its own contiguous chunk of the buffer (the pieces
// split evenly over the grid, 16 B a piece), RUNROLL rows of 512 pieces at a
// time; the XOR of everything is stored only if it equals an arbitrary
// constant. Contiguous chunks keep every workgroup on few DRAM pages at once,
// which a grid-stride loop over the whole buffer does not.
__global__ __launch_bounds__(RTHREADS) void read_kernel(const uint8_t* p, int64_t pieces, v4u* sink) {
  const v4u* src = reinterpret_cast<const v4u*>(p);
  const int64_t per = (pieces + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t end = b0 + per < pieces ? b0 + per : pieces;
  int64_t i = b0 + threadIdx.x;
  v4u x = {0u, 0u, 0u, 0u};
  for (; i + (RUNROLL - 1) * RTHREADS < end; i += RUNROLL * RTHREADS) {
    v4u v[RUNROLL];
#pragma unroll
    for (int u = 0; u < RUNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * RTHREADS);
#pragma unroll
    for (int u = 0; u < RUNROLL; ++u) x ^= v[u];
  }
  for (; i < end; i += RTHREADS) x ^= __builtin_nontemporal_load(src + i);
  if (x.x == 0x9E3779B9u && x.y == 0x7F4A7C15u && x.z == 0x2545F491u && x.w == 0x4F6CDD1Du) *sink = x;
}

}  // namespace

extern "C" {

int mla_measure_read(const void* p, int64_t bytes, void* sink, void* stream) {
  if (bytes < 0 || bytes > (int64_t(1) << 40) || (bytes % 16)) return MLA_POST_EINVAL;
  if (bytes == 0) return MLA_POST_OK;
  if (!p || !sink) return MLA_POST_EINVAL;
  if ((reinterpret_cast<uintptr_t>(p) & 15) || (reinterpret_cast<uintptr_t>(sink) & 15)) return MLA_POST_EALIGN;
  const int64_t pieces = bytes / 16;
  // RPER_CU workgroups of 512 threads per CU, fewer for small buffers
  const int64_t want = (pieces + RTHREADS - 1) / RTHREADS;
  const int64_t most = RPER_CU * (int64_t)mla_dev::device_cus();
  const int64_t grid = want < most ? want : most;
  return launch(read_kernel, dim3((unsigned)grid), dim3(RTHREADS), static_cast<hipStream_t>(stream),
                static_cast<const uint8_t*>(p), pieces, static_cast<v4u*>(sink));
}

}  // extern "C"
