// Measurement kernels for the benchmark (not part of the collection path):
// the ceilings two of the collection's kernels are judged against on the
// machine at hand.
//
//  * weight_stream_kernel: the value kernel streams the packed critic and
//    curiosity weights from L2 into registers once per work item (16 x RT
//    rows; with more than four waves the two 4-tile layers are read once per
//    group of four).  This kernel issues the same bytes with no arithmetic:
//    a persistent grid of 256-thread workgroups, two per CU (the value
//    kernel's 8 waves per CU), each reading the block once per work item in
//    16-byte lanes (1 KiB per wave instruction), 16 loads in flight per
//    lane.  Its time for the value kernel's work-item count is the stream
//    bound the MFMA work competes with.
//  * gae_traffic_kernel: moves exactly the GAE scan's bytes (reads r, V, d;
//    writes two float arrays with streaming stores, as the scan does),
//    element-wise with no recurrence: the copy ceiling of the scan at a
//    given size.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nets.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 16;  // loads in flight per lane

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void
weight_stream_kernel(const uint4* __restrict__ blob, uint32_t rows, int64_t groups,
                     uint32_t* __restrict__ sink) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(blob), 0, (int)(rows * kThreads * 16u), 0x00020000);
  const uint32_t vo = threadIdx.x * 16u;
  uint32_t acc = 0;
  for (int64_t g = blockIdx.x; g < groups; g += gridDim.x) {
    int base = 0;
    asm volatile("" : "+s"(base));  // a fresh stream per work item
    for (uint32_t r0 = 0; r0 < rows; r0 += kBatch) {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      u32x4 v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, (uint32_t)base + (r0 + i) * kThreads * 16u, 0);
#pragma unroll
      for (int i = 0; i < kBatch; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;  // keeps the loads live
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void gae_traffic_kernel(
    const f32x4* __restrict__ r, const f32x4* __restrict__ v, const uint32_t* __restrict__ d,
    f32x4* __restrict__ a, f32x4* __restrict__ b, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n4) return;
  const f32x4 x = r[i], y = v[i];
  const uint32_t z = d[i];
  const f32x4 dz = {(float)(z & 255u), (float)((z >> 8) & 255u), (float)((z >> 16) & 255u),
                    (float)(z >> 24)};
  __builtin_nontemporal_store(x - y * dz, a + i);  // streaming stores, as the scan's
  __builtin_nontemporal_store(x + y, b + i);
}

}  // namespace

extern "C" {

// Bytes of the packed critic + curiosity weight block the value kernel
// streams per work item, and the rows of a work item.
int bench_value_stream_shape(int bf16, long long* block_bytes, int* rows_per_item) {
  if (!block_bytes || !rows_per_item) return 1;
  long long floats = 0;
  // the 4-tile layers (critic 128 -> 64, curiosity 128 -> 51) are read by
  // every group of four waves
  const int rh = rl::value_waves(bf16 != 0) / rl::kSplit;
  if (bf16) {
    for (int l = 0; l < 5; ++l)
      floats += rl::packed_layer_floats_bf16(rl::kCriticB[l]) * (l == 4 ? rh : 1);
    for (int l = 0; l < 2; ++l)
      floats += rl::packed_layer_floats_bf16(rl::kCurB[l]) * (l == 1 ? rh : 1);
  } else {
    for (int l = 0; l < 5; ++l)
      floats += rl::packed_layer_floats(rl::kCritic[l]) * (l == 4 ? rh : 1);
    for (int l = 0; l < 2; ++l) floats += rl::packed_layer_floats(rl::kCur[l]) * (l == 1 ? rh : 1);
  }
  *block_bytes = floats * 4;
  *rows_per_item = 16 * rl::value_row_tiles(bf16 != 0);
  return 0;
}

// Streams `bytes` (a multiple of 4 KiB; the last batch of 16 rows reads
// past the end through the buffer resource, which returns zeros without a
// memory request) from `blob` once per work item for
// `groups` work items on a grid filling every CU; `sink` (256 uint32) is
// written only if the checksum hits a fixed value.
int bench_weight_stream(const void* blob, long long bytes, long long groups, uint32_t* sink,
                        void* stream) {
  const long long row = (long long)kThreads * 16;
  if (!blob || !sink || bytes <= 0 || bytes % row != 0 || bytes >= (1ll << 31) || groups <= 0)
    return (int)hipErrorInvalidValue;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, weight_stream_kernel, kThreads, 0);
  if (e != hipSuccess) return (int)e;
  const long long resident = (long long)cus * (per_cu > 0 ? per_cu : 1);
  const unsigned grid = (unsigned)(groups < resident ? groups : resident);
  hipLaunchKernelGGL(weight_stream_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint4*)blob, (uint32_t)(bytes / (kThreads * 16)), (int64_t)groups, sink);
  return (int)hipGetLastError();
}

// Element-wise kernel with the GAE scan's traffic: n elements (a multiple of
// 4, 16-byte aligned float arrays, 4-byte aligned dones).
int bench_gae_traffic(const float* r, const float* v, const uint8_t* d, float* a, float* b,
                      long long n, void* stream) {
  if (!r || !v || !d || !a || !b || n <= 0 || n % 4 != 0) return (int)hipErrorInvalidValue;
  const long long n4 = n / 4;
  hipLaunchKernelGGL(gae_traffic_kernel, dim3((unsigned)((n4 + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, (hipStream_t)stream, (const f32x4*)r, (const f32x4*)v,
                     (const uint32_t*)d, (f32x4*)a, (f32x4*)b, (int64_t)n4);
  return (int)hipGetLastError();
}

}  // extern "C"
