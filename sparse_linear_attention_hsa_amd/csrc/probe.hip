// Measurement helpers, not on the decode path: the bf16 matrix-core rate and
// the HBM stream-copy rate this GPU sustains, the denominators of the "% of
// the measured peak" figures.
// Every wave runs `iters` rounds of 32 independent v_mfma_f32_16x16x32_bf16
// products on register operands with a workgroup barrier per round: 8 waves
// per workgroup and one workgroup per CU (held there by its LDS footprint),
// i.e. 2 waves per SIMD -- the shape that gave the highest rate.
#include "common.h"
#include "host.h"

namespace hsa {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeAcc = 32;

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* __restrict__ out, int iters, int seed) {
  __shared__ float pad[24 * 1024];  // 96 KB: one workgroup per CU
  f32x4 acc[kProbeAcc];
#pragma unroll
  for (int i = 0; i < kProbeAcc; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint4 ua = make_uint4(threadIdx.x + (unsigned)seed, 1u, 2u, 3u);
  const uint4 ub = make_uint4(4u, threadIdx.x, 6u, (unsigned)seed);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kProbeAcc; ++i) Mma<bf16_t>::run(acc[i], ua, ub);
    __syncthreads();
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kProbeAcc; ++i) s += (acc[i][0] + acc[i][1]) + (acc[i][2] + acc[i][3]);
  if (seed < 0) pad[threadIdx.x] = s;  // never taken: keeps the LDS allocation
  __syncthreads();
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s + (seed < 0 ? pad[threadIdx.x] : 0.f);
}

// Stream copy: each workgroup copies one contiguous chunk, 16 bytes per
// lane, four loads in flight per thread, with non-temporal loads and stores
// (every byte is touched once).  Of the shapes measured (grid-stride or
// chunked, plain or non-temporal, 1024-4096 workgroups, 4 or 8 in flight)
// this one was the fastest.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int kCopyGroups = 4096;
__global__ __launch_bounds__(kCopyThreads) void copy_probe_kernel(const uint4* __restrict__ src,
                                                                  uint4* __restrict__ dst, size_t n16) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t first = (size_t)blockIdx.x * per;
  const size_t end = first + per < n16 ? first + per : n16;
  size_t i = first + threadIdx.x;
  for (; i + (kCopyUnroll - 1) * kCopyThreads < end; i += kCopyUnroll * kCopyThreads) {
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = ld16_nt(src + i + u * kCopyThreads);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const u32x4_nt w = {v[u].x, v[u].y, v[u].z, v[u].w};
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4_nt*>(dst + i + u * kCopyThreads));
    }
  }
  for (; i < end; i += kCopyThreads) dst[i] = src[i];
}

}  // namespace
}  // namespace hsa

extern "C" hsa_rc hsa_probe_mfma_bf16(int32_t n_workgroups, int32_t iters, float* out, hsa_stream stream,
                                      hsa_event ev_begin, hsa_event ev_end) {
  using namespace hsa;
  if (!out) return HSA_ERR_NULL_ARG;
  if (n_workgroups < 1 || n_workgroups > 65536 || iters < 1 || iters > (1 << 20)) return HSA_ERR_BAD_PARAM;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (ev_begin && hipEventRecord(reinterpret_cast<hipEvent_t>(ev_begin), st) != hipSuccess) return HSA_ERR_HIP;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_workgroups), dim3(kProbeThreads), 0, st, out, iters, 1);
  if (ev_end && hipEventRecord(reinterpret_cast<hipEvent_t>(ev_end), st) != hipSuccess) return HSA_ERR_HIP;
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}

extern "C" hsa_rc hsa_probe_hbm_copy(const void* src, void* dst, size_t bytes, hsa_stream stream, hsa_event ev_begin,
                                     hsa_event ev_end) {
  using namespace hsa;
  if (!src || !dst) return HSA_ERR_NULL_ARG;
  if (bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
    return HSA_ERR_BAD_PARAM;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (ev_begin && hipEventRecord(reinterpret_cast<hipEvent_t>(ev_begin), st) != hipSuccess) return HSA_ERR_HIP;
  hipLaunchKernelGGL(copy_probe_kernel, dim3(kCopyGroups), dim3(kCopyThreads), 0, st,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), bytes / 16);
  if (ev_end && hipEventRecord(reinterpret_cast<hipEvent_t>(ev_end), st) != hipSuccess) return HSA_ERR_HIP;
  return hipGetLastError() == hipSuccess ? HSA_OK : HSA_ERR_HIP;
}
