// qg_probe.hip -- HBM bandwidth probes used to put the matvec numbers in
// context: a streaming read (each byte read once, one fp32 written per
// thread) and a streaming copy, both with 16-byte accesses and several loads in
// flight per thread.
#include "../../include/qgemv.h"
#include "qg_internal.h"

namespace qg {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 4;

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                                   size_t n16, uint32_t* out) {
  const size_t tid = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = NT ? __builtin_nontemporal_load(src + i) : src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[tid] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(u32x4* __restrict__ dst,
                                                                   const u32x4* __restrict__ src,
                                                                   size_t n16) {
  const size_t tid = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = tid;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace
}  // namespace qg

extern "C" {

int qg_probe_read(const void* src, size_t bytes, uint32_t* out, int blocks, int flags,
                  hipStream_t stream) {
  if (!src || !out || bytes % 16 || ((uintptr_t)src % 16) || blocks < 1 || blocks > 65536 ||
      (flags & ~1))
    return QG_EINVAL;
  if (flags & 1)
    hipLaunchKernelGGL(qg::probe_read_kernel<false>, dim3(blocks), dim3(qg::kProbeThreads), 0,
                       stream, static_cast<const qg::u32x4*>(src), bytes / 16, out);
  else
    hipLaunchKernelGGL(qg::probe_read_kernel<true>, dim3(blocks), dim3(qg::kProbeThreads), 0,
                       stream, static_cast<const qg::u32x4*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ELAUNCH;
}

int qg_probe_copy(void* dst, const void* src, size_t bytes, int blocks, hipStream_t stream) {
  if (!src || !dst || bytes % 16 || ((uintptr_t)src % 16) || ((uintptr_t)dst % 16) || blocks < 1 ||
      blocks > 65536)
    return QG_EINVAL;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return QG_EINVAL;
  hipLaunchKernelGGL(qg::probe_copy_kernel, dim3(blocks), dim3(qg::kProbeThreads), 0, stream,
                     static_cast<qg::u32x4*>(dst), static_cast<const qg::u32x4*>(src), bytes / 16);
  return hipGetLastError() == hipSuccess ? QG_OK : QG_ELAUNCH;
}

}  // extern "C"
