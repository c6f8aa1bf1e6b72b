// qg_probe.hip -- HBM bandwidth probes used to put the matvec numbers in
// context: a streaming read (each byte read once, one fp32 written per
// thread) and a streaming copy, both with 16-byte accesses and several loads in
// flight per thread.
#include "../../include/qgemv.h"
#include "qg_internal.h"
#include "qg_common.h"

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

// Phase probe: one launch reads several byte ranges of src in order, as a
// persistent whole-token kernel would stream a token's matvecs, optionally
// with a device-wide barrier between ranges (such a kernel needs one, since
// each matvec's x is the previous matvec's output). Against one launch per
// range it prices the launch boundary and the barrier on the same bytes.
// The barrier: each workgroup publishes one agent-coherent word (standing in
// for its outputs), waits for that store, raises its flag to the phase
// number, and wave 0 polls every flag until all have reached it. The poll is
// bounded: past spin_limit rounds the workgroup counts an error and stops.
// Mode 2 issues each thread's first loads of the next range before the wait
// (a matvec's weights do not depend on the barrier, only its x does), so the
// memory pipe has work while the workgroup waits.
constexpr int kPhaseThreads = 512;
constexpr int kPhaseMaxBlocks = 1024;  // with the barrier

__global__ __launch_bounds__(kPhaseThreads) void probe_phases_kernel(
    const u32x4* __restrict__ src, size_t src16, const uint64_t* __restrict__ ranges, int nphases,
    int barrier, uint32_t* flags, uint32_t* out, uint32_t* err, int spin_limit) {
  __shared__ int stop;
  const int G = gridDim.x, g = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t tid = (size_t)g * kPhaseThreads + threadIdx.x;
  const size_t stride = (size_t)G * kPhaseThreads;
  if (threadIdx.x == 0) stop = 0;
  uint32_t acc = 0;
  u32x4 pre[kUnroll];  // mode 2: the next range's first loads
  bool have_pre = false;
  // a range past the end of src is clipped to it
  auto range_of = [&](int q, size_t* n16) {
    const size_t off16 = min((size_t)(ranges[2 * q] / 16), src16);
    *n16 = min((size_t)(ranges[2 * q + 1] / 16), src16 - off16);
    return src + off16;
  };
  for (int q = 0; q < nphases; ++q) {
    size_t n16;
    const u32x4* const base = range_of(q, &n16);
    size_t i = tid;
    if (have_pre) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= pre[u].x ^ pre[u].y ^ pre[u].z ^ pre[u].w;
      i = tid + kUnroll * stride;
      have_pre = false;
    }
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(base + i + u * stride);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
      const u32x4 v = __builtin_nontemporal_load(base + i);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (!barrier || q + 1 == nphases) continue;
    auto prefetch = [&]() {
      if (barrier != 2) return;
      size_t nn;
      const u32x4* const nb = range_of(q + 1, &nn);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const size_t j = tid + u * stride;
        pre[u] = j < nn ? __builtin_nontemporal_load(nb + j) : u32x4{0u, 0u, 0u, 0u};
      }
      have_pre = true;
    };
    // wave 0 issues its loads after raising its flag (its wait for its own
    // stores would wait for them too)
    if (wave != 0) prefetch();
    __syncthreads();
    if (wave == 0) {
      if (lane == 0) handoff_store(&out[(size_t)g * kPhaseThreads], acc);
      stores_done();
      const uint32_t want = (uint32_t)(q + 1);
      if (lane == 0) handoff_store(&flags[g], want);
      prefetch();
      const __amdgpu_buffer_rsrc_t rf = make_rsrc(flags, (uint32_t)G * 4u);
      for (int spins = 0;; ++spins) {
        asm volatile("" ::: "memory");  // a fresh read of the flags every round
        uint32_t v[kPhaseMaxBlocks / 64];  // agent-coherent loads, all in flight together
#pragma unroll
        for (int u = 0; u < kPhaseMaxBlocks / 64; ++u) {
          const int f = lane + u * 64;
          v[u] = __builtin_amdgcn_raw_buffer_load_b32(rf, f < G ? (uint32_t)f * 4u : kOOB, 0, 16);
        }
        bool late = false;
#pragma unroll
        for (int u = 0; u < kPhaseMaxBlocks / 64; ++u) late |= (lane + u * 64 < G) && v[u] < want;
        if (__builtin_amdgcn_ballot_w64(late) == 0) break;
        if (spins >= spin_limit) {
          if (lane == 0) {
            stop = 1;
            atomicAdd(err, 1u);
          }
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
    if (stop) break;
  }
  out[tid] = acc;
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

int qg_probe_phases(const void* src, size_t src_bytes, const uint64_t* ranges, int nphases,
                    int barrier, uint32_t* flags, uint32_t* out, uint32_t* err, int blocks,
                    int spin_limit, hipStream_t stream) {
  if (!src || !ranges || !out || src_bytes % 16 || ((uintptr_t)src % 16) ||
      ((uintptr_t)ranges % 8) || nphases < 1 || nphases > 4096 || blocks < 1 || blocks > 65536 ||
      barrier < 0 || barrier > 2 || spin_limit < 1 || spin_limit > (1 << 22))
    return QG_EINVAL;
  if (barrier) {
    if (!flags || !err || ((uintptr_t)flags % 4)) return QG_EINVAL;
    // every workgroup must be resident at once for the barrier to complete
    int dev = 0, occ = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)qg::probe_phases_kernel,
                                                     qg::kPhaseThreads, 0) != hipSuccess)
      return QG_EDEVICE;
    if (blocks > occ * prop.multiProcessorCount || blocks > qg::kPhaseMaxBlocks) return QG_EUNSUPPORTED;
  }
  hipLaunchKernelGGL(qg::probe_phases_kernel, dim3(blocks), dim3(qg::kPhaseThreads), 0, stream,
                     static_cast<const qg::u32x4*>(src), src_bytes / 16, ranges, nphases, barrier,
                     flags, out, err, spin_limit);
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
