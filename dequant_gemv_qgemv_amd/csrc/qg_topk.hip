// qg_topk.hip -- exact top-k of the logits on the GPU (page "Booster la
// vitesse d'inference sur Apple Silicon", section 1: logits matvec + top-k on
// the GPU so that only the chosen entries come back), and the MoE router's
// top-k + softmax (GeekNews item on the 397B MoE engine, "Architecture du
// modele": a few experts of 512 per token).
//
// Order: larger value first; equal values by lower index; -0 equals +0; NaN is
// below every number. Each (value, index) becomes one unique 64-bit key that
// sorts in exactly that order, so "the k largest keys" is a set with no ties
// and the result cannot depend on scheduling.
//
// Two phases in one launch: every workgroup finds the k largest keys of its
// slice (radix select on 8-bit digits with LDS histograms, then a bitonic sort
// of the k survivors) and writes them to the workspace; the last workgroup to
// finish (integer ticket) repeats the selection over all candidates.
#include "qg_internal.h"

namespace qg {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkPer = 8;  // keys per thread in the slice phase
constexpr int kTkSlice = kTkThreads * kTkPer;
constexpr int kTkMaxK = 1024;

__device__ __forceinline__ uint64_t order_key(float v, uint32_t i) {
  uint32_t u;
  if (v != v) {
    u = 0u;  // NaN sorts below every number
  } else {
    if (v == 0.0f) v = 0.0f;  // -0 and +0 are the same value
    u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - i);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) {
  return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull);
}

struct SelectShared {
  uint32_t hist[256];
  uint64_t list[kTkMaxK];
  uint32_t digit, rem, count;
  int last;
};

// The kk-th largest of the keys visited by for_each (kk >= 1, keys unique).
template <class ForEach>
__device__ uint64_t kth_largest(ForEach for_each, uint32_t kk, SelectShared& sh) {
  uint64_t prefix = 0, mask = 0;
  uint32_t remaining = kk;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) sh.hist[i] = 0u;
    __syncthreads();
    for_each([&](uint64_t key) {
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (threadIdx.x < 64) {
      const int l = threadIdx.x;  // lane l owns bins 255-4l .. 252-4l
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = sh.hist[255 - 4 * l - q];
        tot += c[q];
      }
      uint32_t inc = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(inc, off);
        if (l >= off) inc += t;
      }
      const uint32_t excl = inc - tot;
      if (excl < remaining && remaining <= inc) {
        uint32_t cum = excl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cum + c[q] >= remaining) {
            sh.digit = 255 - 4 * l - q;
            sh.rem = remaining - cum;
            break;
          }
          cum += c[q];
        }
      }
    }
    __syncthreads();
    prefix |= (uint64_t)sh.digit << shift;
    mask |= (uint64_t)255 << shift;
    remaining = sh.rem;
    __syncthreads();
  }
  return prefix;
}

// Collects the keys >= thr (exactly kk of them) into sh.list[0..kk) sorted
// descending; entries [kk, pow2) are zero.
template <class ForEach>
__device__ void gather_sorted(ForEach for_each, uint64_t thr, uint32_t kk, SelectShared& sh) {
  uint32_t p2 = 1;
  while (p2 < kk) p2 <<= 1;
  for (uint32_t i = threadIdx.x; i < p2; i += blockDim.x) sh.list[i] = 0ull;
  if (threadIdx.x == 0) sh.count = 0u;
  __syncthreads();
  for_each([&](uint64_t key) {
    if (key >= thr) sh.list[atomicAdd(&sh.count, 1u)] = key;
  });
  __syncthreads();
  for (uint32_t size = 2; size <= p2; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t i = threadIdx.x; i < p2; i += blockDim.x) {
        const uint32_t j = i ^ stride;
        if (j > i) {
          const uint64_t a = sh.list[i], b = sh.list[j];
          const bool desc = (i & size) == 0;
          if (desc ? (a < b) : (a > b)) {
            sh.list[i] = b;
            sh.list[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float* __restrict__ z, int V, int k,
                                                          uint64_t* cand, uint32_t* ticket,
                                                          int32_t* idx, float* vals) {
  __shared__ SelectShared sh;
  const int b = blockIdx.x;
  const int base = b * kTkSlice;
  const int n = min(kTkSlice, V - base);
  uint64_t keys[kTkPer];
#pragma unroll
  for (int j = 0; j < kTkPer; ++j) {
    const int i = threadIdx.x + j * kTkThreads;
    keys[j] = i < n ? order_key(z[base + i], (uint32_t)(base + i)) : 0ull;
  }
  auto regs = [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) f(keys[j]);
  };
  const uint32_t kk = (uint32_t)min(k, n);
  const uint64_t thr = kth_largest(regs, kk, sh);
  gather_sorted(regs, thr, kk, sh);
  for (int r = threadIdx.x; r < k; r += kTkThreads)
    cand[(size_t)b * k + r] = r < (int)kk ? sh.list[r] : 0ull;

  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) sh.last = atomicAdd(ticket, 1u) == gridDim.x - 1;
  __syncthreads();
  if (!sh.last) return;
  __threadfence();

  const int total = gridDim.x * k;
  auto all = [&](auto&& f) {
    for (int i = threadIdx.x; i < total; i += kTkThreads) f(__builtin_nontemporal_load(&cand[i]));
  };
  const uint64_t thr2 = kth_largest(all, (uint32_t)k, sh);
  gather_sorted(all, thr2, (uint32_t)k, sh);
  for (int r = threadIdx.x; r < k; r += kTkThreads) {
    const uint32_t i = key_index(sh.list[r]);
    idx[r] = (int32_t)i;
    vals[r] = z[i];
  }
  if (threadIdx.x == 0) *ticket = 0u;
}

// Router: one wave. ids = top_k of the logits (order above), w = softmax over
// the chosen logits only.
__global__ __launch_bounds__(64) void route_kernel(const float* __restrict__ logits, int E,
                                                   int top_k, int32_t* ids_ws, float* w_ws,
                                                   int32_t* ids_out, float* w_out) {
  const int l = threadIdx.x;
  uint64_t chosen[kMaxRoutes];
#pragma unroll
  for (int r = 0; r < kMaxRoutes; ++r) {
    chosen[r] = 0ull;
    if (r < top_k) {
      uint64_t best = 0ull;
      for (int i = l; i < E; i += 64) {
        const uint64_t key = order_key(logits[i], (uint32_t)i);
        bool taken = false;
#pragma unroll
        for (int q = 0; q < r; ++q) taken |= (chosen[q] == key);
        if (!taken && key > best) best = key;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(best, off);
        if (o > best) best = o;
      }
      chosen[r] = best;
    }
  }
  if (l == 0) {
    float lv[kMaxRoutes];
    float lmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < kMaxRoutes; ++r) {
      lv[r] = r < top_k ? logits[key_index(chosen[r])] : -INFINITY;
      lmax = fmaxf(lmax, lv[r]);
    }
    float den = 0.f;
#pragma unroll
    for (int r = 0; r < kMaxRoutes; ++r)
      if (r < top_k) den += expf(lv[r] - lmax);
#pragma unroll
    for (int r = 0; r < kMaxRoutes; ++r) {
      if (r < top_k) {
        const int32_t id = (int32_t)key_index(chosen[r]);
        const float w = expf(lv[r] - lmax) / den;
        ids_ws[r] = id;
        w_ws[r] = w;
        if (ids_out) ids_out[r] = id;
        if (w_out) w_out[r] = w;
      }
    }
  }
}

}  // namespace

size_t topk_workspace_bytes(int V, int k) {
  const size_t G = ((size_t)V + kTkSlice - 1) / kTkSlice;
  return 256 + ((G * (size_t)k * 8 + 255) / 256) * 256;
}

int plan_and_launch_topk(const float* logits, int V, int k, int32_t* idx, float* vals, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (ws_bytes < topk_workspace_bytes(V, k)) return -3;
  const int G = (V + kTkSlice - 1) / kTkSlice;
  uint32_t* ticket = static_cast<uint32_t*>(ws);
  uint64_t* cand = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + 256);
  hipLaunchKernelGGL(topk_kernel, dim3(G), dim3(kTkThreads), 0, stream, logits, V, k, cand,
                     ticket, idx, vals);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

hipError_t launch_route(const float* logits, int E, int top_k, int32_t* ids_ws, float* w_ws,
                        int32_t* ids_out, float* w_out, hipStream_t stream) {
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(64), 0, stream, logits, E, top_k, ids_ws, w_ws,
                     ids_out, w_out);
  return hipGetLastError();
}

}  // namespace qg
