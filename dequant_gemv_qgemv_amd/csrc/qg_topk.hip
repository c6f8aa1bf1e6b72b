// qg_topk.hip -- exact top-k of the logits on the GPU (page "Booster la
// vitesse d'inference sur Apple Silicon", section 1: logits matvec + top-k on
// the GPU so that only the chosen entries come back). The MoE router's top-k
// (route_wave, qg_common.h) uses the same key order.
//
// Order: larger value first; equal values by lower index; -0 equals +0; NaN is
// below every number. Each (value, index) becomes one unique 64-bit key that
// sorts in exactly that order, so "the k largest keys" is a set with no ties
// and the result cannot depend on scheduling.
//
// Two phases in one launch: every workgroup finds the k largest keys of its
// slice (radix select on 8-bit digits with per-wave LDS histograms, stopping
// once a digit bin holds exactly the keys still wanted) and writes them to the
// workspace; the last workgroup to finish (integer ticket) repeats the
// selection over all candidates and sorts the k winners, and can then draw the
// token from them (same page and section: top-k sampling on the GPU, only the
// token comes back).
#include "qg_common.h"

namespace qg {
namespace {

// Slices of 4096 keys: measured on MI355X for the 151936 x 1024 logits +
// top-40 (matvec 18.0 us of it), 8192-key slices with 8 candidates per thread
// in the last workgroup 40.5 us, 4096 / 2 35.7 us, 2048 / 4 36.1 us,
// 1024 / 4 38.7 us: the selection is bound by its chain of barriers and
// memory round trips, and shorter slices shorten the first phase until the
// last workgroup's candidate list grows too long.
constexpr int kTkThreads = 1024;
constexpr int kTkPer = 4;  // keys per thread in the slice phase
constexpr int kTkSlice = kTkThreads * kTkPer;
constexpr int kFinPer = 2;  // candidate keys per thread held in registers by the last workgroup
constexpr int kFinKeys = kTkThreads * kFinPer;
constexpr int kTkMaxK = 1024;

constexpr int kTkWaves = kTkThreads / 64;

struct SelectShared {
  uint32_t hist[kTkWaves][256];  // one histogram per wave (fewer colliding atomics)
  uint32_t tot[256];             // their sum
  uint64_t list[kTkMaxK];
  uint32_t digit, rem, count, done;
  int last;
};
static_assert(sizeof(SelectShared::hist) >= kTkMaxK * sizeof(double), "the draw reuses the histograms");

// Bitwise AND and OR of all nonzero keys of the block (for the common prefix).
template <class ForEach>
__device__ void and_or(ForEach for_each, SelectShared& sh, uint64_t* a_out, uint64_t* o_out) {
  uint64_t a = ~0ull, o = 0ull;
  for_each([&](uint64_t key) {
    if (key) {
      a &= key;
      o |= key;
    }
  });
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a &= __shfl_xor(a, off);
    o |= __shfl_xor(o, off);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh.list[2 * wave] = a;
    sh.list[2 * wave + 1] = o;
  }
  __syncthreads();
  a = ~0ull;
  o = 0ull;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    a &= sh.list[2 * w];
    o |= sh.list[2 * w + 1];
  }
  __syncthreads();
  *a_out = a;
  *o_out = o;
}

// Adds 1 to bin d of this wave's histogram for every active lane: lanes that
// share the digit of the wave's first active lane are counted with one atomic
// (two rounds), the rest individually; keeps same-address collisions low when
// the keys crowd into a few bins.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool active, uint32_t d) {
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const uint64_t act = __ballot(active);
    if (act == 0ull) return;
    const int leader = __builtin_ctzll(act);
    const uint32_t ld = __shfl(d, leader);
    const bool same = active && d == ld;
    const uint64_t m = __ballot(same);
    if ((int)(threadIdx.x & 63) == leader) atomicAdd(&hist[ld], (uint32_t)__builtin_popcountll(m));
    active = active && !same;
  }
  if (active) atomicAdd(&hist[d], 1u);
}

// The kk-th largest of the nonzero keys visited by for_each (1 <= kk <= their
// count, keys unique), or a smaller key t such that exactly kk keys are >= t:
// radix select from the highest bit where the keys differ, in windows of up to
// 8 bits, stopping as soon as the chosen digit's bin holds exactly the keys
// still wanted (every key with that prefix is then in). Called by all
// kTkThreads threads of the block.
template <class ForEach>
__device__ uint64_t kth_largest(ForEach for_each, uint32_t kk, SelectShared& sh) {
  const int wave = threadIdx.x >> 6;
  uint64_t all_and, all_or;
  and_or(for_each, sh, &all_and, &all_or);
  const uint64_t diff = all_and ^ all_or;
  if (diff == 0ull) return all_and;  // a single key
  int top = 63 - __builtin_clzll(diff);  // highest bit where keys differ
  uint64_t mask = top == 63 ? 0ull : ~0ull << (top + 1);
  uint64_t prefix = all_and & mask;  // the bits every key shares
  uint32_t remaining = kk;
  while (top >= 0) {
    const int lo = top >= 7 ? top - 7 : 0;
    const uint64_t wmask = ((1ull << (top - lo + 1)) - 1ull) << lo;
#pragma unroll
    for (int j = 0; j < kTkWaves * 256 / kTkThreads; ++j)
      (&sh.hist[0][0])[threadIdx.x + j * kTkThreads] = 0u;
    __syncthreads();
    for_each([&](uint64_t key) {
      hist_add(sh.hist[wave], key != 0ull && (key & mask) == prefix, (uint32_t)((key & wmask) >> lo));
    });
    __syncthreads();
    if (threadIdx.x < 256) {
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < kTkWaves; ++w) t += sh.hist[w][threadIdx.x];
      sh.tot[threadIdx.x] = t;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int l = threadIdx.x;  // lane l owns bins 255-4l .. 252-4l
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = sh.tot[255 - 4 * l - q];
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
            sh.done = (c[q] == remaining - cum);  // the whole bin is wanted
            break;
          }
          cum += c[q];
        }
      }
    }
    __syncthreads();
    prefix |= (uint64_t)sh.digit << lo;
    mask |= wmask;
    remaining = sh.rem;
    const bool done = sh.done;
    __syncthreads();
    if (done) break;
    top = lo - 1;
  }
  return prefix;
}

// Collects the keys >= thr (exactly kk of them) into sh.list[0..kk), in no
// particular order.
template <class ForEach>
__device__ void gather(ForEach for_each, uint64_t thr, SelectShared& sh) {
  if (threadIdx.x == 0) sh.count = 0u;
  __syncthreads();
  for_each([&](uint64_t key) {
    if (key >= thr) sh.list[atomicAdd(&sh.count, 1u)] = key;
  });
  __syncthreads();
}

// Sorts sh.list[0..kk) descending (entries kk..pow2 are set to zero first):
// one wave with shuffles for kk <= 64, else a block bitonic network.
__device__ void sort_desc(uint32_t kk, SelectShared& sh) {
  if (kk <= 64) {
    if (threadIdx.x < 64) {
      const uint32_t l = threadIdx.x;
      uint64_t v = l < kk ? sh.list[l] : 0ull;
      for (uint32_t size = 2; size <= 64; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
          const uint64_t o = __shfl_xor(v, stride);
          const bool up = (l & stride) == 0;          // lower index of the pair
          const bool desc = (l & size) == 0 || size == 64;
          const uint64_t hi = v > o ? v : o, lo = v > o ? o : v;
          v = (up == desc) ? hi : lo;
        }
      }
      if (l < kk) sh.list[l] = v;
    }
    __syncthreads();
    return;
  }
  uint32_t p2 = 1;
  while (p2 < kk) p2 <<= 1;
  for (uint32_t i = kk + threadIdx.x; i < p2; i += blockDim.x) sh.list[i] = 0ull;
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

__global__ __launch_bounds__(64) void sample_kernel(const int32_t* __restrict__ idx,
                                                    const float* __restrict__ vals, int k,
                                                    DrawParams dp) {
  __shared__ double w[kTkMaxK];
  draw_token(
      k, [&](int i) { return vals[i]; }, [&](int i) { return idx[i]; }, dp, w);
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float* __restrict__ z, int V, int k,
                                                          uint64_t* cand, uint32_t* ticket,
                                                          int32_t* idx, float* vals,
                                                          DrawParams dp) {
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
  // this slice's k largest (fewer if the slice is shorter), unsorted
  const uint32_t kk = (uint32_t)min(k, n);
  const uint64_t thr = kth_largest(regs, kk, sh);
  gather(regs, thr, sh);
  for (int r = threadIdx.x; r < k; r += kTkThreads)
    handoff_store(&cand[(size_t)b * k + r], r < (int)kk ? sh.list[r] : (uint64_t)0);

  // every thread's candidate stores are complete before the barrier; one
  // thread then takes the ticket
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) sh.last = take_ticket(ticket) == gridDim.x - 1;
  __syncthreads();
  if (!sh.last) return;

  // the last workgroup: the k largest of all candidates (held in registers
  // when they fit), sorted
  const int total = gridDim.x * k;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(cand, (uint32_t)total * 8u);
  if (total <= kFinKeys) {
    uint64_t ck[kFinPer];
#pragma unroll
    for (int j = 0; j < kFinPer; ++j) {
      const int i = threadIdx.x + j * kTkThreads;
      ck[j] = coherent_u64(rc, i < total ? (uint32_t)i * 8u : kOOB);
    }
    auto cregs = [&](auto&& f) {
#pragma unroll
      for (int j = 0; j < kFinPer; ++j) f(ck[j]);
    };
    const uint64_t thr2 = kth_largest(cregs, (uint32_t)k, sh);
    gather(cregs, thr2, sh);
  } else {
    auto all = [&](auto&& f) {
      for (int i = threadIdx.x; i < total; i += kTkThreads) f(coherent_u64(rc, (uint32_t)i * 8u));
    };
    const uint64_t thr2 = kth_largest(all, (uint32_t)k, sh);
    gather(all, thr2, sh);
  }
  sort_desc((uint32_t)k, sh);
  for (int r = threadIdx.x; r < k; r += kTkThreads) {
    const uint32_t i = key_index(sh.list[r]);
    idx[r] = (int32_t)i;
    vals[r] = z[i];
  }
  if (threadIdx.x == 0) handoff_store(ticket, 0u);
  if (dp.token) {
    __syncthreads();  // the histograms are free: they hold the draw's weights
    if (threadIdx.x < 64)
      draw_token(
          k, [&](int i) { return key_value(sh.list[i]); },  // the logit, without a trip to memory
          [&](int i) { return (int32_t)key_index(sh.list[i]); }, dp,
          reinterpret_cast<double*>(&sh.hist[0][0]));
  }
}

}  // namespace

size_t topk_workspace_bytes(int V, int k) {
  const size_t G = ((size_t)V + kTkSlice - 1) / kTkSlice;
  const size_t two = ((G * (size_t)k * 8 + 255) / 256) * 256;  // slice lists of the top-k kernel
  // workgroup and group lists of the fused form (at most kTkMaxGroups groups)
  const size_t fused = (size_t)(kTkMaxGroups * kTkGroup + kTkMaxGroups) * kTkList * 8;
  return kTkTicketBytes + (two > fused ? two : fused);
}

int plan_and_launch_topk(const float* logits, int V, int k, int32_t* idx, float* vals, void* ws,
                         size_t ws_bytes, const DrawParams& dp, hipStream_t stream) {
  if (ws_bytes < topk_workspace_bytes(V, k)) return -3;
  const int G = (V + kTkSlice - 1) / kTkSlice;
  uint32_t* ticket = static_cast<uint32_t*>(ws);
  uint64_t* cand = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + kTkTicketBytes);
  hipLaunchKernelGGL(topk_kernel, dim3(G), dim3(kTkThreads), 0, stream, logits, V, k, cand,
                     ticket, idx, vals, dp);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

hipError_t launch_sample(const int32_t* idx, const float* vals, int k, const DrawParams& dp,
                         hipStream_t stream) {
  hipLaunchKernelGGL(sample_kernel, dim3(1), dim3(64), 0, stream, idx, vals, k, dp);
  return hipGetLastError();
}

}  // namespace qg
