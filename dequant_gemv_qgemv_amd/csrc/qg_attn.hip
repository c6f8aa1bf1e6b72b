// qg_attn.hip -- decode attention against a KV cache for gfx950 (page
// "Booster la vitesse d'inference sur Apple Silicon", section 2 "KV cache":
// the cache is preallocated at its maximum length, coalesced along the time
// axis per head ([head][seq][d] per layer), fp16; a dedicated decode kernel
// serves one query and splits the cache along time for long contexts; GQA
// shares one kv head among several query heads).
//
// What is computed, for query head h (kv head g = h / G, G = H / Hkv) over
// positions t = 0..n-1 (n = pos + 1):
//   s_t = scale * q[h] . K[g][t],   out[h] = sum_t softmax(s)_t V[g][t].
// When new k/v rows are given they are first written (rounded to fp16) at
// position pos of every kv head.
//
// Work mapping. One workgroup (4 waves) per (kv head, slice of positions);
// it serves all G query heads of its kv head, so every K/V row is read once.
// A lane holds 8 of the d dimensions of one position (d/8 lanes per
// position, 64/(d/8) positions per wave step), the G query rows for those
// dimensions, and per head a running (max, sum, 8 accumulators) of the
// online softmax over the positions its slot has seen. Scores are summed
// across the d/8 lanes with shuffles. At the end the position slots of a
// wave, then the waves (through LDS), then the slices (through the
// workspace: the last workgroup of a kv head takes an integer ticket and
// adds the slices in slice order) are merged with the usual rescaling:
//   m = max(m1, m2), l = l1 2^(m1-m) + l2 2^(m2-m), acc likewise.
// Scores are kept in base 2 (q pre-multiplied by scale * log2 e). K/V rows
// are loaded two steps ahead through buffer descriptors that end at the
// slice's last position, so the tail needs no branch around a load.
#include "qg_common.h"

namespace qg {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr float kNeg = -3.0e38f;  // "no position yet": finite, so empty merges stay 0 * 1
// Slices: about kAttnTargetGroups workgroups over all kv heads, at most
// kAttnMaxSlices per kv head, each at least kAttnMinPositions positions long.
constexpr int kAttnTargetGroups = 256;
constexpr int kAttnMaxSlices = 256;
constexpr int kAttnMinPositions = 128;

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Sum over aligned groups of N lanes (8 or 16), every lane of the group
// getting the same bits: quad swaps, then the mirror within 8 and within 16.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<0xb1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4e>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror: lanes of each 8 see the other quad
  if constexpr (N == 16) v += dpp_f<0x140>(v);  // row_mirror: the other half of the row
  return v;
}

// 2^x for x <= 0 (the softmax weights): the hardware exp2, whose results
// below the normal range flush to zero.
__device__ __forceinline__ float exp2_neg(float x) { return __builtin_amdgcn_exp2f(x); }

template <int G>
struct Slot {
  float m[G], l[G], acc[G][8];
};

// Merges the partner's (m, l, acc) into ours.
template <int G>
__device__ __forceinline__ void merge(Slot<G>& a, const float* m2, const float* l2, const float (*acc2)[8]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = fmaxf(a.m[h], m2[h]);
    const float ca = exp2_neg(a.m[h] - M), cb = exp2_neg(m2[h] - M);
    a.l[h] = a.l[h] * ca + l2[h] * cb;
#pragma unroll
    for (int i = 0; i < 8; ++i) a.acc[h][i] = a.acc[h][i] * ca + acc2[h][i] * cb;
    a.m[h] = M;
  }
}

__device__ __forceinline__ void unpack8(const u32x4 w, float* f) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = as_f16x2(v[i]);
    f[2 * i] = (float)h.x;
    f[2 * i + 1] = (float)h.y;
  }
}

struct AttnParams {
  const float* q;       // [H][d]
  const float* k_new;   // [Hkv][d] or nullptr
  const float* v_new;
  uint16_t* k_cache;    // [Hkv][T_max][d]
  uint16_t* v_cache;
  int H, Hkv, T_max, pos, n;
  int per_slice;        // positions per workgroup
  int nslice;
  float scale_log2;     // scale * log2(e)
  float* out;           // [H][d]
  float* partials;      // [Hkv][nslice][G][2 + d] when nslice > 1
  uint32_t* tickets;    // [Hkv]
};

template <int G, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(const AttnParams p) {
  constexpr int LPP = D / 8;         // lanes per position
  constexpr int PPW = 64 / LPP;      // positions per wave step
  constexpr int STEP = PPW * kAttnWaves;
  __shared__ float red_m[kAttnWaves][G], red_l[kAttnWaves][G];
  __shared__ float red_acc[kAttnWaves][G][D];
  __shared__ float sl_m[kAttnMaxSlices * G], sl_l[kAttnMaxSlices * G], tot_l[G];
  __shared__ int last_flag;

  const int g = blockIdx.x / p.nslice;
  const int slice = blockIdx.x - g * p.nslice;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int slot = lane / LPP;
  const int j0 = (lane % LPP) * 8;
  const int t0 = slice * p.per_slice;
  const int t1 = min(p.n, t0 + p.per_slice);

  uint16_t* kg = p.k_cache + (size_t)g * p.T_max * D;
  uint16_t* vg = p.v_cache + (size_t)g * p.T_max * D;

  // the new row goes into the cache first (only the slice that holds it)
  if (p.k_new && p.pos >= t0 && p.pos < t1) {
    for (int j = threadIdx.x; j < D; j += kAttnThreads) {
      kg[(size_t)p.pos * D + j] = __builtin_bit_cast(uint16_t, (_Float16)p.k_new[(size_t)g * D + j]);
      vg[(size_t)p.pos * D + j] = __builtin_bit_cast(uint16_t, (_Float16)p.v_new[(size_t)g * D + j]);
    }
    stores_done();
  }
  __syncthreads();

  // q rows of the G heads for this lane's dimensions, in base-2 score units
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float4* src = reinterpret_cast<const float4*>(p.q + (size_t)(g * G + h) * D + j0);
    const float4 a = src[0], b = src[1];
    qv[h][0] = a.x * p.scale_log2; qv[h][1] = a.y * p.scale_log2;
    qv[h][2] = a.z * p.scale_log2; qv[h][3] = a.w * p.scale_log2;
    qv[h][4] = b.x * p.scale_log2; qv[h][5] = b.y * p.scale_log2;
    qv[h][6] = b.z * p.scale_log2; qv[h][7] = b.w * p.scale_log2;
  }

  // rows [t0, t1) of this kv head; loads past t1 return zeros
  const uint32_t row_bytes = (uint32_t)D * 2u;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)t0 * D, (uint32_t)max(t1 - t0, 0) * row_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)t0 * D, (uint32_t)max(t1 - t0, 0) * row_bytes);
  const int nsteps = (t1 - t0 + STEP - 1) / STEP;
  const int my0 = wave * PPW + slot;  // this lane's position within a step
  auto off = [&](int step) -> uint32_t {
    return (uint32_t)(step * STEP + my0) * row_bytes + (uint32_t)j0 * 2u;
  };

  Slot<G> s;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s.m[h] = kNeg;
    s.l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s.acc[h][i] = 0.f;
  }

  // Two steps in flight. Every load sits at a fixed place in one sequence
  // (prologue and loop issue in the same order) so the waits before each use
  // count exactly the loads issued after it.
  u32x4 kb[2], vb[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    kb[b] = __builtin_amdgcn_raw_buffer_load_b128(rk, off(b), 0, 0);
    asm volatile("" ::: "memory");
    vb[b] = __builtin_amdgcn_raw_buffer_load_b128(rv, off(b), 0, 0);
    asm volatile("" ::: "memory");
  }
  for (int st = 0; st < nsteps; st += 2) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int step = st + b;
      const bool valid = step * STEP + my0 < t1 - t0;
      float kf[8], vf[8];
      // this step's rows are used from here on, not earlier (their wait then
      // leaves the loads issued since in flight)
      asm volatile("" : "+v"(kb[b]), "+v"(vb[b]));
      unpack8(kb[b], kf);
      unpack8(vb[b], vf);
      // the rows are converted before their registers take the next load (a
      // conversion folded into later arithmetic would keep them live, and the
      // loop would then wait for the new loads to copy them around)
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(kf[i]), "+v"(vf[i]));
      kb[b] = __builtin_amdgcn_raw_buffer_load_b128(rk, off(step + 2), 0, 0);
      asm volatile("" ::: "memory");
      vb[b] = __builtin_amdgcn_raw_buffer_load_b128(rv, off(step + 2), 0, 0);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float sc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sc = fmaf(qv[h][i], kf[i], sc);
        sc = group_sum<LPP>(sc);
        const float M = valid ? fmaxf(s.m[h], sc) : s.m[h];
        const float c = exp2_neg(s.m[h] - M);
        const float e = valid ? exp2_neg(sc - M) : 0.f;
        s.l[h] = s.l[h] * c + e;
#pragma unroll
        for (int i = 0; i < 8; ++i) s.acc[h][i] = fmaf(e, vf[i], s.acc[h][i] * c);
        s.m[h] = M;
      }
    }
  }

  // merge the position slots of the wave (lanes with the same dimensions)
#pragma unroll
  for (int msk = LPP; msk < 64; msk <<= 1) {
    float m2[G], l2[G], a2[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m2[h] = shfl_xor_f(s.m[h], msk);
      l2[h] = shfl_xor_f(s.l[h], msk);
#pragma unroll
      for (int i = 0; i < 8; ++i) a2[h][i] = shfl_xor_f(s.acc[h][i], msk);
    }
    merge<G>(s, m2, l2, a2);
  }
  // then the waves, through LDS (lanes 0..LPP-1 hold the wave's result)
  if (lane < LPP) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (lane == 0) {
        red_m[wave][h] = s.m[h];
        red_l[wave][h] = s.l[h];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) red_acc[wave][h][j0 + i] = s.acc[h][i];
    }
  }
  __syncthreads();
  // thread (h, j) forms the workgroup's result for head h, dimension j
  for (int e = threadIdx.x; e < G * D; e += kAttnThreads) {
    const int h = e / D, j = e % D;
    float M = kNeg;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, red_m[w][h]);
    float l = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float c = exp2_neg(red_m[w][h] - M);
      l = fmaf(red_l[w][h], c, l);
      a = fmaf(red_acc[w][h][j], c, a);
    }
    if (p.nslice == 1) {
      p.out[(size_t)(g * G + h) * D + j] = a / l;
    } else {
      float* part = p.partials + (((size_t)g * p.nslice + slice) * G + h) * (2 + D);
      if (j == 0) {
        handoff_store(&part[0], M);
        handoff_store(&part[1], l);
      }
      handoff_store(&part[2 + j], a);
    }
  }
  if (p.nslice == 1) return;

  // the last slice of this kv head to finish adds the slices in order
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) last_flag = take_ticket(&p.tickets[g]) == (uint32_t)(p.nslice - 1);
  __syncthreads();
  if (!last_flag) return;
  const size_t rec = 2 + D;  // floats per (slice, head) record
  const __amdgpu_buffer_rsrc_t rp =
      make_rsrc(p.partials + (size_t)g * p.nslice * G * rec, (uint32_t)(p.nslice * G * rec * 4));
  // every slice's (max, sum) into LDS; each head's overall max, the slice
  // weights 2^(m - max) and the weighted sum, in slice order
  for (int e = threadIdx.x; e < p.nslice * G; e += kAttnThreads) {
    sl_m[e] = coherent_f32(rp, (uint32_t)(e * rec * 4));
    sl_l[e] = coherent_f32(rp, (uint32_t)((e * rec + 1) * 4));
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = kNeg;
    for (int sl = 0; sl < p.nslice; ++sl) M = fmaxf(M, sl_m[sl * G + h]);
    float l = 0.f;
    for (int sl = 0; sl < p.nslice; ++sl) {
      const float w = exp2_neg(sl_m[sl * G + h] - M);
      sl_m[sl * G + h] = w;
      l = fmaf(sl_l[sl * G + h], w, l);
    }
    tot_l[h] = l;
  }
  __syncthreads();
  // element (h, j): the weighted sum of the slices' accumulators, sixteen
  // loads in flight at a time
  for (int e = threadIdx.x; e < G * D; e += kAttnThreads) {
    const int h = e / D, j = e % D;
    float a = 0.f;
    for (int sl0 = 0; sl0 < p.nslice; sl0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int sl = min(sl0 + u, p.nslice - 1);
        v[u] = coherent_f32(rp, (uint32_t)(((sl * G + h) * rec + 2 + j) * 4));
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (sl0 + u < p.nslice) a = fmaf(sl_m[(sl0 + u) * G + h], v[u], a);
    }
    p.out[(size_t)(g * G + h) * D + j] = a / tot_l[h];
  }
  if (threadIdx.x == 0) handoff_store(&p.tickets[g], 0u);
}

template <int D>
hipError_t launch_d(int G, const AttnParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.Hkv * p.nslice)), block(kAttnThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL((attn_kernel<1, D>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((attn_kernel<2, D>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((attn_kernel<4, D>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((attn_kernel<8, D>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int attn_max_slices(int Hkv) { return min((kAttnTargetGroups + Hkv - 1) / Hkv, kAttnMaxSlices); }

size_t attn_ws_bytes(int H, int Hkv, int d) {
  const size_t tickets = ((size_t)Hkv * 4 + 255) / 256 * 256;
  return tickets + (size_t)Hkv * attn_max_slices(Hkv) * (size_t)(H / Hkv) * (2 + d) * 4;
}

hipError_t launch_attn(const float* q, const float* k_new, const float* v_new, uint16_t* k_cache,
                       uint16_t* v_cache, int H, int Hkv, int d, int T_max, int pos, float scale,
                       float* out, void* ws, hipStream_t stream) {
  AttnParams p;
  p.q = q;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.H = H;
  p.Hkv = Hkv;
  p.T_max = T_max;
  p.pos = pos;
  p.n = pos + 1;
  const int max_slices = attn_max_slices(Hkv);
  int per = (p.n + max_slices - 1) / max_slices;
  per = max(per, kAttnMinPositions);
  per = (per + 63) / 64 * 64;  // whole steps of the wave loop
  p.per_slice = per;
  p.nslice = (p.n + per - 1) / per;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.out = out;
  p.tickets = static_cast<uint32_t*>(ws);
  p.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + ((size_t)Hkv * 4 + 255) / 256 * 256);
  const int G = H / Hkv;
  if (d == 128) return launch_d<128>(G, p, stream);
  if (d == 64) return launch_d<64>(G, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace qg
