// qg_common.h -- device helpers shared by the matvec (M = 1) and the small-M
// MFMA kernels: fp16 bit helpers, the staging geometry and permuted fp16
// staging of x, activation loads, the per-chunk power-of-two range scale,
// buffer descriptors over one matrix, and small wave utilities.
#pragma once

#include "qg_internal.h"

namespace qg {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t v) {
  return (float)__builtin_bit_cast(_Float16, v);
}

constexpr int kMaxLdsBytes = 64 * 1024;

// Per-format staging geometry: codes per 16-byte chunk, 16-byte pieces of
// staged x per chunk, chunks per group of 64.
template <int BITS, int FMT>
struct Geo;
template <>
struct Geo<4, 0> {  // 32 codes; x as 16 fp16 pairs = 4 pieces
  static constexpr int kPerChunk = 32, kPieces = 4, kChunksPerGroup = 2;
};
template <>
struct Geo<2, 0> {  // 64 codes; x as 32 fp16 pairs = 8 pieces
  static constexpr int kPerChunk = 64, kPieces = 8, kChunksPerGroup = 1;
};
template <>
struct Geo<4, 1> {  // LUT: 32 codes; x as 16 fp16 pairs in natural order = 4 pieces
  static constexpr int kPerChunk = 32, kPieces = 4, kChunksPerGroup = 2;
};
template <>
struct Geo<8, 0> {  // 16 codes; x as 8 fp16 pairs = 2 pieces
  static constexpr int kPerChunk = 16, kPieces = 2, kChunksPerGroup = 4;
};
template <>
struct Geo<16, 2> {  // dense fp16: 8 weights; x as 4 fp16 pairs = 1 piece (no groups)
  static constexpr int kPerChunk = 8, kPieces = 1, kChunksPerGroup = 8;
};

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const uint32_t a = __builtin_bit_cast(uint16_t, (_Float16)lo);
  const uint32_t b = __builtin_bit_cast(uint16_t, (_Float16)hi);
  return a | (b << 16);
}

// Writes the staged pieces of one chunk: v holds the chunk's x already
// multiplied by the range scale.
template <int BITS, int FMT>
__device__ __forceinline__ void write_pieces(const float* v, u32x4* dst, int stride) {
  if constexpr (FMT == 1) {
    // table format: piece p holds the pairs (x[8p+2b], x[8p+2b+1]), b = 0..3,
    // matching byte b of code word p (codes 2b and 2b+1)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float* w = v + 8 * p;
      dst[p * stride] = u32x4{pack_f16(w[0], w[1]), pack_f16(w[2], w[3]), pack_f16(w[4], w[5]),
                              pack_f16(w[6], w[7])};
    }
  } else if constexpr (FMT == 2) {
    // dense fp16: word i holds weights (2i, 2i+1)
    dst[0] = u32x4{pack_f16(v[0], v[1]), pack_f16(v[2], v[3]), pack_f16(v[4], v[5]),
                   pack_f16(v[6], v[7])};
  } else if constexpr (BITS == 8) {
    // word i holds codes 4i..4i+3; mask 0x00FF00FF takes fields (0, 2), the
    // same mask after a shift by 8 takes fields (1, 3)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float* w = v + 8 * p;
      dst[p * stride] = u32x4{pack_f16(w[0], w[2]), pack_f16(w[1], w[3]), pack_f16(w[4], w[6]),
                              pack_f16(w[5], w[7])};
    }
  } else if constexpr (BITS == 4) {
    constexpr float r16 = 1.0f / 16.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* w = v + 8 * i;
      dst[i * stride] = u32x4{pack_f16(w[0], w[4]), pack_f16(w[1] * r16, w[5] * r16),
                              pack_f16(w[2], w[6]), pack_f16(w[3] * r16, w[7] * r16)};
    }
  } else {
    constexpr float r4 = 0.25f, r16 = 1.0f / 16.0f, r64 = 1.0f / 64.0f, r256 = 1.0f / 256.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* w = v + 16 * i;
      dst[(2 * i) * stride] = u32x4{pack_f16(w[0], w[8]), pack_f16(w[1] * r4, w[9] * r4),
                                    pack_f16(w[2] * r16, w[10] * r16),
                                    pack_f16(w[3] * r64, w[11] * r64)};
      dst[(2 * i + 1) * stride] = u32x4{pack_f16(w[4] * r256, w[12] * r256), pack_f16(w[5], w[13]),
                                        pack_f16(w[6] * r4, w[14] * r4),
                                        pack_f16(w[7] * r16, w[15] * r16)};
    }
  }
}

// Loads n consecutive activations starting at element k0 as fp32.
template <int n>
__device__ __forceinline__ void load_x(const void* x, int x_f32, int k0, float* v) {
  if (x_f32) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + k0);
#pragma unroll
    for (int i = 0; i < n / 4; ++i) {
      const float4 t = src[i];
      v[4 * i] = t.x;
      v[4 * i + 1] = t.y;
      v[4 * i + 2] = t.z;
      v[4 * i + 3] = t.w;
    }
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + k0);
#pragma unroll
    for (int i = 0; i < n / 8; ++i) {
      const uint4 t = src[i];
      const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2 h = as_f16x2(w[j]);
        v[8 * i + 2 * j] = (float)h.x;
        v[8 * i + 2 * j + 1] = (float)h.y;
      }
    }
  }
}

template <int n>
__device__ __forceinline__ void load_f16(const uint16_t* src16, int k0, float* v) {
  const uint4* src = reinterpret_cast<const uint4*>(src16 + k0);
#pragma unroll
  for (int i = 0; i < n / 8; ++i) {
    const uint4 t = src[i];
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x2 h = as_f16x2(w[j]);
      v[8 * i + 2 * j] = (float)h.x;
      v[8 * i + 2 * j + 1] = (float)h.y;
    }
  }
}

// Power-of-two range scale for the fp16 staging of one chunk: with m = max|x|
// over the chunk, x * 2^-e stays below 2^14; returns 2^-e and sets
// *back = 2^(24+e), which also undoes the 2^-24 of the subnormal codes.
__device__ __forceinline__ float range_scale(float m, float* back) {
  int E = 0;
  if (m > 0.f && m < INFINITY) frexpf(m, &E);
  const int e = (m > 0.f && m < INFINITY) ? E - 14 : 0;
  *back = ldexpf(1.0f, 24 + e);
  return ldexpf(1.0f, -e);
}

// Per-chunk staging record next to the staged x: the chunk's sum of x (for
// the bias term), the factor 2^(24+e) that undoes the chunk's range scale and
// the subnormal code scale, and the chunk's sum of squares of the raw x (for
// the RMSNorm).
struct ChunkInfo {
  float xsum, back, ss, pad;
};

// ---------------------------------------------------------------------------
// Loads through buffer descriptors. A descriptor covers one matrix (or one
// expert's rows); loads at offsets past its end return zero without touching
// memory, which handles the last band's missing rows, padding chunks and the
// prefetch past the last item without branches.

constexpr uint32_t kOOB = 0x80000000u;  // an offset past every descriptor's end

struct MatRsrc {
  __amdgpu_buffer_rsrc_t q, s, b, l;  // codes, scales, biases, tables
};

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(p)), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// ---------------------------------------------------------------------------
// Hand-off between workgroups of one launch (split-K partials, top-k
// candidates) without cache-wide maintenance. A device-scope fence on gfx950
// writes back and invalidates the whole L2 of the issuing XCD, so every other
// workgroup there fetches its activations again; a split launch slowed down
// about threefold that way. Instead the data goes through agent-coherent
// (sc1) stores and loads, every wave waits for its own stores to complete
// before the workgroup barrier, and one thread then takes the ticket with a
// relaxed device-scope atomic.
template <typename T>
__device__ __forceinline__ void handoff_store(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Agent-coherent (sc1) reads as ordinary buffer loads. (Relaxed atomic loads
// compile to the same instruction, but the compiler waits for each one before
// issuing the next, which serializes a reduction over many partials at a full
// memory latency per term; these are issued back to back.)
__device__ __forceinline__ float coherent_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 16));
}
__device__ __forceinline__ uint64_t coherent_u64(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 16);
  return ((uint64_t)v[1] << 32) | (uint64_t)v[0];
}
// sum over s < n of the floats at byte offsets off0 + s * stride, added in s
// order, four loads in flight at a time (offsets past n read nothing).
__device__ __forceinline__ float coherent_sum(__amdgpu_buffer_rsrc_t r, uint32_t off0, uint32_t stride,
                                              int n) {
  float t = 0.f;
  for (int s0 = 0; s0 < n; s0 += 4) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = coherent_f32(r, s0 + u < n ? off0 + (uint32_t)(s0 + u) * stride : kOOB);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + u < n) t += v[u];
  }
  return t;
}
__device__ __forceinline__ uint32_t take_ticket(uint32_t* t) {
  return __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Descriptors for `rows` rows of matrix M (codes, scales, biases, tables;
// an absent array gets an empty descriptor).
__device__ __forceinline__ MatRsrc mat_rsrc(const QMat& M, int rows, int wpr, int gpr) {
  MatRsrc r;
  r.q = make_rsrc(M.q, (uint32_t)rows * (uint32_t)wpr * 4u);
  r.s = make_rsrc(M.s ? (const void*)M.s : (const void*)M.q, M.s ? (uint32_t)rows * (uint32_t)gpr * 2u : 0u);
  r.b = make_rsrc(M.b ? (const void*)M.b : (const void*)M.q, M.b ? (uint32_t)rows * (uint32_t)gpr * 2u : 0u);
  r.l = make_rsrc(M.lut ? (const void*)M.lut : (const void*)M.q, M.lut ? (uint32_t)rows * 32u : 0u);
  return r;
}

// Descriptors over nothing: every access reads zero.
__device__ __forceinline__ MatRsrc empty_rsrc(const MvParams& p) {
  MatRsrc r;
  r.q = r.s = r.b = r.l = make_rsrc(p.y, 0u);
  return r;
}

// Makes every workgroup fetch the launch parameters it needs first in one
// round of scalar loads. Without it the compiler sinks part of them below the
// first data-dependent branch, and a second dependent round trip to the
// argument buffer (a scalar-cache miss, ~0.6 us) precedes the first weight load.
__device__ __forceinline__ void params_now(const MvParams& p) {
  asm volatile("" ::"s"(p.N), "s"(p.K), "s"(p.M), "s"(p.wpr), "s"(p.gpr), "s"(p.grid_x),
               "s"(p.splits), "s"(p.slice_chunks), "s"(p.x_f32), "s"(p.nseg), "s"(p.seg_mode),
               "s"(p.seg_len), "s"(p.eps), "s"((uint64_t)p.x), "s"((uint64_t)p.norm_w),
               "s"((uint64_t)p.y), "s"((uint64_t)p.residual), "s"((uint64_t)p.A[0].q),
               "s"((uint64_t)p.A[0].s), "s"((uint64_t)p.A[0].b), "s"((uint64_t)p.A[0].lut),
               "s"((uint64_t)p.B[0].q), "s"((uint64_t)p.B[0].s), "s"((uint64_t)p.B[0].b),
               "s"((uint64_t)p.B[0].lut), "s"((uint64_t)p.partials), "s"((uint64_t)p.tickets));
}

// A unique 64-bit key per (value, index) that sorts as: larger value first,
// equal values by lower index, -0 equal to +0, NaN below every number.
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

// The value a key was made from (-0 comes back as +0, NaN as a NaN): the
// inverse of the sign-dependent bit flip in order_key.
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t hi = (uint32_t)(key >> 32);
  return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) {
  return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull);
}

// Router, run by one whole wave: ids = the top_k (<= kMaxRoutes) logits in
// the order above, w = softmax over the chosen logits only. Each lane keeps
// its own top_k keys (sorted, in registers) over batches of loads issued
// together; the wave then takes the largest head top_k times. Lane 0 returns
// the result in ids / w (registers).
__device__ __forceinline__ void route_wave(const float* __restrict__ logits, int E, int top_k,
                                           int32_t* ids, float* w) {
  constexpr int B = 8;  // loads per lane per batch
  const int l = threadIdx.x & 63;
  uint64_t mine[kMaxRoutes];
#pragma unroll
  for (int r = 0; r < kMaxRoutes; ++r) mine[r] = 0ull;
  for (int base = 0; base < E; base += 64 * B) {
    float v[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = base + l + 64 * j;
      v[j] = i < E ? logits[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = base + l + 64 * j;
      uint64_t key = i < E ? order_key(v[j], (uint32_t)i) : 0ull;
#pragma unroll
      for (int r = 0; r < kMaxRoutes; ++r) {  // insert into the lane's descending list
        const uint64_t cur = mine[r];
        const bool take = key > cur;
        mine[r] = take ? key : cur;
        key = take ? cur : key;
      }
    }
  }
  uint64_t chosen[kMaxRoutes];
#pragma unroll
  for (int r = 0; r < kMaxRoutes; ++r) {
    chosen[r] = 0ull;
    if (r < top_k) {
      uint64_t best = mine[0];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(best, off);
        if (o > best) best = o;
      }
      chosen[r] = best;
      if (mine[0] == best) {  // keys are unique: exactly one lane pops its head
#pragma unroll
        for (int q = 0; q + 1 < kMaxRoutes; ++q) mine[q] = mine[q + 1];
        mine[kMaxRoutes - 1] = 0ull;
      }
    }
  }
  float lv[kMaxRoutes];
  float lmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < kMaxRoutes; ++r) {
    lv[r] = r < top_k ? key_value(chosen[r]) : -INFINITY;  // no second trip to memory
    lmax = fmaxf(lmax, lv[r]);
  }
  float den = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxRoutes; ++r)
    if (r < top_k) den += expf(lv[r] - lmax);
#pragma unroll
  for (int r = 0; r < kMaxRoutes; ++r) {
    ids[r] = r < top_k ? (int32_t)key_index(chosen[r]) : 0;
    w[r] = r < top_k ? expf(lv[r] - lmax) / den : 0.f;
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// Sorting 64 keys held one per lane. The partner of a compare-exchange is
// reached through DPP and the gfx950 lane-swap instructions, in registers; a
// shuffle through the LDS crossbar (ds_bpermute) costs an LDS round trip per
// step (measured: merging 64 lists that way in one wave took ~24 us).

// the value held by lane (lane ^ S), S = 1, 2, ..., 32
template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const uint32_t l = threadIdx.x & 63;
  if constexpr (S == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  } else if constexpr (S == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  } else if constexpr (S == 4) {
    // row_ror:4 brings lane - 4, row_ror:12 lane + 4 (within rows of 16)
    const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false);
    const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x12C, 0xF, 0xF, false);
    return (l & 4) ? dn : up;
  } else if constexpr (S == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (S == 16) {
    // odd rows of the first operand trade places with even rows of the second
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (l & 16) ? r[0] : r[1];
  } else {
    static_assert(S == 32, "lane strides 1..32");
    // upper half of the first operand trades places with lower half of the second
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (l & 32) ? r[0] : r[1];
  }
}

template <int S>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
  return ((uint64_t)xor_lane<S>((uint32_t)(v >> 32)) << 32) | (uint64_t)xor_lane<S>((uint32_t)v);
}

// One compare-exchange at lane stride S over a run of sorted direction
// `desc`: each lane keeps its own key or its partner's, the larger one when
// it is the lower lane of a descending run (or the upper of an ascending).
template <int S>
__device__ __forceinline__ uint64_t cmp_xchg(uint64_t v, bool desc) {
  const uint64_t o = xor_lane64<S>(v);
  const bool keep_larger = (((threadIdx.x & 63) & S) == 0) == desc;
  return ((v > o) == keep_larger) ? v : o;  // keys are distinct: v == o never happens
}

// A bitonic sequence over the wave, sorted larger first (half-cleaners at
// strides 32 down to 1).
__device__ __forceinline__ uint64_t bitonic_clean_desc(uint64_t v) {
  v = cmp_xchg<32>(v, true);
  v = cmp_xchg<16>(v, true);
  v = cmp_xchg<8>(v, true);
  v = cmp_xchg<4>(v, true);
  v = cmp_xchg<2>(v, true);
  return cmp_xchg<1>(v, true);
}

// Bitonic sort of the wave's 64 keys, larger first (lane 0 ends with the
// largest): runs of 2, 4, ..., 32 sorted in alternating directions (the
// direction of a lane's run of length m is bit m of its lane number), each
// pair of runs then forming one bitonic run of twice the length.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
  const uint32_t l = threadIdx.x & 63;
  v = cmp_xchg<1>(v, (l & 2) == 0);
  v = cmp_xchg<2>(v, (l & 4) == 0);
  v = cmp_xchg<1>(v, (l & 4) == 0);
  v = cmp_xchg<4>(v, (l & 8) == 0);
  v = cmp_xchg<2>(v, (l & 8) == 0);
  v = cmp_xchg<1>(v, (l & 8) == 0);
  v = cmp_xchg<8>(v, (l & 16) == 0);
  v = cmp_xchg<4>(v, (l & 16) == 0);
  v = cmp_xchg<2>(v, (l & 16) == 0);
  v = cmp_xchg<1>(v, (l & 16) == 0);
  v = cmp_xchg<16>(v, (l & 32) == 0);
  v = cmp_xchg<8>(v, (l & 32) == 0);
  v = cmp_xchg<4>(v, (l & 32) == 0);
  v = cmp_xchg<2>(v, (l & 32) == 0);
  v = cmp_xchg<1>(v, (l & 32) == 0);
  return bitonic_clean_desc(v);
}

// The 64 largest of two lists of distinct keys, sorted larger first: `a`
// sorted larger first, `b_rev` smaller first (a list read back in reverse
// lane order). The lane-wise larger of the two is the upper half of the
// union as a bitonic sequence.
__device__ __forceinline__ uint64_t wave_merge_top(uint64_t a, uint64_t b_rev) {
  return bitonic_clean_desc(a > b_rev ? a : b_rev);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// The draw. The page names the step, not its rule; the reading used:
// temperature 0 is greedy (the first candidate); otherwise the weights
// w_i = exp((v_i - v_0) / T) of the k candidates in order (v_0 the largest),
// the shortest prefix whose weight sum reaches top_p of the total (at least
// one candidate), and the first candidate whose running sum exceeds u times
// that prefix sum. u is the top 53 bits of output number `counter` of the
// SplitMix64 generator started at `seed` (Steele, Lea and Flood, "Fast
// splittable pseudorandom number generators", OOPSLA 2014: the state advances
// by the golden-ratio increment and each output is the state through two
// xor-shift-multiply rounds and a final xor-shift). Double precision; the
// lanes compute the weights, one lane forms the sums in index order, so the
// choice is that of a plain sequential evaluation (the device exp may differ
// from another library's in the last bit, which can only matter when u lands
// within a few ulps of a boundary).

__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t counter) {
  uint64_t z = seed + (counter + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Called by all 64 lanes of one wave. val(i), id(i): candidate i of k
// (larger first). w: LDS scratch for k doubles. Every call consumes one draw
// number (also the greedy ones), so a captured graph replayed n times draws
// n successive numbers.
template <class Val, class Id>
__device__ void draw_token(int k, Val val, Id id, const DrawParams& dp, double* w) {
  const int lane = threadIdx.x & 63;
  const bool greedy = dp.temperature == 0.f;
  if (!greedy) {
    const double T = (double)dp.temperature;
    const double v0 = (double)val(0);
    for (int i = lane; i < k; i += 64) w[i] = exp(((double)val(i) - v0) / T);
  }
  wave_sync_lds();
  if (lane == 0) {
    const uint64_t c = dp.counter ? *dp.counter : 0ull;
    int pick = 0;
    if (!greedy) {
      const double u = (double)(splitmix64_at(dp.seed, c) >> 11) * 0x1.0p-53;
      double total = 0.0;
      for (int i = 0; i < k; ++i) total += w[i];
      const double cut = (double)dp.top_p * total;
      int m = 0;
      double prefix = 0.0;
      while (m < k) {
        prefix += w[m];
        ++m;
        if (prefix >= cut) break;
      }
      const double target = u * prefix;
      double run = 0.0;
      pick = m - 1;
      for (int i = 0; i < m; ++i) {
        run += w[i];
        if (run > target) {
          pick = i;
          break;
        }
      }
    }
    *dp.token = id(pick);
    if (dp.counter) *dp.counter = c + 1ull;
  }
}


}  // namespace
}  // namespace qg
