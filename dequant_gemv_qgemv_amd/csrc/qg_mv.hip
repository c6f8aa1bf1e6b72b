// qg_mv.hip -- the decode matrix-vector kernels for gfx950 (CDNA4).
//
// What is computed (page "Booster la vitesse d'inference sur Apple Silicon --
// avec le format .forge", section 1 and section 3 item 4; GeekNews item on the
// 397B MoE engine, "Noyau de dequantification optimise FMA"):
//   y[n] = sum_k W[n][k] x[k],  W[n][k] = code * scale + bias  (affine, group 64)
//                               W[n][k] = lut[n][code]         (LUT, 16 entries)
// with the weights dequantized inside the inner loop and never written out.
//
// The pages' rewrite fma(code, scale*x, bias*x) is applied at group level:
//   sum_{k in g} (c_k s + b) x_k = s * sum_{k in g} c_k x_k + b * sum_{k in g} x_k,
// so the per-weight work is one fused multiply-add of the code with x, and the
// scale and bias enter once per 16-byte chunk of codes.
//
// Work mapping (one workgroup = 8 wave64s):
//  * x (the slice of it this workgroup needs) is staged once in LDS as fp32,
//    permuted and pre-scaled by powers of two so that the codes can be used
//    straight out of the packed words (see below), plus one sum of x per chunk
//    for the bias term. Conflict-free layout: the float4 a lane reads for chunk
//    j of pass i, piece p sits at [i][p][j].
//  * Each wave owns a band of rows: 64/LPR sub-waves of LPR lanes, each lane
//    accumulating R rows. Lanes stride along K in 16-byte chunks (coalesced
//    dwordx4 loads of the row-major codes), two passes in flight at a time.
//  * Row sums are reduced across the LPR lanes with cross-lane shuffles.
//  * Optional split-K: workgroup (tile t, slice s) writes fp32 partials; the
//    last workgroup of tile t to finish (integer ticket, no float atomics)
//    adds the slices in fixed order and applies the epilogue, so results do
//    not depend on timing.
//
// Code extraction: masking a packed word with 0x000F000F leaves two fp16 bit
// patterns that are the subnormal numbers code*2^-24 exactly. v_fma_mix_f32
// multiplies such an fp16 operand with an fp32 x, so 8 codes of a word cost
// 1 shift + 4 masks + 8 mixed FMAs. Codes at odd nibble positions come out
// multiplied by 16 (mask 0x00F000F0); their x is pre-divided by 16 in LDS.
// 2-bit fields come out multiplied by 4^j; their x is pre-divided by 4^j.
#include "qg_internal.h"

namespace qg {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t v) {
  return (float)__builtin_bit_cast(_Float16, v);
}

constexpr float kTwo24 = 16777216.0f;   // 2^24: undoes the subnormal code scale
constexpr int kMaxLdsBytes = 64 * 1024;

template <int BITS>
struct Codes;
template <>
struct Codes<4> {
  static constexpr int kPerChunk = 32;       // codes in one 16-byte chunk
  static constexpr int kPieces = 8;          // float4 of staged x per chunk
  static constexpr int kChunksPerGroup = 2;  // a group of 64 spans two chunks
};
template <>
struct Codes<2> {
  static constexpr int kPerChunk = 64;
  static constexpr int kPieces = 16;
  static constexpr int kChunksPerGroup = 1;
};

// ---------------------------------------------------------------------------
// Inner products of one 16-byte chunk of codes with its staged x.

// 4-bit: returns 2^-24 * sum_k code_k x_k over the chunk's 32 codes.
__device__ __forceinline__ float dot_q4(const u32x4 q, const float4* xr) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = w[i] >> 8;
    const f16x2 h0 = as_f16x2(w[i] & 0x000F000Fu);  // fields 0, 4
    const f16x2 h1 = as_f16x2(w[i] & 0x00F000F0u);  // fields 1, 5 (times 16)
    const f16x2 h2 = as_f16x2(t & 0x000F000Fu);     // fields 2, 6
    const f16x2 h3 = as_f16x2(t & 0x00F000F0u);     // fields 3, 7 (times 16)
    const float4 u = xr[2 * i], v = xr[2 * i + 1];
    a0 = fmaf((float)h0.x, u.x, a0);
    a1 = fmaf((float)h0.y, u.y, a1);
    a0 = fmaf((float)h1.x, u.z, a0);
    a1 = fmaf((float)h1.y, u.w, a1);
    a0 = fmaf((float)h2.x, v.x, a0);
    a1 = fmaf((float)h2.y, v.y, a1);
    a0 = fmaf((float)h3.x, v.z, a0);
    a1 = fmaf((float)h3.y, v.w, a1);
  }
  return a0 + a1;
}

// 2-bit: returns 2^-24 * sum_k code_k x_k over the chunk's 64 codes.
__device__ __forceinline__ float dot_q2(const u32x4 q, const float4* xr) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = w[i] >> 10;
    const f16x2 h0 = as_f16x2(w[i] & 0x00030003u);  // fields 0, 8
    const f16x2 h1 = as_f16x2(w[i] & 0x000C000Cu);  // fields 1, 9   (x4)
    const f16x2 h2 = as_f16x2(w[i] & 0x00300030u);  // fields 2, 10  (x16)
    const f16x2 h3 = as_f16x2(w[i] & 0x00C000C0u);  // fields 3, 11  (x64)
    const f16x2 h4 = as_f16x2(w[i] & 0x03000300u);  // fields 4, 12  (x256)
    const f16x2 h5 = as_f16x2(t & 0x00030003u);     // fields 5, 13
    const f16x2 h6 = as_f16x2(t & 0x000C000Cu);     // fields 6, 14  (x4)
    const f16x2 h7 = as_f16x2(t & 0x00300030u);     // fields 7, 15  (x16)
    const float4 p0 = xr[4 * i], p1 = xr[4 * i + 1], p2 = xr[4 * i + 2], p3 = xr[4 * i + 3];
    a0 = fmaf((float)h0.x, p0.x, a0);
    a1 = fmaf((float)h0.y, p0.y, a1);
    a0 = fmaf((float)h1.x, p0.z, a0);
    a1 = fmaf((float)h1.y, p0.w, a1);
    a0 = fmaf((float)h2.x, p1.x, a0);
    a1 = fmaf((float)h2.y, p1.y, a1);
    a0 = fmaf((float)h3.x, p1.z, a0);
    a1 = fmaf((float)h3.y, p1.w, a1);
    a0 = fmaf((float)h4.x, p2.x, a0);
    a1 = fmaf((float)h4.y, p2.y, a1);
    a0 = fmaf((float)h5.x, p2.z, a0);
    a1 = fmaf((float)h5.y, p2.w, a1);
    a0 = fmaf((float)h6.x, p3.x, a0);
    a1 = fmaf((float)h6.y, p3.y, a1);
    a0 = fmaf((float)h7.x, p3.z, a0);
    a1 = fmaf((float)h7.y, p3.w, a1);
  }
  return a0 + a1;
}

// LUT (4-bit codes, 16-entry table per row, held in this wave's LDS slot):
// returns sum_k lut[code_k] x_k over the chunk's 32 codes (x in natural order).
__device__ __forceinline__ float dot_lut(const u32x4 q, const float4* xr, const float* tab) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 u = xr[2 * i], v = xr[2 * i + 1];
    a0 = fmaf(tab[(w[i] >> 0) & 15u], u.x, a0);
    a1 = fmaf(tab[(w[i] >> 4) & 15u], u.y, a1);
    a0 = fmaf(tab[(w[i] >> 8) & 15u], u.z, a0);
    a1 = fmaf(tab[(w[i] >> 12) & 15u], u.w, a1);
    a0 = fmaf(tab[(w[i] >> 16) & 15u], v.x, a0);
    a1 = fmaf(tab[(w[i] >> 20) & 15u], v.y, a1);
    a0 = fmaf(tab[(w[i] >> 24) & 15u], v.z, a0);
    a1 = fmaf(tab[(w[i] >> 28) & 15u], v.w, a1);
  }
  return a0 + a1;
}

// ---------------------------------------------------------------------------
// Staging of x into LDS.

// Writes the staged pieces of one chunk (codes-order permutation + power-of-two
// pre-scales matching the masks in dot_q4 / dot_q2; natural order for LUT).
template <int BITS, int FMT>
__device__ __forceinline__ void write_pieces(const float* v, float4* dst, int stride) {
  if constexpr (FMT == 1) {
#pragma unroll
    for (int p = 0; p < 8; ++p)
      dst[p * stride] = make_float4(v[4 * p], v[4 * p + 1], v[4 * p + 2], v[4 * p + 3]);
  } else if constexpr (BITS == 4) {
    constexpr float r16 = 1.0f / 16.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* w = v + 8 * i;
      dst[(2 * i) * stride] = make_float4(w[0], w[4], w[1] * r16, w[5] * r16);
      dst[(2 * i + 1) * stride] = make_float4(w[2], w[6], w[3] * r16, w[7] * r16);
    }
  } else {
    constexpr float r4 = 0.25f, r16 = 1.0f / 16.0f, r64 = 1.0f / 64.0f, r256 = 1.0f / 256.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* w = v + 16 * i;
      dst[(4 * i) * stride] = make_float4(w[0], w[8], w[1] * r4, w[9] * r4);
      dst[(4 * i + 1) * stride] = make_float4(w[2] * r16, w[10] * r16, w[3] * r64, w[11] * r64);
      dst[(4 * i + 2) * stride] = make_float4(w[4] * r256, w[12] * r256, w[5], w[13]);
      dst[(4 * i + 3) * stride] = make_float4(w[6] * r4, w[14] * r4, w[7] * r16, w[15] * r16);
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

// Block-wide sum (all threads receive it). `red` holds kWaves floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += red[w];  // fixed order: same value in every block
  return s;
}

// 1/sqrt(mean(x^2) + eps) over all K activations (each workgroup computes it
// itself, in the same order, so every workgroup gets the same value).
__device__ float rms_scale(const MvParams& p, float* red) {
  float ss = 0.f;
  const int K8 = p.K / 8;
  for (int i = threadIdx.x; i < K8; i += kThreads) {
    float v[8];
    load_x<8>(p.x, p.x_f32, 8 * i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
  }
  const float tot = block_sum(ss, red);
  return 1.0f / sqrtf(tot / (float)p.K + p.eps);
}

// Stages chunks [c0, c0 + nch) of x (padded with zeros up to npass*LPR chunks).
// For K segments with routing weights, chunk c of segment j is scaled by w_j.
template <int BITS, int FMT, int LPR>
__device__ void stage_x(const MvParams& p, int c0, int nch, int npass, float4* xl, float* xsum,
                        float* red) {
  constexpr int CPC = Codes<BITS>::kPerChunk;
  constexpr int PIECES = Codes<BITS>::kPieces;
  const float rs = p.norm_w ? rms_scale(p, red) : 1.0f;
  const int total = npass * LPR;
  for (int c = threadIdx.x; c < total; c += kThreads) {
    float v[CPC];
    float s = 0.f;
    if (c < nch) {
      const int cg = c0 + c;
      load_x<CPC>(p.x, p.x_f32, cg * CPC, v);
      if (p.norm_w) {
        float g[CPC];
        load_f16<CPC>(p.norm_w, cg * CPC, g);
#pragma unroll
        for (int i = 0; i < CPC; ++i) v[i] = v[i] * g[i] * rs;
      }
      if (p.seg_mode == kSegCols && p.route.weights) {
        const int seg = cg / p.seg_len;
        const float wseg = seg < p.route.n_routed ? p.route.weights[seg] : 1.0f;
#pragma unroll
        for (int i = 0; i < CPC; ++i) v[i] *= wseg;
      }
#pragma unroll
      for (int i = 0; i < CPC; ++i) s += v[i];
    } else {
#pragma unroll
      for (int i = 0; i < CPC; ++i) v[i] = 0.f;
    }
    const int pass = c / LPR, j = c % LPR;
    write_pieces<BITS, FMT>(v, xl + pass * PIECES * LPR + j, LPR);
    xsum[c] = s;
  }
}

// ---------------------------------------------------------------------------
// Per-pass loads through buffer descriptors. A descriptor covers one matrix
// (or one expert's rows); loads at offsets past its end return zero without
// touching memory, which handles the last band's missing rows, padding chunks
// and the prefetch past the last pass without branches.

constexpr uint32_t kOOB = 0x80000000u;  // an offset past every descriptor's end

struct MatRsrc {
  __amdgpu_buffer_rsrc_t q, s, b;
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

// Descriptors for `rows` rows of matrix M (codes, scales, biases).
__device__ __forceinline__ MatRsrc mat_rsrc(const QMat& M, int rows, int wpr, int gpr) {
  MatRsrc r;
  r.q = make_rsrc(M.q, (uint32_t)rows * (uint32_t)wpr * 4u);
  r.s = make_rsrc(M.s ? (const void*)M.s : (const void*)M.q, M.s ? (uint32_t)rows * (uint32_t)gpr * 2u : 0u);
  r.b = make_rsrc(M.b ? (const void*)M.b : (const void*)M.q, M.b ? (uint32_t)rows * (uint32_t)gpr * 2u : 0u);
  return r;
}

template <int R, bool TWO>
struct PassData {
  u32x4 qa[R];
  uint16_t sa[R], ba[R];
  u32x4 qb[TWO ? R : 1];
  uint16_t sb[TWO ? R : 1], bb[TWO ? R : 1];
};

// Loads one pass for the lane's R rows. qoff/soff are the byte offsets of the
// lane's chunk (codes) and group (scales/biases) in each row for this pass;
// ok = false turns the pass into zero loads that touch no memory.
template <int FMT, int R, bool TWO>
__device__ __forceinline__ void load_pass(const MatRsrc& ra, const MatRsrc& rb, const uint32_t* qoff,
                                          const uint32_t* soff, uint32_t dq, uint32_t ds, bool ok,
                                          PassData<R, TWO>& d) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t oq = ok ? qoff[r] + dq : kOOB;
    const uint32_t os = ok ? soff[r] + ds : kOOB;
    d.qa[r] = __builtin_amdgcn_raw_buffer_load_b128(ra.q, oq, 0, 2);
    if constexpr (FMT == 0) {
      d.sa[r] = __builtin_amdgcn_raw_buffer_load_b16(ra.s, os, 0, 0);
      d.ba[r] = __builtin_amdgcn_raw_buffer_load_b16(ra.b, os, 0, 0);
    }
    if constexpr (TWO) {
      d.qb[r] = __builtin_amdgcn_raw_buffer_load_b128(rb.q, oq, 0, 2);
      if constexpr (FMT == 0) {
        d.sb[r] = __builtin_amdgcn_raw_buffer_load_b16(rb.s, os, 0, 0);
        d.bb[r] = __builtin_amdgcn_raw_buffer_load_b16(rb.b, os, 0, 0);
      }
    }
  }
  // Keep the prefetch where it is: without this the compiler sinks the loads
  // next to their first use and the next pass no longer overlaps this one.
  asm volatile("" ::: "memory");
}

template <int BITS, int FMT, int LPR, int R, bool TWO>
__device__ __forceinline__ void compute_pass(const PassData<R, TWO>& d, const float4* xl,
                                             const float* xsum, int pass, int j,
                                             const float* tabs, float* acc_a, float* acc_b) {
  constexpr int PIECES = Codes<BITS>::kPieces;
  float4 xr[PIECES];
  const float4* src = xl + pass * PIECES * LPR + j;
#pragma unroll
  for (int i = 0; i < PIECES; ++i) xr[i] = src[i * LPR];
  if constexpr (FMT == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc_a[r] += dot_lut(d.qa[r], xr, tabs + (2 * r) * 16);
      if constexpr (TWO) acc_b[r] += dot_lut(d.qb[r], xr, tabs + (2 * r + 1) * 16);
    }
  } else {
    const float xs = xsum[pass * LPR + j];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float da = (BITS == 4 ? dot_q4(d.qa[r], xr) : dot_q2(d.qa[r], xr)) * kTwo24;
      acc_a[r] = fmaf(f16_bits_to_f32(d.sa[r]), da, acc_a[r]);
      acc_a[r] = fmaf(f16_bits_to_f32(d.ba[r]), xs, acc_a[r]);
      if constexpr (TWO) {
        const float db = (BITS == 4 ? dot_q4(d.qb[r], xr) : dot_q2(d.qb[r], xr)) * kTwo24;
        acc_b[r] = fmaf(f16_bits_to_f32(d.sb[r]), db, acc_b[r]);
        acc_b[r] = fmaf(f16_bits_to_f32(d.bb[r]), xs, acc_b[r]);
      }
    }
  }
}

template <int LPR>
__device__ __forceinline__ float lanes_sum(float v) {
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Segment tables resolved at kernel start (routing ids are device data).
struct SegTable {
  QMat A[kMaxSeg];
  QMat B[kMaxSeg];
  int rows[kMaxSeg];  // rows of each segment's matrix
};

// ---------------------------------------------------------------------------
template <int BITS, int FMT, int LPR, int R, int EPI, int SEG>
__global__ __launch_bounds__(kThreads) void qmv_kernel(const MvParams p) {
  constexpr int PIECES = Codes<BITS>::kPieces;
  constexpr int CPC = Codes<BITS>::kPerChunk;
  constexpr int SUB = 64 / LPR;
  constexpr int RPB = SUB * R;  // rows per band
  constexpr bool TWO = (EPI == kEpiSwiglu);
  constexpr int NACC = TWO ? 2 : 1;

  extern __shared__ float4 smem[];
  __shared__ float red[kWaves];
  __shared__ SegTable st;
  __shared__ int last_flag;

  const int slice = blockIdx.x / p.grid_x;
  const int tile = blockIdx.x - slice * p.grid_x;
  const int C = p.K / CPC;
  const int c0 = slice * p.slice_chunks;
  const int nch = min(p.slice_chunks, C - c0);
  const int npass = (nch + LPR - 1) / LPR;
  const int nbands = (p.N + RPB - 1) / RPB;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int j = lane % LPR;
  const int first_band = tile * kWaves;
  if (first_band >= nbands) return;  // same for every slice of this tile: no ticket needed

  if constexpr (SEG != kSegNone) {
    if (threadIdx.x < p.nseg) {
      const int i = threadIdx.x;
      QMat a = p.A[i], b = p.B[i];
      int rows = (SEG == kSegRows) ? p.seg_len : p.N;
      if (p.route.ids && i < p.route.n_routed) {
        const size_t e = (size_t)p.route.ids[i];
        const size_t r0 = e * (size_t)p.route.expert_rows;
        a.q = p.route.all_A.q + r0 * p.wpr;
        a.s = p.route.all_A.s ? p.route.all_A.s + r0 * p.gpr : nullptr;
        a.b = p.route.all_A.b ? p.route.all_A.b + r0 * p.gpr : nullptr;
        a.lut = p.route.all_A.lut ? p.route.all_A.lut + r0 * 16 : nullptr;
        b.q = p.route.all_B.q ? p.route.all_B.q + r0 * p.wpr : nullptr;
        b.s = p.route.all_B.s ? p.route.all_B.s + r0 * p.gpr : nullptr;
        b.b = p.route.all_B.b ? p.route.all_B.b + r0 * p.gpr : nullptr;
        b.lut = p.route.all_B.lut ? p.route.all_B.lut + r0 * 16 : nullptr;
        rows = p.route.expert_rows;
      }
      st.A[i] = a;
      st.B[i] = b;
      st.rows[i] = rows;
    }
  }

  float4* xl = smem;
  float* xsum = reinterpret_cast<float*>(smem + (size_t)npass * LPR * PIECES);
  float* tabs_all = xsum + npass * LPR;  // LUT: [kWaves][SUB][R][2][16]
  stage_x<BITS, FMT, LPR>(p, c0, nch, npass, xl, xsum, red);
  __syncthreads();

  float* tabs = tabs_all + (wave * SUB + sub) * R * 2 * 16;
  const int band_stride = p.grid_x * kWaves;

  MatRsrc ra{}, rb{};
  if constexpr (SEG == kSegNone) {
    ra = mat_rsrc(p.A[0], p.N, p.wpr, p.gpr);
    if constexpr (TWO) rb = mat_rsrc(p.B[0], p.N, p.wpr, p.gpr);
  }

  for (int band = first_band + wave; band < nbands; band += band_stride) {
    // rows of this lane (logical) and their offsets inside their matrix
    int seg_band = 0;
    if constexpr (SEG == kSegRows) {
      seg_band = (band * RPB) / p.seg_len;  // a band never straddles two segments
      ra = mat_rsrc(st.A[seg_band], st.rows[seg_band], p.wpr, p.gpr);
      if constexpr (TWO) rb = mat_rsrc(st.B[seg_band], st.rows[seg_band], p.wpr, p.gpr);
    }
    // byte offsets of this lane's first chunk / group in each of its rows
    constexpr int CPG = Codes<BITS>::kChunksPerGroup;
    uint32_t qoff[R], soff[R];
    int local_row[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = band * RPB + sub * R + r;
      const int lr = (SEG == kSegRows) ? n - seg_band * p.seg_len : n;
      local_row[r] = lr;
      const bool ok = n < p.N;
      // chunk of pass 0; K segments add their (segment-local) chunk per pass
      const uint32_t cfirst = (SEG == kSegCols) ? 0u : (uint32_t)(c0 + j);
      qoff[r] = ok ? (uint32_t)lr * (uint32_t)p.wpr * 4u + cfirst * 16u : kOOB;
      soff[r] = ok ? (uint32_t)lr * (uint32_t)p.gpr * 2u + (cfirst / CPG) * 2u : kOOB;
    }

    if constexpr (FMT == 1) {
      // this sub-wave's row tables: [R][2][16] floats
      wave_sync_lds();
      for (int e = j; e < R * NACC * 16; e += LPR) {
        const int r = e / (NACC * 16), m = (e / 16) % NACC, t = e % 16;
        const int n = band * RPB + sub * R + r;
        float val = 0.f;
        if (n < p.N) {
          const QMat M = (SEG == kSegRows) ? (m ? st.B[seg_band] : st.A[seg_band])
                                           : (m ? p.B[0] : p.A[0]);
          val = f16_bits_to_f32(M.lut[(size_t)local_row[r] * 16 + t]);
        }
        tabs[(2 * r + m) * 16 + t] = val;
      }
      wave_sync_lds();
    }

    float acc_a[R], acc_b[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc_a[r] = acc_b[r] = 0.f;

    // Issues the loads of pass i into d. For K segments, the descriptors of
    // the pass's segment are (re)built here; when a pass straddles segments
    // (segments shorter than LPR chunks) each segment gets its own load with
    // the other lanes pointed past the end, and the zero-filled results merge.
    auto issue = [&](int i, PassData<R, TWO>& d) {
      const bool ok = i < npass && i * LPR + j < nch;
      if constexpr (SEG == kSegCols) {
        const int cpass = c0 + i * LPR;
        const int s_lo = min(cpass / p.seg_len, p.nseg - 1);
        const int s_hi = min((cpass + LPR - 1) / p.seg_len, p.nseg - 1);
        const int cg = cpass + j;
        if (s_lo == s_hi) {
          ra = mat_rsrc(st.A[s_lo], st.rows[s_lo], p.wpr, p.gpr);
          const int cl = cg - s_lo * p.seg_len;
          load_pass<FMT, R, TWO>(ra, rb, qoff, soff, (uint32_t)cl * 16u,
                                 (uint32_t)(cl / CPG) * 2u, ok, d);
        } else {
          const int mine = cg / p.seg_len;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            d.qa[r] = u32x4{0u, 0u, 0u, 0u};
            d.sa[r] = d.ba[r] = 0;
          }
          for (int sg = s_lo; sg <= s_hi; ++sg) {
            PassData<R, TWO> t;
            ra = mat_rsrc(st.A[sg], st.rows[sg], p.wpr, p.gpr);
            const int cl = cg - sg * p.seg_len;
            load_pass<FMT, R, TWO>(ra, rb, qoff, soff, (uint32_t)cl * 16u,
                                   (uint32_t)(cl / CPG) * 2u, ok && mine == sg, t);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              d.qa[r] |= t.qa[r];
              d.sa[r] |= t.sa[r];
              d.ba[r] |= t.ba[r];
            }
          }
        }
      } else {
        load_pass<FMT, R, TWO>(ra, rb, qoff, soff, (uint32_t)(i * LPR) * 16u,
                               (uint32_t)(i * LPR / CPG) * 2u, ok, d);
      }
    };

    PassData<R, TWO> d0, d1;
    issue(0, d0);
    for (int i = 0; i < npass; i += 2) {
      issue(i + 1, d1);
      compute_pass<BITS, FMT, LPR, R, TWO>(d0, xl, xsum, i, j, tabs, acc_a, acc_b);
      issue(i + 2, d0);
      if (i + 1 < npass) compute_pass<BITS, FMT, LPR, R, TWO>(d1, xl, xsum, i + 1, j, tabs, acc_a, acc_b);
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc_a[r] = lanes_sum<LPR>(acc_a[r]);
      if constexpr (TWO) acc_b[r] = lanes_sum<LPR>(acc_b[r]);
    }
    if (j == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = band * RPB + sub * R + r;
        if (n >= p.N) continue;
        if (p.splits > 1) {
          p.partials[((size_t)slice * NACC) * p.N + n] = acc_a[r];
          if constexpr (TWO) p.partials[((size_t)slice * NACC + 1) * p.N + n] = acc_b[r];
        } else if constexpr (TWO) {
          p.y[n] = silu(acc_a[r]) * acc_b[r];
        } else {
          p.y[n] = p.residual ? p.residual[n] + acc_a[r] : acc_a[r];
        }
      }
    }
  }

  if (p.splits > 1) {
    // Last workgroup of this tile adds the slices in fixed order.
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t prev = atomicAdd(&p.tickets[tile], 1u);
      last_flag = (prev == (uint32_t)(p.splits - 1));
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    for (int band = first_band + wave; band < nbands; band += band_stride) {
      if (lane < RPB) {
        const int n = band * RPB + lane;
        if (n < p.N) {
          float a = 0.f, b = 0.f;
          for (int s = 0; s < p.splits; ++s) {
            a += __builtin_nontemporal_load(&p.partials[((size_t)s * NACC) * p.N + n]);
            if constexpr (TWO) b += __builtin_nontemporal_load(&p.partials[((size_t)s * NACC + 1) * p.N + n]);
          }
          if constexpr (TWO) {
            p.y[n] = silu(a) * b;
          } else {
            p.y[n] = p.residual ? p.residual[n] + a : a;
          }
        }
      }
    }
    if (threadIdx.x == 0) p.tickets[tile] = 0u;  // ready for the next call on this stream
  }
}

__global__ void fill_u32_kernel(uint32_t* dst, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = v;
}

typedef void (*KernelFn)(const MvParams);

template <int BITS, int FMT, int EPI, int SEG>
KernelFn pick_kernel(int lpr, int rows) {
  if (lpr == 64) return rows == 2 ? qmv_kernel<BITS, FMT, 64, 2, EPI, SEG> : qmv_kernel<BITS, FMT, 64, 1, EPI, SEG>;
  if (lpr == 32) return rows == 2 ? qmv_kernel<BITS, FMT, 32, 2, EPI, SEG> : qmv_kernel<BITS, FMT, 32, 1, EPI, SEG>;
  if (lpr == 16) return rows == 2 ? qmv_kernel<BITS, FMT, 16, 2, EPI, SEG> : qmv_kernel<BITS, FMT, 16, 1, EPI, SEG>;
  return nullptr;
}

template <int BITS, int FMT>
KernelFn pick_kernel_epi(int epi, int seg, int lpr, int rows) {
  if (epi == kEpiStore) {
    if (seg == kSegNone) return pick_kernel<BITS, FMT, kEpiStore, kSegNone>(lpr, rows);
    if (seg == kSegCols) return pick_kernel<BITS, FMT, kEpiStore, kSegCols>(lpr, rows);
  } else if (epi == kEpiSwiglu) {
    if (seg == kSegNone) return pick_kernel<BITS, FMT, kEpiSwiglu, kSegNone>(lpr, rows);
    if (seg == kSegRows) return pick_kernel<BITS, FMT, kEpiSwiglu, kSegRows>(lpr, rows);
  }
  return nullptr;
}

}  // namespace

hipError_t launch_mv(int bits, int fmt, int epi, const MvPlan& plan, const MvParams& p,
                     hipStream_t stream) {
  KernelFn fn = nullptr;
  if (bits == 4 && fmt == 0) fn = pick_kernel_epi<4, 0>(epi, p.seg_mode, plan.lpr, plan.rows);
  else if (bits == 2 && fmt == 0) fn = pick_kernel_epi<2, 0>(epi, p.seg_mode, plan.lpr, plan.rows);
  else if (bits == 4 && fmt == 1) fn = pick_kernel_epi<4, 1>(epi, p.seg_mode, plan.lpr, plan.rows);
  if (!fn) return hipErrorInvalidValue;
  if (plan.lds_bytes > (size_t)kMaxLdsBytes) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(plan.grid_x * plan.splits));
  hipLaunchKernelGGL(fn, grid, dim3(kThreads), plan.lds_bytes, stream, p);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* dst, size_t n, uint32_t value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, n, value);
  return hipGetLastError();
}

}  // namespace qg
