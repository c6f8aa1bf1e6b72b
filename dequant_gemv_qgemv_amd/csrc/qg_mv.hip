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
// so the per-weight work is a multiply-add of the code with x, and the scale
// and bias enter once per 16-byte chunk of codes, in fp32.
//
// Work mapping (one workgroup = 8 wave64s):
//  * x (the slice of it this workgroup needs) is staged once in LDS, permuted
//    to match the code extraction below, plus one fp32 sum of x per chunk for
//    the bias term. Conflict-free layout: the 16-byte piece a lane reads for
//    chunk j of pass i, piece p sits at [i][p][j].
//  * Each wave owns bands of rows: 64/LPR sub-waves of LPR lanes, each lane
//    accumulating R rows. Lanes stride along K in 16-byte chunks (coalesced
//    dwordx4 buffer loads of the row-major codes).
//  * The (band, pass) items of a wave form one software pipeline: loads for
//    the next items are in flight while the current one is computed, across
//    band boundaries, and the first ones are issued before x is staged.
//  * Row sums are reduced across the LPR lanes with DPP.
//  * Optional split-K: workgroup (tile t, slice s) writes fp32 partials; the
//    last workgroup of tile t to finish (integer ticket, no float atomics)
//    adds the slices in fixed order and applies the epilogue, so results do
//    not depend on timing.
//
// Code extraction (affine formats): masking a packed word with 0x000F000F
// leaves two fp16 bit patterns that are exactly the subnormal numbers
// code*2^-24. v_dot2_f32_f16 multiplies such a pair with a pair of fp16 x
// values and adds both products to an fp32 accumulator, so 8 codes of a word
// cost 1 shift + 4 masks + 4 dot2. Codes at odd nibble positions come out
// multiplied by 16 (mask 0x00F000F0) and 2-bit fields by 4^j; their x is
// pre-divided by that power of two when staged. x is staged in fp16 after an
// exact power-of-two range scale 2^-e chosen from max|x| over the slice; the
// chunk result is multiplied back by 2^(24+e). The table format stages x the
// same way, as natural-order fp16 pairs that meet the row's table of code
// pairs (lut[lo], lut[hi]) in v_dot2_f32_f16.
#include <mutex>
#include <type_traits>
#include <unordered_map>

#include "qg_common.h"

namespace qg {
namespace {

__device__ __forceinline__ float dot2(uint32_t codes, uint32_t xpair, float acc) {
  return __builtin_amdgcn_fdot2(as_f16x2(codes), as_f16x2(xpair), acc, false);
}

// ---------------------------------------------------------------------------
// Inner products of one 16-byte chunk of codes with its staged x.

// 4-bit: 2^-24 * sum_k code_k x_k over 32 codes; xr[i] holds word i's pairs
// (x0,x4) (x1/16,x5/16) (x2,x6) (x3/16,x7/16) as fp16.
__device__ __forceinline__ float dot_q4(const u32x4 q, const u32x4* xr) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = w[i] >> 8;
    a0 = dot2(w[i] & 0x000F000Fu, xr[i].x, a0);  // fields 0, 4
    a1 = dot2(w[i] & 0x00F000F0u, xr[i].y, a1);  // fields 1, 5 (x16)
    a0 = dot2(t & 0x000F000Fu, xr[i].z, a0);     // fields 2, 6
    a1 = dot2(t & 0x00F000F0u, xr[i].w, a1);     // fields 3, 7 (x16)
  }
  return a0 + a1;
}

// 2-bit: 2^-24 * sum_k code_k x_k over 64 codes; word i uses xr[2i], xr[2i+1]
// holding the pairs (f0,f8) (f1,f9)/4 (f2,f10)/16 (f3,f11)/64 (f4,f12)/256
// (f5,f13) (f6,f14)/4 (f7,f15)/16.
__device__ __forceinline__ float dot_q2(const u32x4 q, const u32x4* xr) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = w[i] >> 10;
    const u32x4 u = xr[2 * i], v = xr[2 * i + 1];
    a0 = dot2(w[i] & 0x00030003u, u.x, a0);
    a1 = dot2(w[i] & 0x000C000Cu, u.y, a1);
    a0 = dot2(w[i] & 0x00300030u, u.z, a0);
    a1 = dot2(w[i] & 0x00C000C0u, u.w, a1);
    a0 = dot2(w[i] & 0x03000300u, v.x, a0);
    a1 = dot2(t & 0x00030003u, v.y, a1);
    a0 = dot2(t & 0x000C000Cu, v.z, a0);
    a1 = dot2(t & 0x00300030u, v.w, a1);
  }
  return a0 + a1;
}

// 8-bit: 2^-24 * sum_k code_k x_k over 16 codes; word i uses half of piece
// i/2: the pairs (x0,x2) (x1,x3) of its four codes. Codes up to 255 are
// still exact fp16 subnormals.
__device__ __forceinline__ float dot_q8(const u32x4 q, const u32x4* xr) {
  float a0 = 0.f, a1 = 0.f;
  a0 = dot2(q.x & 0x00FF00FFu, xr[0].x, a0);
  a1 = dot2((q.x >> 8) & 0x00FF00FFu, xr[0].y, a1);
  a0 = dot2(q.y & 0x00FF00FFu, xr[0].z, a0);
  a1 = dot2((q.y >> 8) & 0x00FF00FFu, xr[0].w, a1);
  a0 = dot2(q.z & 0x00FF00FFu, xr[1].x, a0);
  a1 = dot2((q.z >> 8) & 0x00FF00FFu, xr[1].y, a1);
  a0 = dot2(q.w & 0x00FF00FFu, xr[1].z, a0);
  a1 = dot2((q.w >> 8) & 0x00FF00FFu, xr[1].w, a1);
  return a0 + a1;
}

// Dense fp16 weights: sum_k w_k x_k over 8 weights, x in natural order.
__device__ __forceinline__ float dot_f16w(const u32x4 q, const u32x4* xr) {
  float a0 = dot2(q.x, xr[0].x, 0.f);
  float a1 = dot2(q.y, xr[0].y, 0.f);
  a0 = dot2(q.z, xr[0].z, a0);
  a1 = dot2(q.w, xr[0].w, a1);
  return a0 + a1;
}

// LUT (4-bit codes, 16-entry table per row): sum_k lut[code_k] x_k over the
// chunk's 32 codes, two codes per step. Byte b of code word i holds codes
// 2b (low nibble) and 2b + 1; as an index into the row's table of the 256
// pairs (lut[lo], lut[hi]) (fp16, in the sub-wave's LDS slot) it gives both
// weights at once, and v_dot2_f32_f16 takes them with the fp16 pair
// (x[8i+2b], x[8i+2b+1]) staged in piece i.
__device__ __forceinline__ float dot_lut(const u32x4 q, const u32x4* xr, const uint32_t* ptab) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 u = xr[i];
    a0 = dot2(ptab[w[i] & 0xFFu], u.x, a0);
    a1 = dot2(ptab[(w[i] >> 8) & 0xFFu], u.y, a1);
    a0 = dot2(ptab[(w[i] >> 16) & 0xFFu], u.z, a0);
    a1 = dot2(ptab[w[i] >> 24], u.w, a1);
  }
  return a0 + a1;
}

// ---------------------------------------------------------------------------
// Staging of x into LDS.

template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = MAX ? fmaxf(v, o) : v + o;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) s = MAX ? fmaxf(s, red[w]) : s + red[w];
  return s;
}

// This thread's share of sum(x^2) over all K (strided groups of 8).
__device__ float sumsq_all(const MvParams& p, const void* xp) {
  float ss = 0.f;
  const int K8 = p.K / 8;
  for (int i = threadIdx.x; i < K8; i += kThreads) {
    float v[8];
    load_x<8>(xp, p.x_f32, 8 * i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
  }
  return ss;
}

// One thread's chunk of x (and of the norm weights), loaded into registers
// before the weight prefetch is issued: vector loads return in order, so x
// must be requested first for its staging not to wait behind the weights.
template <int CPC>
struct XChunk {
  float v[CPC];
  u32x4 g[CPC / 8];  // norm weights as raw fp16 pairs
};

template <int CPC>
__device__ __forceinline__ void stage_load(const MvParams& p, const void* xp, int cg, bool have,
                                           XChunk<CPC>& xc) {
  if (have) {
    load_x<CPC>(xp, p.x_f32, cg * CPC, xc.v);
    if (p.norm_w) {
      const u32x4* src = reinterpret_cast<const u32x4*>(p.norm_w + cg * CPC);
#pragma unroll
      for (int i = 0; i < CPC / 8; ++i) xc.g[i] = src[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < CPC; ++i) xc.v[i] = 0.f;
#pragma unroll
    for (int i = 0; i < CPC / 8; ++i) xc.g[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Stages one chunk (v: its x values in natural order; cg: its logical index,
// valid = inside the slice): x*g (RMSNorm weight; the 1/rms scalar is applied
// to the row sums instead), times the K-segment routing weight, then the
// chunk's own power-of-two range scale (affine formats) and the LDS write.
// No block-wide reduction is involved. Returns the chunk's sum of squares of
// x (0 without a norm or outside the slice).
template <int BITS, int FMT, int LPR>
__device__ __forceinline__ float stage_chunk(const MvParams& p, const float* rw, float* v, const u32x4* g, int c,
                                            int cg, bool valid, u32x4* xl, ChunkInfo* info) {
  constexpr int CPC = Geo<BITS, FMT>::kPerChunk;
  constexpr int PIECES = Geo<BITS, FMT>::kPieces;
  float ss = 0.f;
  if (p.norm_w) {
#pragma unroll
    for (int i = 0; i < CPC / 8; ++i) {
      const uint32_t w[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x2 h = as_f16x2(w[q]);
        const float a = v[8 * i + 2 * q], b = v[8 * i + 2 * q + 1];
        ss = fmaf(a, a, fmaf(b, b, ss));
        v[8 * i + 2 * q] = a * (float)h.x;
        v[8 * i + 2 * q + 1] = b * (float)h.y;
      }
    }
  }
  float wseg = 1.0f;
  if (valid && p.seg_mode == kSegCols && rw) {
    const int seg = cg / p.seg_len;
    wseg = seg < p.route.n_routed ? rw[seg] : 1.0f;
  }
  float s = 0.f, m = 0.f;
#pragma unroll
  for (int i = 0; i < CPC; ++i) {
    v[i] *= wseg;
    s += v[i];
    m = fmaxf(m, fabsf(v[i]));
  }
  float back = 1.0f;
  {  // x staged in fp16 (every format)
    const float inv = range_scale(m, &back);
#pragma unroll
    for (int i = 0; i < CPC; ++i) v[i] *= inv;
  }
  write_pieces<BITS, FMT>(v, xl + (c / LPR) * PIECES * LPR + (c % LPR), LPR);
  ChunkInfo ci;
  ci.xsum = valid ? s : 0.f;
  ci.back = back;
  ci.ss = valid ? ss : 0.f;
  ci.pad = 0.f;
  info[c] = ci;
  return ci.ss;
}

// ---------------------------------------------------------------------------
// Staging in quarters (slices of at most 128 chunks). Each chunk's x is cut
// into four quarters of CPC/4 consecutive values held by four adjacent lanes;
// quarter unit u (chunk u/4, quarter u%4) belongs to thread u. Every wave of
// the workgroup then carries a few x loads at the head of its memory queue,
// ahead of its weight prefetch, instead of two waves carrying all of them
// behind the weight requests of the others. The chunk's sum and maximum are
// combined over the quad with DPP.

// Makes a value pass through an empty instruction at this point: the compiler
// must have it here and cannot hoist its uses above, so a load issued earlier
// is waited for here and not before the loads issued in between.
__device__ __forceinline__ void hold(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void hold(float& v) { asm volatile("" : "+v"(v)); }

struct XRsrc {
  __amdgpu_buffer_rsrc_t x, g;
};

__device__ __forceinline__ XRsrc x_rsrc(const MvParams& p, const void* xp) {
  XRsrc r;
  r.x = make_rsrc(xp, (uint32_t)p.K * (p.x_f32 ? 4u : 2u));
  r.g = make_rsrc(p.norm_w ? (const void*)p.norm_w : xp, p.norm_w ? (uint32_t)p.K * 2u : 0u);
  return r;
}

// Requests quarter unit u of the slice starting at chunk c0 (nch chunks;
// units of padding chunks and past nunits load nothing and hold zeros). The
// words stay raw until staging so that nothing waits for them here, and the
// instruction count is the same on every path (fp16 x and a missing norm read
// past their descriptors and get zeros) so that the later wait for them counts
// exactly the loads issued after.
template <int CPC>
__device__ __forceinline__ void quarter_load(const MvParams& p, const XRsrc& r, int c0, int nch, int u,
                                             int nunits, u32x4* x, u32x4* g) {
  constexpr int QV = CPC / 4;
  const int c = u >> 2, q = u & 3;
  const bool ok = u < nunits && c < nch;
  const uint32_t k0 = (uint32_t)((c0 + c) * CPC + q * QV);
  const uint32_t es = p.x_f32 ? 4u : 2u;
#pragma unroll
  for (int i = 0; i < QV / 4; ++i) {
    const bool in = ok && (p.x_f32 || i < QV / 8);
    x[i] = __builtin_amdgcn_raw_buffer_load_b128(r.x, in ? (k0 + (p.x_f32 ? 4 : 8) * i) * es : kOOB, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < QV / 8; ++i)
    g[i] = __builtin_amdgcn_raw_buffer_load_b128(r.g, ok && p.norm_w ? (k0 + 8 * i) * 2u : kOOB, 0, 0);
}

// Routing weight that scales quarter unit u's K segment (1 outside the routed
// segments or without K segments), requested together with x so that staging
// does not wait for a second round trip.
__device__ __forceinline__ float quarter_seg_weight(const MvParams& p, const float* rw, int c0, int u,
                                                   int nunits) {
  float w = 1.0f;
  if (p.seg_mode == kSegCols && rw && u < nunits) {
    const int seg = (c0 + (u >> 2)) / p.seg_len;
    if (seg < p.route.n_routed) w = rw[seg];
  }
  return w;
}

// Writes quarter q of a chunk's staged x (w already range scaled for the
// affine formats): the same pieces write_pieces produces for those values.
template <int BITS, int FMT>
__device__ __forceinline__ void write_quarter(const float* w, u32x4* dst, int stride, int q) {
  if constexpr (FMT == 1) {  // natural-order fp16 pairs of code word q
    dst[q * stride] = u32x4{pack_f16(w[0], w[1]), pack_f16(w[2], w[3]), pack_f16(w[4], w[5]),
                            pack_f16(w[6], w[7])};
  } else if constexpr (BITS == 4) {
    constexpr float r16 = 1.0f / 16.0f;
    dst[q * stride] = u32x4{pack_f16(w[0], w[4]), pack_f16(w[1] * r16, w[5] * r16), pack_f16(w[2], w[6]),
                            pack_f16(w[3] * r16, w[7] * r16)};
  } else {
    constexpr float r4 = 0.25f, r16 = 1.0f / 16.0f, r64 = 1.0f / 64.0f, r256 = 1.0f / 256.0f;
    dst[(2 * q) * stride] = u32x4{pack_f16(w[0], w[8]), pack_f16(w[1] * r4, w[9] * r4),
                                  pack_f16(w[2] * r16, w[10] * r16), pack_f16(w[3] * r64, w[11] * r64)};
    dst[(2 * q + 1) * stride] = u32x4{pack_f16(w[4] * r256, w[12] * r256), pack_f16(w[5], w[13]),
                                      pack_f16(w[6] * r4, w[14] * r4), pack_f16(w[7] * r16, w[15] * r16)};
  }
}

__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false)));
}

// Stages quarter unit u (as stage_chunk does for a whole chunk). The four
// lanes of a quad always hold the four quarters of one chunk, all inside or
// all past nunits, so the quad reductions see only their own chunk. Returns
// this lane's sum of squares of its raw x (0 without a norm or outside the
// slice).
template <int BITS, int FMT, int LPR>
__device__ __forceinline__ float stage_quarter(const MvParams& p, const u32x4* x, const u32x4* g, float wseg,
                                               int u, int nunits, int c0, int nch, u32x4* xl,
                                               ChunkInfo* info) {
  constexpr int CPC = Geo<BITS, FMT>::kPerChunk;
  constexpr int QV = CPC / 4;
  constexpr int PIECES = Geo<BITS, FMT>::kPieces;
  const int c = u >> 2, q = u & 3;
  const bool valid = u < nunits && c < nch;
  float v[QV];
  if (p.x_f32) {
#pragma unroll
    for (int i = 0; i < QV / 4; ++i) {
      v[4 * i] = __uint_as_float(x[i].x);
      v[4 * i + 1] = __uint_as_float(x[i].y);
      v[4 * i + 2] = __uint_as_float(x[i].z);
      v[4 * i + 3] = __uint_as_float(x[i].w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < QV / 8; ++i) {
      const uint32_t w[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2 h = as_f16x2(w[j]);
        v[8 * i + 2 * j] = (float)h.x;
        v[8 * i + 2 * j + 1] = (float)h.y;
      }
    }
  }
  float ss = 0.f;
  if (p.norm_w) {
#pragma unroll
    for (int i = 0; i < QV / 8; ++i) {
      const uint32_t w[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f16x2 h = as_f16x2(w[t]);
        const float a = v[8 * i + 2 * t], b = v[8 * i + 2 * t + 1];
        ss = fmaf(a, a, fmaf(b, b, ss));
        v[8 * i + 2 * t] = a * (float)h.x;
        v[8 * i + 2 * t + 1] = b * (float)h.y;
      }
    }
  }
  float s = 0.f, m = 0.f;
#pragma unroll
  for (int i = 0; i < QV; ++i) {
    v[i] *= wseg;
    s += v[i];
    m = fmaxf(m, fabsf(v[i]));
  }
  s = quad_sum(s);
  m = quad_max(m);
  float back = 1.0f;
  {
    const float inv = range_scale(m, &back);
#pragma unroll
    for (int i = 0; i < QV; ++i) v[i] *= inv;
  }
  const float css = quad_sum(ss);
  if (u < nunits) {
    write_quarter<BITS, FMT>(v, xl + (c / LPR) * PIECES * LPR + (c % LPR), LPR, q);
    if (q == 0) {
      ChunkInfo ci;
      ci.xsum = valid ? s : 0.f;
      ci.back = back;
      ci.ss = valid ? css : 0.f;
      ci.pad = 0.f;
      info[c] = ci;
    }
  }
  return valid ? ss : 0.f;
}

// Stages chunks [c0, c0 + nch) (zero padded to npass*LPR) when the chunks
// outnumber the threads: each thread loops over its chunks, reading x again.
template <int BITS, int FMT, int LPR>
__device__ float stage_loop(const MvParams& p, const void* xp, const float* rw, int c0, int nch, int npass, u32x4* xl,
                            ChunkInfo* info) {
  constexpr int CPC = Geo<BITS, FMT>::kPerChunk;
  float ss = 0.f;
  for (int c = threadIdx.x; c < npass * LPR; c += kThreads) {
    XChunk<CPC> xc;
    stage_load<CPC>(p, xp, c0 + c, c < nch, xc);
    ss += stage_chunk<BITS, FMT, LPR>(p, rw, xc.v, xc.g, c, c0 + c, c < nch, xl, info);
  }
  return ss;
}

// 1/sqrt(mean(x^2) + eps) over all of K read from memory (used when this
// workgroup stages only a slice of K). Every thread of the block calls it.
__device__ float rms_all(const MvParams& p, const void* xp, float* red) {
  return 1.0f / sqrtf(block_reduce<false>(sumsq_all(p, xp), red) / (float)p.K + p.eps);
}

// Matrix of segment `seg` (routed experts are looked up from the chosen ids:
// device memory, or the workgroup's own routing in LDS).
__device__ __forceinline__ QMat seg_mat(const MvParams& p, const int32_t* ids, int seg, bool second) {
  if (ids && seg < p.route.n_routed) {
    const size_t r0 = (size_t)ids[seg] * (size_t)p.route.expert_rows;
    const QMat all = second ? p.route.all_B : p.route.all_A;
    QMat m;
    m.q = all.q ? all.q + r0 * p.wpr : nullptr;
    m.s = all.s ? all.s + r0 * p.gpr : nullptr;
    m.b = all.b ? all.b + r0 * p.gpr : nullptr;
    m.lut = all.lut ? all.lut + r0 * 16 : nullptr;
    return m;
  }
  return second ? p.B[seg] : p.A[seg];
}

__device__ __forceinline__ int seg_rows(const MvParams& p, const int32_t* ids, int seg) {
  if (ids && seg < p.route.n_routed) return p.route.expert_rows;
  return p.seg_mode == kSegRows ? p.seg_len : p.N;
}

template <int R, bool TWO, int LUTN, int SBL>
struct PassData {
  u32x4 qa[R];
  uint16_t sa[R], ba[R];  // this pass's scale/bias (SBL = 0)
  u32x4 qb[TWO ? R : 1];
  uint16_t sb[TWO ? R : 1], bb[TWO ? R : 1];
  uint16_t lut[LUTN > 0 ? LUTN : 1];  // LUT entries of the band, carried by its pass 0
  u32x4 sbq[SBL > 0 ? SBL : 1];       // the band's scale/bias row pieces, carried by its pass 0
};

// One pass for the lane's R rows. qoff/soff are the byte offsets of the
// lane's chunk (codes) and group (scales/biases) in each row for pass 0;
// dq/ds move them to this pass. ok = false gives zero loads.
template <int FMT, int R, bool TWO, int LUTN, int SBL>
__device__ __forceinline__ void load_pass(const MatRsrc& ra, const MatRsrc& rb, const uint32_t* qoff,
                                          const uint32_t* soff, uint32_t dq, uint32_t ds, bool ok,
                                          PassData<R, TWO, LUTN, SBL>& d) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t oq = ok ? qoff[r] + dq : kOOB;
    const uint32_t os = ok ? soff[r] + ds : kOOB;
    d.qa[r] = __builtin_amdgcn_raw_buffer_load_b128(ra.q, oq, 0, 2);
    if constexpr (FMT == 0 && SBL == 0) {
      d.sa[r] = __builtin_amdgcn_raw_buffer_load_b16(ra.s, os, 0, 0);
      d.ba[r] = __builtin_amdgcn_raw_buffer_load_b16(ra.b, os, 0, 0);
    }
    if constexpr (TWO) {
      d.qb[r] = __builtin_amdgcn_raw_buffer_load_b128(rb.q, oq, 0, 2);
      if constexpr (FMT == 0 && SBL == 0) {
        d.sb[r] = __builtin_amdgcn_raw_buffer_load_b16(rb.s, os, 0, 0);
        d.bb[r] = __builtin_amdgcn_raw_buffer_load_b16(rb.b, os, 0, 0);
      }
    }
  }
}

// sbw (SBL > 0): the lane's sub-wave's staged scale/bias row segments,
// [R][NACC][scales, biases][segh halfwords] (group g of the slice at index
// g); gsl groups hold this slice's values, a lane past them (a padding chunk,
// whose codes load as zero) takes scale and bias 0 as the per-pass loads do.
template <int BITS, int FMT, int LPR, int R, bool TWO, int LUTN, int SBL>
__device__ __forceinline__ void compute_pass(const PassData<R, TWO, LUTN, SBL>& d, const u32x4* xl,
                                             const ChunkInfo* info, int pass, int j,
                                             const uint32_t* ptab, const uint16_t* sbw, int segh, int gsl,
                                             float* acc_a, float* acc_b) {
  constexpr int PIECES = Geo<BITS, FMT>::kPieces;
  // staged scale/bias values first: LDS reads complete in order, so they are
  // in by the time the dot products over x need them
  constexpr int NSB = (FMT == 0 && SBL > 0) ? R * (TWO ? 4 : 2) : 1;
  uint16_t sbv[NSB];
  uint16_t sbmask = 0;
  if constexpr (FMT == 0 && SBL > 0) {
    constexpr int CPG = Geo<BITS, FMT>::kChunksPerGroup;
    const int gl = (pass * LPR + j) / CPG;
    sbmask = gl < gsl ? (uint16_t)0xFFFF : (uint16_t)0;
    const int glc = gl < segh ? gl : segh - 1;  // an address inside the segment either way
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int q = 0; q < (TWO ? 4 : 2); ++q) sbv[r * (TWO ? 4 : 2) + q] = sbw[(r * (TWO ? 4 : 2) + q) * segh + glc];
  }
  u32x4 xr[PIECES];
  const u32x4* src = xl + pass * PIECES * LPR + j;
#pragma unroll
  for (int i = 0; i < PIECES; ++i) xr[i] = src[i * LPR];
  if constexpr (FMT == 1) {
    // x was staged in fp16 after the chunk's range scale: the back factor
    // carries 2^24 for the codes' subnormal scale, which table weights lack
    constexpr int NACC = TWO ? 2 : 1;
    const float back = info[pass * LPR + j].back * 0x1p-24f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc_a[r] = fmaf(dot_lut(d.qa[r], xr, ptab + (r * NACC) * kLutPairWords), back, acc_a[r]);
      if constexpr (TWO)
        acc_b[r] = fmaf(dot_lut(d.qb[r], xr, ptab + (r * NACC + 1) * kLutPairWords), back, acc_b[r]);
    }
  } else if constexpr (FMT == 2) {
    // dense fp16 weights: the chunk's back factor carries 2^24 for the codes'
    // subnormal scale, which these weights do not have
    const float back = info[pass * LPR + j].back * 0x1p-24f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc_a[r] = fmaf(dot_f16w(d.qa[r], xr), back, acc_a[r]);
      if constexpr (TWO) acc_b[r] = fmaf(dot_f16w(d.qb[r], xr), back, acc_b[r]);
    }
  } else {
    constexpr int NACC = TWO ? 2 : 1;
    uint16_t sa[R], ba[R], sb2[TWO ? R : 1], bb2[TWO ? R : 1];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if constexpr (SBL > 0) {
        sa[r] = sbv[r * NACC * 2] & sbmask;
        ba[r] = sbv[r * NACC * 2 + 1] & sbmask;
        if constexpr (TWO) {
          sb2[r] = sbv[r * NACC * 2 + 2] & sbmask;
          bb2[r] = sbv[r * NACC * 2 + 3] & sbmask;
        }
      } else {
        sa[r] = d.sa[r];
        ba[r] = d.ba[r];
        if constexpr (TWO) {
          sb2[r] = d.sb[r];
          bb2[r] = d.bb[r];
        }
      }
    }
    const float2 sb = *reinterpret_cast<const float2*>(&info[pass * LPR + j]);  // (xsum, back)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float da = (BITS == 4 ? dot_q4(d.qa[r], xr) : BITS == 8 ? dot_q8(d.qa[r], xr) : dot_q2(d.qa[r], xr)) * sb.y;
      acc_a[r] = fmaf(f16_bits_to_f32(sa[r]), da, acc_a[r]);
      acc_a[r] = fmaf(f16_bits_to_f32(ba[r]), sb.x, acc_a[r]);
      if constexpr (TWO) {
        const float db = (BITS == 4 ? dot_q4(d.qb[r], xr) : BITS == 8 ? dot_q8(d.qb[r], xr) : dot_q2(d.qb[r], xr)) * sb.y;
        acc_b[r] = fmaf(f16_bits_to_f32(sb2[r]), db, acc_b[r]);
        acc_b[r] = fmaf(f16_bits_to_f32(bb2[r]), sb.x, acc_b[r]);
      }
    }
  }
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

template <int LPR>
__device__ __forceinline__ float lanes_sum(float v) {
  v += dpp_f32<0xb1, 0xf>(v);   // quad_perm 1,0,3,2
  v += dpp_f32<0x4e, 0xf>(v);   // quad_perm 2,3,0,1
  v += dpp_f32<0x141, 0xf>(v);  // row_half_mirror
  v += dpp_f32<0x140, 0xf>(v);  // row_mirror: every lane of a row of 16 holds the row sum
  if constexpr (LPR >= 32) v += dpp_f32<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  if constexpr (LPR >= 64) v += dpp_f32<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// ---------------------------------------------------------------------------
// One workgroup = 8 waves; workgroup (tile t, slice s). Each wave walks its
// bands t*8 + w, + grid_x*8, ... and within a band the passes over its K
// slice. That (band, pass) sequence is one software pipeline DEPTH items
// deep: the first DEPTH items are requested before x is staged, and a slot is
// refilled with the item DEPTH ahead as soon as it has been consumed, across
// band boundaries, so the memory queue never drains inside a wave.
template <int BITS, int FMT, int LPR, int R, int EPI, int SEG, int DEPTH, int SBL>
__global__ __launch_bounds__(kThreads) void qmv_kernel(const MvParams p) {
  constexpr int PIECES = Geo<BITS, FMT>::kPieces;
  constexpr int CPC = Geo<BITS, FMT>::kPerChunk;
  constexpr int CPG = Geo<BITS, FMT>::kChunksPerGroup;
  constexpr int SUB = 64 / LPR;
  constexpr int RPB = SUB * R;  // rows per band
  constexpr bool TWO = (EPI == kEpiSwiglu);
  constexpr bool TOPK = (EPI == kEpiTopk);
  constexpr int NACC = TWO ? 2 : 1;
  constexpr int LUTN = (FMT == 1) ? (R * NACC * 16 + LPR - 1) / LPR : 0;
  typedef PassData<R, TWO, LUTN, SBL> PD;
  static_assert(SBL == 0 || (FMT == 0 && SEG != kSegCols), "staged scale/bias rows: affine, one K segment");

  extern __shared__ u32x4 smem[];
  __shared__ float red[2 * kWaves];
  __shared__ int last_flag;
  __shared__ uint64_t tk_keys[TOPK ? kWaves : 1][kTkList];  // each wave's row keys, then sorted
  __shared__ int32_t rt_ids[kMaxRoutes];
  __shared__ float rt_w[kMaxRoutes];

  params_now(p);
  // A launch over several vectors (a batched expert launch, or several
  // activation vectors of 8-bit or dense weights): each workgroup serves one
  // vector, whose data follow the first one's at fixed strides (x [M][K], y
  // and residual [M][N], router logits [M][n_experts], stored routes
  // [M][kMaxRoutes], returned routes [M][n_routed]). A launch with one vector
  // uses its own pointers.
  // Workgroup id -> (vector, tile): with several vectors, the workgroups of
  // one tile for the successive vectors get ids 8 apart, so they land on the
  // same XCD (workgroups go round-robin over the 8) one after the other and
  // share its L2 copy of the tile's weights. One vector: the id is the tile.
  int tok = 0, bid = (int)blockIdx.x;
  if (p.tokens > 1) {
    const int lo = bid & 7, rest = bid >> 3;
    tok = rest % p.tokens;
    bid = (rest / p.tokens) * 8 + lo;
  }
  const void* const xp = static_cast<const char*>(p.x) + (size_t)tok * p.K * (p.x_f32 ? 4 : 2);
  float* const yp = p.y + (size_t)tok * p.N;
  const float* const resp = p.residual ? p.residual + (size_t)tok * p.N : nullptr;
  const float* const rwp = p.route.weights ? p.route.weights + tok * kMaxRoutes : nullptr;
  const int slice = bid / p.grid_x;
  const int tile = bid - slice * p.grid_x;
  const int C = p.K / CPC;
  const int c0 = slice * p.slice_chunks;
  const int nch = min(p.slice_chunks, C - c0);
  const int npass = (nch + LPR - 1) / LPR;
  const int nbands = (p.N + RPB - 1) / RPB;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int j = lane % LPR;
  // same for every slice of this tile: no split-K ticket needed (a fused
  // top-k launch keeps every workgroup: each takes its group's ticket)
  if (!TOPK && tile * kWaves >= nbands) return;
  const int band_stride = p.grid_x * kWaves;

  // Staged scale/bias rows (SBL > 0): the scale and bias row segments over
  // this K slice of a band's rows, [RPB][NACC][scales, biases][segp pieces of
  // 16 bytes], come with SBL 16-byte loads per lane carried by the band's
  // first pass, and go to the wave's LDS area when that pass is computed;
  // every pass then reads its two values per row from there (instead of two
  // 2-byte loads per row and matrix per pass). The piece a lane loads is the
  // same in every band: (row, matrix, array, piece) from its lane number.
  const int segp = SBL > 0 ? p.sb_segp : 1;
  const int g0 = c0 / CPG;    // the slice's first group
  const int gsl = nch / CPG;  // groups in this slice (a multiple of 8 when staged)
  int sb_t[SBL > 0 ? SBL : 1], sb_a[SBL > 0 ? SBL : 1], sb_m[SBL > 0 ? SBL : 1], sb_rr[SBL > 0 ? SBL : 1];
  bool sb_in[SBL > 0 ? SBL : 1];
  const uint16_t* sb_src[SBL > 0 ? SBL : 1];
  if constexpr (SBL > 0) {
#pragma unroll
    for (int i = 0; i < SBL; ++i) {
      const int P = lane + 64 * i;
      const int rest = P / segp;
      sb_t[i] = P - rest * segp;
      sb_a[i] = rest & 1;
      sb_m[i] = (rest >> 1) % NACC;
      sb_rr[i] = (rest >> 1) / NACC;
      sb_in[i] = P < RPB * NACC * 2 * segp && sb_t[i] * 8 + 8 <= gsl;
      sb_src[i] = p.A[0].s;
    }
  }

  // Quarter staging (one quarter unit of x per thread): x and the segment
  // routing weight are requested before the weight prefetch (loads return in
  // order, so they arrive first); in a launch that routes its experts itself,
  // already before the routing, which then overlaps their round trip.
  const bool quarter = CPC >= 32 && 4 * npass * LPR <= kThreads;
  const int nunits = 4 * npass * LPR;
  u32x4 qx[CPC >= 32 ? CPC / 16 : 1], qg[CPC >= 32 ? (CPC / 4 + 7) / 8 : 1];
  float qw = 1.0f;
  // requests quarter unit u (zeros past nunits)
  auto load_quarters_at = [&](int u) {
    if constexpr (CPC >= 32) {
      const XRsrc xr = x_rsrc(p, xp);
#pragma unroll
      for (int i = 0; i < CPC / 16; ++i) qx[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < (CPC / 4 + 7) / 8; ++i) qg[i] = u32x4{0u, 0u, 0u, 0u};
      quarter_load<CPC>(p, xr, c0, nch, u, nunits, qx, qg);
      qw = quarter_seg_weight(p, rwp, c0, u, nunits);
      asm volatile("" ::: "memory");
    }
  };
  auto load_quarters = [&]() {
    if (quarter) load_quarters_at(threadIdx.x);
  };
  // Expert ids of a gathered launch: from device memory, or chosen here
  // (workgroup 0 stores them for the launches that follow).
  const int32_t* rids = p.route.ids ? p.route.ids + tok * kMaxRoutes : nullptr;
  // A K-segmented launch (the experts' down projections) switches expert at
  // every pass; its ids come from device memory once per workgroup into LDS,
  // requested ahead of x, instead of one dependent lookup per pass.
  int32_t my_id = 0;
  if constexpr (SEG == kSegCols) {
    if (rids && (int)threadIdx.x < p.route.n_routed) my_id = rids[threadIdx.x];
    asm volatile("" ::: "memory");
  }
  // (measured: loading x this early in the launches that do not route costs
  // the 4096 x 14336 gate.up 3 %)
  if constexpr (SEG != kSegNone) load_quarters();
  if constexpr (SEG == kSegCols) {
    if (rids) {
      if ((int)threadIdx.x < p.route.n_routed) rt_ids[threadIdx.x] = my_id;
      __syncthreads();
      rids = rt_ids;
    }
  }
  if constexpr (SEG == kSegRows) {
    if (p.route.logits) {
      if (wave == 0) {
        int32_t ids[kMaxRoutes];
        float w[kMaxRoutes];
        route_wave(p.route.logits + (size_t)tok * p.route.n_experts, p.route.n_experts,
                   p.route.n_routed, ids, w);
        if (lane == 0) {
          const int so = tok * kMaxRoutes, sl = tok * p.route.n_routed;
          for (int r = 0; r < p.route.n_routed; ++r) {
            rt_ids[r] = ids[r];
            rt_w[r] = w[r];
            if (bid == 0) {  // the vector's first workgroup
              p.route.ids_store[so + r] = ids[r];
              p.route.w_store[so + r] = w[r];
              if (p.route.sel_ids) p.route.sel_ids[sl + r] = ids[r];
              if (p.route.sel_w) p.route.sel_w[sl + r] = w[r];
            }
          }
        }
      }
      __syncthreads();
      rids = rt_ids;
    }
  }

  // ---- loader: requests (band, pass) items ahead of the compute ----------
  int ld_band = tile * kWaves + wave, ld_pass = 0, ld_seg = 0;
  uint32_t qoff[R], soff[R];
  int ld_row[R];
  MatRsrc ra = empty_rsrc(p), rb = empty_rsrc(p);
  if constexpr (SEG != kSegRows) {
    if constexpr (SEG == kSegNone) ra = mat_rsrc(p.A[0], p.N, p.wpr, p.gpr);
    if constexpr (TWO) rb = mat_rsrc(p.B[0], p.N, p.wpr, p.gpr);
  }

  auto band_setup = [&](int band) {
    if constexpr (SEG == kSegRows) {
      ld_seg = (band * RPB) / p.seg_len;  // a band never straddles two row segments
      const int rows = seg_rows(p, rids, ld_seg);
      ra = mat_rsrc(seg_mat(p, rids, ld_seg, false), rows, p.wpr, p.gpr);
      if constexpr (TWO) rb = mat_rsrc(seg_mat(p, rids, ld_seg, true), rows, p.wpr, p.gpr);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = band * RPB + sub * R + r;
      const int lr = (SEG == kSegRows) ? n - ld_seg * p.seg_len : n;
      const bool ok = n < p.N;
      ld_row[r] = ok ? lr : -1;
      // chunk of pass 0; K segments add their (segment-local) chunk per pass
      const uint32_t cfirst = (SEG == kSegCols) ? 0u : (uint32_t)(c0 + j);
      qoff[r] = ok ? (uint32_t)lr * (uint32_t)p.wpr * 4u + cfirst * 16u : kOOB;
      soff[r] = ok ? (uint32_t)lr * (uint32_t)p.gpr * 2u + (cfirst / CPG) * 2u : kOOB;
    }
    if constexpr (SBL > 0) {
      // the band's row matrices; a lane with no piece reads the first 16
      // bytes of A's scales (always present) and keeps nothing of them
      QMat ma, mb;
      int rows_m;
      if constexpr (SEG == kSegRows) {
        ma = seg_mat(p, rids, ld_seg, false);
        mb = TWO ? seg_mat(p, rids, ld_seg, true) : ma;
        rows_m = seg_rows(p, rids, ld_seg);
      } else {
        ma = p.A[0];
        mb = TWO ? p.B[0] : ma;
        rows_m = p.N;
      }
#pragma unroll
      for (int i = 0; i < SBL; ++i) {
        const int n = band * RPB + sb_rr[i];
        const int lr = (SEG == kSegRows) ? n - ld_seg * p.seg_len : n;
        const bool ok = sb_in[i] && n < p.N && lr < rows_m;
        const uint16_t* base = sb_m[i] ? (sb_a[i] ? mb.b : mb.s) : (sb_a[i] ? ma.b : ma.s);
        sb_src[i] = ok ? base + (size_t)lr * p.gpr + g0 + sb_t[i] * 8 : ma.s;
      }
    }
  };

  // One request of the pipeline: item (ld_band, ld_pass), or loads that
  // return zeros past the last band. Every call issues the same instructions
  // on one straight path (offsets past a descriptor's end where there is
  // nothing to load): with a branch around the loads the compiler reuses the
  // destinations of loads still in flight as temporaries on the other path,
  // and the wait this forces drains the whole pipeline at every request.
  auto issue = [&](PD& d) {
    const bool have = ld_band < nbands;  // uniform
    if (have && ld_pass == 0) band_setup(ld_band);
    if constexpr (SBL > 0) {
      if (have && ld_pass == 0) {
#pragma unroll
        for (int i = 0; i < SBL; ++i) d.sbq[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sb_src[i]));
      }
    }
    if constexpr (FMT == 1) {
      // a band's tables ride along with its first pass
      const bool first = have && ld_pass == 0;
#pragma unroll
      for (int q = 0; q < LUTN; ++q) {
        const int e = j + q * LPR;  // entry e of [R][NACC][16]
        const int r = min(e / (NACC * 16), R - 1), m = (e / 16) % NACC, t = e % 16;
        const bool ok = first && e < R * NACC * 16 && ld_row[r] >= 0;
        const uint32_t off = ((uint32_t)ld_row[r] * 16u + (uint32_t)t) * 2u;
        uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(ra.l, ok && m == 0 ? off : kOOB, 0, 0);
        if constexpr (TWO) v |= __builtin_amdgcn_raw_buffer_load_b16(rb.l, ok && m == 1 ? off : kOOB, 0, 0);
        d.lut[q] = v;
      }
    }
    const bool ok = have && ld_pass * LPR + j < nch;
    if constexpr (SEG == kSegCols) {
      const int cpass = c0 + ld_pass * LPR;
      const int s_lo = min(cpass / p.seg_len, p.nseg - 1);
      const int s_hi = min((cpass + LPR - 1) / p.seg_len, p.nseg - 1);
      const int cg = cpass + j;
      if (s_lo == s_hi) {
        ra = mat_rsrc(seg_mat(p, rids, s_lo, false), seg_rows(p, rids, s_lo), p.wpr, p.gpr);
        const int cl = cg - s_lo * p.seg_len;
        load_pass<FMT, R, TWO, LUTN, SBL>(ra, rb, qoff, soff, (uint32_t)cl * 16u, (uint32_t)(cl / CPG) * 2u, ok,
                                     d);
      } else {
        // several segments in one pass: one masked load per segment, merged
        const int mine = cg / p.seg_len;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          d.qa[r] = u32x4{0u, 0u, 0u, 0u};
          d.sa[r] = d.ba[r] = 0;
        }
        for (int sg = s_lo; sg <= s_hi; ++sg) {
          PD t;
          ra = mat_rsrc(seg_mat(p, rids, sg, false), seg_rows(p, rids, sg), p.wpr, p.gpr);
          const int cl = cg - sg * p.seg_len;
          load_pass<FMT, R, TWO, LUTN, SBL>(ra, rb, qoff, soff, (uint32_t)cl * 16u, (uint32_t)(cl / CPG) * 2u,
                                       ok && mine == sg, t);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            d.qa[r] |= t.qa[r];
            d.sa[r] |= t.sa[r];
            d.ba[r] |= t.ba[r];
          }
        }
      }
    } else {
      load_pass<FMT, R, TWO, LUTN, SBL>(ra, rb, qoff, soff, (uint32_t)(ld_pass * LPR) * 16u,
                                   (uint32_t)(ld_pass * LPR / CPG) * 2u, ok, d);
    }
    if (have && ++ld_pass == npass) {
      ld_pass = 0;
      ld_band += band_stride;
    }
    // Keep each request where it is issued: otherwise the compiler sinks the
    // loads next to their first use and the pipeline collapses.
    asm volatile("" ::: "memory");
  };

  u32x4* xl = smem;
  ChunkInfo* info = reinterpret_cast<ChunkInfo*>(smem + (size_t)npass * LPR * PIECES);
  // table format: per sub-wave, [R][NACC] pair tables of kLutPairWords words,
  // then the [R][NACC][16] fp16 entries they are built from
  uint32_t* const ptab = reinterpret_cast<uint32_t*>(info + npass * LPR) + (size_t)(wave * SUB + sub) * R * NACC * kLutRowWords;
  uint16_t* const l16 = reinterpret_cast<uint16_t*>(ptab + R * NACC * kLutPairWords);
  // affine formats with staged scale/bias rows: [kWaves][RPB][NACC][2][segp] pieces there instead
  u32x4* const sbw4 = reinterpret_cast<u32x4*>(info + npass * LPR) + (size_t)wave * RPB * NACC * 2 * segp;
  const uint16_t* const sbw = reinterpret_cast<const uint16_t*>(sbw4) + (size_t)sub * R * NACC * 2 * segp * 8;

  // x first, then the weight prefetch, then the staging arithmetic: the
  // staging then waits for x only while the weights are in flight.
  PD d[DEPTH];
  const bool whole_k = (c0 == 0 && nch == C);
  float ss = 0.f;
  // Quarter staging needs quarters of at least 8 values (one 16-byte fp16
  // load): chunks of 32 codes or more. x is waited for only after the weight
  // requests are out.
  if (quarter) {
    if constexpr (CPC >= 32) {
      if constexpr (SEG == kSegNone) load_quarters();
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) issue(d[k]);
#pragma unroll
      for (int i = 0; i < CPC / 16; ++i) hold(qx[i]);
#pragma unroll
      for (int i = 0; i < (CPC / 4 + 7) / 8; ++i) hold(qg[i]);
      hold(qw);
      ss = stage_quarter<BITS, FMT, LPR>(p, qx, qg, qw, threadIdx.x, nunits, c0, nch, xl, info);
    }
  } else if constexpr (CPC >= 32) {
    // More quarter units than threads: the same quarter staging in uniform
    // rounds (every thread runs every round, so the quads' DPP sums see whole
    // chunks); the first round's x is requested before the weights. Holding
    // a whole chunk of x per thread instead (64 values for 2-bit codes) set
    // the register allocation of every 2-bit kernel to 190-203 VGPRs, one
    // workgroup per CU.
    // The first kPre rounds' x is requested before the weights: a request
    // made after them waits until the memory system has served them (the
    // 4096 x 14336 down projection staged its fourth round ~1.5 us late).
    const int rounds = (nunits + kThreads - 1) / kThreads;
    constexpr int kPre = CPC >= 64 ? 2 : 4;
    constexpr int QXN = CPC / 16, QGN = (CPC / 4 + 7) / 8;
    u32x4 pqx[kPre][QXN], pqg[kPre][QGN];
    float pqw[kPre];
#pragma unroll
    for (int r = 0; r < kPre; ++r) {
      if (r < rounds) {
        load_quarters_at(r * kThreads + (int)threadIdx.x);
#pragma unroll
        for (int i = 0; i < QXN; ++i) pqx[r][i] = qx[i];
#pragma unroll
        for (int i = 0; i < QGN; ++i) pqg[r][i] = qg[i];
        pqw[r] = qw;
      }
    }
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) issue(d[k]);
#pragma unroll
    for (int r = 0; r < kPre; ++r) {
      if (r < rounds) {
#pragma unroll
        for (int i = 0; i < QXN; ++i) hold(pqx[r][i]);
#pragma unroll
        for (int i = 0; i < QGN; ++i) hold(pqg[r][i]);
        hold(pqw[r]);
        ss += stage_quarter<BITS, FMT, LPR>(p, pqx[r], pqg[r], pqw[r], r * kThreads + (int)threadIdx.x, nunits,
                                            c0, nch, xl, info);
      }
    }
    for (int r = kPre; r < rounds; ++r) {
      const int u = r * kThreads + (int)threadIdx.x;
      load_quarters_at(u);
      ss += stage_quarter<BITS, FMT, LPR>(p, qx, qg, qw, u, nunits, c0, nch, xl, info);
    }
  } else if (npass * LPR <= kThreads) {
    XChunk<CPC> xc;
    const int c = threadIdx.x;
    stage_load<CPC>(p, xp, c0 + c, c < nch, xc);
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) issue(d[k]);
#pragma unroll
    for (int i = 0; i < CPC; ++i) hold(xc.v[i]);
#pragma unroll
    for (int i = 0; i < CPC / 8; ++i) hold(xc.g[i]);
    if (c < npass * LPR) ss = stage_chunk<BITS, FMT, LPR>(p, rwp, xc.v, xc.g, c, c0 + c, c < nch, xl, info);
  } else {
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) issue(d[k]);
    ss = stage_loop<BITS, FMT, LPR>(p, xp, rwp, c0, nch, npass, xl, info);
  }
  // RMSNorm scalar: applied to the row sums (W (g*x) / rms = W (g*x/rms)).
  // Whole K staged here: each wave sums its chunks' squares before the
  // barrier, the eight partials are added after it in fixed order.
  float rs = 1.0f;
  if (p.norm_w && !whole_k) rs = rms_all(p, xp, red);  // contains barriers: every thread
  if (p.norm_w && whole_k) {
    const float w_ss = lanes_sum<64>(ss);
    if (lane == 63) red[wave] = w_ss;
  }
  __syncthreads();
  if (p.norm_w && whole_k) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[w];
    rs = 1.0f / sqrtf(t / (float)p.K + p.eps);
  }

  float acc_a[R], acc_b[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc_a[r] = acc_b[r] = 0.f;
  int cur_band = tile * kWaves + wave, cur_pass = 0;

  int tk_n = 0;  // fused top-k: this wave's keys recorded so far (uniform)
  auto finish_band = [&](int band) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc_a[r] = lanes_sum<LPR>(acc_a[r]) * rs;
      if constexpr (TWO) acc_b[r] = lanes_sum<LPR>(acc_b[r]) * rs;
    }
    if (j == LPR - 1) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = band * RPB + sub * R + r;
        if constexpr (TOPK) {
          if (band < nbands) tk_keys[wave][tk_n + sub * R + r] = n < p.N ? order_key(acc_a[r], (uint32_t)n) : 0ull;
          if (n < p.N) handoff_store(&yp[n], acc_a[r]);  // read back by the last workgroup
          continue;
        }
        if (n < p.N) {
          if (p.splits > 1) {
            handoff_store(&p.partials[((size_t)slice * NACC) * p.N + n], acc_a[r]);
            if constexpr (TWO) handoff_store(&p.partials[((size_t)slice * NACC + 1) * p.N + n], acc_b[r]);
          } else if constexpr (TWO) {
            yp[n] = silu(acc_a[r]) * acc_b[r];
          } else {
            yp[n] = resp ? resp[n] + acc_a[r] : acc_a[r];
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc_a[r] = acc_b[r] = 0.f;
    if constexpr (TOPK) tk_n += band < nbands ? RPB : 0;
  };

  // Every slot runs on every round, also past the last band (zeros in, no
  // stores out), so that the loads of the loop stay on one straight path.
  while (cur_band < nbands) {
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) {
      if constexpr (FMT == 1) {
        if (cur_pass == 0) {  // this band's row tables into the sub-wave's LDS slot
          wave_sync_lds();
#pragma unroll
          for (int q = 0; q < LUTN; ++q) {
            const int e = j + q * LPR;  // entry t of table (r, m) at (r * NACC + m) * 16 + t
            if (e < R * NACC * 16) l16[e] = d[k].lut[q];
          }
          wave_sync_lds();
          // the pair tables: slot s of a table (64 per table) writes the four
          // pairs (lut[4(s&3) + i], lut[s>>2]), i = 0..3, at 16 (s>>2) + 4 (s&3)
#pragma unroll
          for (int s2 = j; s2 < R * NACC * 64; s2 += LPR) {
            const int tb = s2 >> 6, sl = s2 & 63;
            const uint16_t* L = l16 + tb * 16;
            const uint32_t hi = (uint32_t)L[sl >> 2] << 16;
            const int lo4 = 4 * (sl & 3);
            *reinterpret_cast<u32x4*>(ptab + tb * kLutPairWords + (sl >> 2) * 16 + lo4) =
                u32x4{L[lo4] | hi, L[lo4 + 1] | hi, L[lo4 + 2] | hi, L[lo4 + 3] | hi};
          }
          wave_sync_lds();
        }
      }
      if constexpr (SBL > 0) {
        if (cur_pass == 0) {  // this band's scale/bias rows into the wave's LDS area
          wave_sync_lds();
#pragma unroll
          for (int i = 0; i < SBL; ++i)
            if (lane + 64 * i < RPB * NACC * 2 * segp) sbw4[lane + 64 * i] = d[k].sbq[i];
          wave_sync_lds();
        }
      }
      compute_pass<BITS, FMT, LPR, R, TWO, LUTN, SBL>(d[k], xl, info, cur_pass, j, ptab, sbw, segp * 8, gsl,
                                                      acc_a, acc_b);
      issue(d[k]);
      if (++cur_pass == npass) {
        finish_band(cur_band);
        cur_pass = 0;
        cur_band += band_stride;
      }
    }
  }

  if constexpr (TOPK) {
    // Fused top-k (page "Booster la vitesse d'inference sur Apple Silicon",
    // section 1: logits matvec + top-k on the GPU). Keys order values larger
    // first, equal values by lower row, so every list below is a set with no
    // ties and each merge is exact: the workgroup's 64 largest keys, then a
    // group's, then the launch's. A list taken as the second operand of a
    // merge is read in reverse lane order (smaller first).
    static_assert(kTkGroup % kWaves == 0 && kTkMaxGroups % kWaves == 0, "lists per wave");
    // Merges the waves' lists (each sorted larger first) in three rounds of
    // pairs through LDS; wave 0 returns the result. Every thread calls it.
    auto merge_waves = [&](uint64_t a) -> uint64_t {
      tk_keys[wave][lane] = a;
      __syncthreads();
#pragma unroll
      for (int half = kWaves / 2; half >= 1; half >>= 1) {
        if (wave < half) {  // reads slots [half, 2 half), writes [0, half)
          a = wave_merge_top(a, tk_keys[wave + half][63 - lane]);
          tk_keys[wave][lane] = a;
        }
        __syncthreads();
      }
      return a;
    };
    // Wave w merges lists w, w + kWaves, ... (< n) of `base`; zeros past n.
    auto merge_strided = [&](const __amdgpu_buffer_rsrc_t r, int first, int n, auto per) -> uint64_t {
      constexpr int PER = decltype(per)::value;
      uint64_t b[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int t = wave + i * kWaves;
        b[i] = coherent_u64(r, t < n ? (uint32_t)(((first + t) * kTkList + (i ? 63 - lane : lane)) * 8) : kOOB);
      }
      uint64_t a = b[0];
#pragma unroll
      for (int i = 1; i < PER; ++i)
        if (wave + i * kWaves < n) a = wave_merge_top(a, b[i]);
      return a;
    };
    wave_sync_lds();
    uint64_t v = lane < tk_n ? tk_keys[wave][lane] : 0ull;
    v = merge_waves(wave_sort_desc(v));
    const int ngroups = (p.grid_x + kTkGroup - 1) / kTkGroup;
    uint64_t* const wg_lists = p.tk_cand;
    uint64_t* const grp_lists = p.tk_cand + (size_t)p.grid_x * kTkList;
    if (wave == 0) handoff_store(&wg_lists[(size_t)tile * kTkList + lane], v);
    stores_done();  // this workgroup's logits and list, before its ticket
    __syncthreads();
    const int g = tile / kTkGroup;
    const int g0 = g * kTkGroup, gsize = min(kTkGroup, p.grid_x - g0);
    if (threadIdx.x == 0) last_flag = take_ticket(&p.tk_tickets[g]) == (uint32_t)(gsize - 1);
    __syncthreads();
    if (!last_flag) return;
    // the group's last workgroup merges its lists
    v = merge_strided(make_rsrc(wg_lists, (uint32_t)(p.grid_x * kTkList * 8)), g0, gsize,
                      std::integral_constant<int, kTkGroup / kWaves>{});
    v = merge_waves(v);
    if (wave == 0) {
      handoff_store(&grp_lists[(size_t)g * kTkList + lane], v);
      if (lane == 0) handoff_store(&p.tk_tickets[g], 0u);  // ready for the next call
    }
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) last_flag = take_ticket(&p.tk_tickets[kTkMaxGroups]) == (uint32_t)(ngroups - 1);
    __syncthreads();
    if (!last_flag) return;
    // the last group merger: the launch's k largest, larger first
    v = merge_strided(make_rsrc(grp_lists, (uint32_t)(ngroups * kTkList * 8)), 0, ngroups,
                      std::integral_constant<int, kTkMaxGroups / kWaves>{});
    v = merge_waves(v);
    if (wave == 0) {
      if (lane < p.tk_k) {
        const uint32_t i = key_index(v);
        float val = key_value(v);
        // a zero (its sign) and a NaN (its payload) come back from memory
        if (val == 0.f || val != val) val = coherent_f32(make_rsrc(yp, (uint32_t)p.N * 4u), i * 4u);
        p.tk_idx[lane] = (int32_t)i;
        p.tk_vals[lane] = val;
      }
      if (lane == 0) handoff_store(&p.tk_tickets[kTkMaxGroups], 0u);
      if (p.tk_draw.token) {
        // and one token drawn from them, as the two-launch form draws it
        // (tk_keys[0] holds the sorted list, tk_keys[1] is free for the weights)
        draw_token(
            p.tk_k, [&](int i) { return key_value(tk_keys[0][i]); },
            [&](int i) { return (int32_t)key_index(tk_keys[0][i]); }, p.tk_draw,
            reinterpret_cast<double*>(&tk_keys[1][0]));
      }
    }
    return;
  }

  if (p.splits > 1) {
    // Last workgroup of this tile adds the slices in fixed order: the partial
    // stores are complete before the barrier, then one thread takes the ticket.
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) last_flag = take_ticket(&p.tickets[tile]) == (uint32_t)(p.splits - 1);
    __syncthreads();
    if (!last_flag) return;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.partials, (uint32_t)(p.splits * NACC * p.N * 4));
    const uint32_t sstride = (uint32_t)(NACC * p.N * 4);
    for (int band = tile * kWaves + wave; band < nbands; band += band_stride) {
      if (lane < RPB) {
        const int n = band * RPB + lane;
        if (n < p.N) {
          const float a = coherent_sum(rp, (uint32_t)n * 4u, sstride, p.splits);
          const float b = TWO ? coherent_sum(rp, (uint32_t)(p.N + n) * 4u, sstride, p.splits) : 0.f;
          if constexpr (TWO) {
            yp[n] = silu(a) * b;
          } else {
            yp[n] = resp ? resp[n] + a : a;
          }
        }
      }
    }
    if (threadIdx.x == 0) handoff_store(&p.tickets[tile], 0u);  // ready for the next call on this stream
  }
}

__global__ void fill_u32_kernel(uint32_t* dst, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = v;
}

typedef void (*KernelFn)(const MvParams);

// sbl: staged scale/bias rows (affine formats with one K segment; the host
// asks for them only where the rows are 16-byte aligned and fit).
template <int BITS, int FMT, int EPI, int SEG, int LPR>
KernelFn pick_rd(int rows, int depth, int sbl) {
  constexpr bool kSb = FMT == 0 && SEG != kSegCols;
  if (rows == 2) {  // two rows: depth 2 only
    // (two rows of two matrices stage four row segments: more than two loads
    // per lane at the K >= 8192 that takes two rows)
    if constexpr (kSb && EPI != kEpiSwiglu) {
      if (sbl) return qmv_kernel<BITS, FMT, LPR, 2, EPI, SEG, 2, 2>;
    }
    return qmv_kernel<BITS, FMT, LPR, 2, EPI, SEG, 2, 0>;
  }
  if constexpr (kSb) {
    if (sbl)
      return depth == 4 ? qmv_kernel<BITS, FMT, LPR, 1, EPI, SEG, 4, 1> : qmv_kernel<BITS, FMT, LPR, 1, EPI, SEG, 2, 1>;
  }
  return depth == 4 ? qmv_kernel<BITS, FMT, LPR, 1, EPI, SEG, 4, 0> : qmv_kernel<BITS, FMT, LPR, 1, EPI, SEG, 2, 0>;
}

template <int BITS, int FMT, int EPI, int SEG>
KernelFn pick_kernel(int lpr, int rows, int depth, int sbl) {
  if (lpr == 64) return pick_rd<BITS, FMT, EPI, SEG, 64>(rows, depth, sbl);
  if (lpr == 32) return pick_rd<BITS, FMT, EPI, SEG, 32>(rows, depth, sbl);
  if (lpr == 16) return pick_rd<BITS, FMT, EPI, SEG, 16>(rows, depth, sbl);
  return nullptr;
}

// the fused top-k: one row per lane slot, pipeline depth 2
template <int BITS, int FMT, int LPR>
KernelFn pick_topk(int rows, int sbl) {
  if (rows != 1) return nullptr;
  if constexpr (FMT == 0) {
    if (sbl) return qmv_kernel<BITS, FMT, LPR, 1, kEpiTopk, kSegNone, 2, 1>;
  }
  return qmv_kernel<BITS, FMT, LPR, 1, kEpiTopk, kSegNone, 2, 0>;
}

template <int BITS, int FMT>
KernelFn pick_kernel_epi(int epi, int seg, int lpr, int rows, int depth, int sbl) {
  if (epi == kEpiTopk) {
    if (seg != kSegNone) return nullptr;
    if (lpr == 64) return pick_topk<BITS, FMT, 64>(rows, sbl);
    if (lpr == 32) return pick_topk<BITS, FMT, 32>(rows, sbl);
    if (lpr == 16) return pick_topk<BITS, FMT, 16>(rows, sbl);
    return nullptr;
  }
  if constexpr (FMT != 0) {  // the LUT and dense formats are not gathered by experts
    if (seg != kSegNone) return nullptr;
    if (epi == kEpiStore) return pick_kernel<BITS, FMT, kEpiStore, kSegNone>(lpr, rows, depth, 0);
    if (epi == kEpiSwiglu) return pick_kernel<BITS, FMT, kEpiSwiglu, kSegNone>(lpr, rows, depth, 0);
    return nullptr;
  } else {
    if (epi == kEpiStore) {
      if (seg == kSegNone) return pick_kernel<BITS, FMT, kEpiStore, kSegNone>(lpr, rows, depth, sbl);
      if (seg == kSegCols) return pick_kernel<BITS, FMT, kEpiStore, kSegCols>(lpr, rows, depth, 0);
    } else if (epi == kEpiSwiglu) {
      if (seg == kSegNone) return pick_kernel<BITS, FMT, kEpiSwiglu, kSegNone>(lpr, rows, depth, sbl);
      if (seg == kSegRows) return pick_kernel<BITS, FMT, kEpiSwiglu, kSegRows>(lpr, rows, depth, sbl);
    }
    return nullptr;
  }
}

}  // namespace

namespace {
KernelFn select_mv(int bits, int fmt, int epi, int seg, const MvPlan& plan) {
  const int sbl = plan.sbl;
  if (bits == 4 && fmt == 0) return pick_kernel_epi<4, 0>(epi, seg, plan.lpr, plan.rows, plan.depth, sbl);
  if (bits == 2 && fmt == 0) return pick_kernel_epi<2, 0>(epi, seg, plan.lpr, plan.rows, plan.depth, sbl);
  if (bits == 8 && fmt == 0) return pick_kernel_epi<8, 0>(epi, seg, plan.lpr, plan.rows, plan.depth, sbl);
  if (bits == 16 && fmt == 2 && seg == kSegNone)
    return pick_kernel_epi<16, 2>(epi, seg, plan.lpr, plan.rows, plan.depth, 0);
  if (bits == 4 && fmt == 1 && seg == kSegNone)
    return pick_kernel_epi<4, 1>(epi, seg, plan.lpr, plan.rows, plan.depth, 0);
  return nullptr;
}
}  // namespace

int mv_resident_per_cu(int bits, int fmt, int epi, int seg, const MvPlan& plan) {
  const KernelFn fn = select_mv(bits, fmt, epi, seg, plan);
  if (!fn) return 1;
  static std::mutex mu;
  static std::unordered_map<const void*, int> cache;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find((const void*)fn);
  if (it != cache.end()) return it->second;
  int n = 0;
  // registers decide; the dynamic LDS of one workgroup is at most kMaxLdsBytes
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)fn, kThreads, kMaxLdsBytes) !=
          hipSuccess ||
      n < 1)
    n = 1;
  cache[(const void*)fn] = n;
  return n;
}

hipError_t launch_mv(int bits, int fmt, int epi, const MvPlan& plan, const MvParams& p,
                     hipStream_t stream) {
  const KernelFn fn = select_mv(bits, fmt, epi, p.seg_mode, plan);
  if (!fn) return hipErrorInvalidValue;
  if (plan.lds_bytes > (size_t)kMaxLdsBytes) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(plan.grid_x * plan.splits * (plan.tokens > 1 ? plan.tokens : 1)));
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
