// qg_mm.hip -- the small-M decode matvec (M = 2..8 activation vectors) on the
// matrix cores of gfx950.
//
// Y[m][n] = R[m][n] + sum_k W[n][k] X[m][k] with W planar 4-bit or 2-bit,
// group 64, or 4-bit codes into a per-row 16-entry table (page "Booster la
// vitesse d'inference sur Apple Silicon", section 1: the dispatcher routes by
// M; section 3 item 4: planar codes + scale + bias). With several activation
// vectors the per-weight work is a dense contraction, so it goes to
// v_mfma_f32_16x16x32_f16: A = 16 activation rows (M used) x 32 k, B = 32 k x
// 16 weight rows, D = 16 x 16 fp32 (token x weight row).
//
// Work split. A workgroup (8 waves) owns a K slice of 8 x 512 codes and a set
// of 16-row bands; wave w owns 512 consecutive codes of the slice. Its share
// of X (M x 512 values, as fp16 MFMA operands) is staged once into registers,
// so the inner loop reads no activations at all. For each band the wave
// streams its 16 x 512 codes (one 16-byte load per lane per item of four
// chunks), turns the loads into B operands with a 4 x 4 exchange across the
// four 16-lane rows (v_permlane32_swap / v_permlane16_swap, no LDS), and
// issues one MFMA per 32 codes. The eight waves' results for a band are summed
// in LDS in a fixed order. K longer than one slice is split across
// workgroups, combined by the last one to finish (integer ticket).
//
// Arithmetic (page "Optimisation FMA du noyau de dequantification":
// fma(code, s*x, b*x) per group). Codes become fp16 operands exactly: masking
// a word with 0x000F000F gives two fp16 bit patterns equal to code*2^-24
// (subnormals, kept exact by the matrix cores); the matching activations are
// prescaled by 1/16, 1/64, ... where the mask leaves a code shifted left.
// Each token's activations are scaled by one power of two so that its largest
// magnitude over the wave's range sits in [2^13, 2^14); D then carries the
// factor 2^-24 * 2^-e. Per group the fp32 D is folded in as acc += s * D; the
// bias term sum_g b_g * sum_{k in g} x_k is one more MFMA whose A operand holds
// the group sums (split in two fp16 parts, hi + lo) in the same scaled units.
// The wave's result is multiplied by 2^(24+e) once per band. The table format
// uses the looked-up fp16 entries as the B operand and natural-order
// activations, with no scale or bias.
#include "qg_common.h"

namespace qg {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBand = 16;       // weight rows per band (MFMA B columns)
constexpr int kTok = 8;         // activation vectors (MFMA A rows used)
constexpr int kGW = 8;          // groups of 64 per wave range (512 codes)
constexpr int kLutStride = 18;  // halves per row of a wave's table copy (16 + 2 pad)

template <int BITS, int FMT>
struct MmGeo;
template <>
struct MmGeo<4, 0> {  // 32 codes per 16-byte chunk, one MFMA per chunk, 2 chunks per group
  static constexpr int kCodes = 32, kSteps = 1, kCPG = 2;
};
template <>
struct MmGeo<2, 0> {  // 64 codes per chunk, two MFMAs per chunk, 1 chunk per group
  static constexpr int kCodes = 64, kSteps = 2, kCPG = 1;
};
template <>
struct MmGeo<4, 1> {  // table format: as 4-bit, no scale/bias
  static constexpr int kCodes = 32, kSteps = 1, kCPG = 2;
};

__device__ __forceinline__ f16x8 f16x8_of(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(f16x8, u32x4{a, b, c, d});
}

// 4 x 4 exchange across the 16-lane rows: on entry row r holds words 0..3 of
// its own chunk r; on exit row r holds word r of chunks 0..3 (w[c]).
__device__ __forceinline__ void cross_rows_4x4(uint32_t& w0, uint32_t& w1, uint32_t& w2,
                                               uint32_t& w3) {
  // rows 2,3 of w0/w1 <-> rows 0,1 of w2/w3
  auto a = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
  w0 = a[0];
  w2 = a[1];
  w1 = b[0];
  w3 = b[1];
  // rows 1,3 of w0/w2 <-> rows 0,2 of w1/w3
  auto c = __builtin_amdgcn_permlane16_swap(w0, w1, false, false);
  auto d = __builtin_amdgcn_permlane16_swap(w2, w3, false, false);
  w0 = c[0];
  w1 = c[1];
  w2 = d[0];
  w3 = d[1];
}

// B operand of step h for one code word (affine formats): eight fp16 code
// values code*2^-24 (times 16^j / 4^j where the mask leaves them shifted), in
// the order the activation operand is staged.
template <int BITS>
__device__ __forceinline__ f16x8 code_operand(uint32_t w, int h) {
  if constexpr (BITS == 4) {
    const uint32_t t = w >> 8;
    return f16x8_of(w & 0x000F000Fu, w & 0x00F000F0u, t & 0x000F000Fu, t & 0x00F000F0u);
  } else {
    if (h == 0) return f16x8_of(w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u);
    const uint32_t t = w >> 10;
    return f16x8_of(w & 0x03000300u, t & 0x00030003u, t & 0x000C000Cu, t & 0x00300030u);
  }
}

// B operand for the table format: the eight nibbles of w looked up in the
// lane's row of the wave's table copy (LDS).
__device__ __forceinline__ f16x8 lut_operand(uint32_t w, const uint16_t* t) {
  uint32_t d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = t[(w >> (8 * j)) & 15u];
    const uint32_t hi = t[(w >> (8 * j + 4)) & 15u];
    d[j] = lo | (hi << 16);
  }
  return f16x8_of(d[0], d[1], d[2], d[3]);
}

// Activation operand(s) of one 64-code group, from 16 values v (this lane's
// share, already multiplied by 2^-e_g): 4-bit and table format hold elements
// 8q..8q+7 of two chunks; 2-bit holds elements 16q..16q+15 of one chunk.
template <int BITS, int FMT>
__device__ __forceinline__ void group_operands(const float* v, f16x8* dst) {
  if constexpr (FMT == 1) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float* u = v + 8 * c;
      dst[c] = f16x8_of(pack_f16(u[0], u[1]), pack_f16(u[2], u[3]), pack_f16(u[4], u[5]),
                        pack_f16(u[6], u[7]));
    }
  } else if constexpr (BITS == 4) {
    constexpr float r16 = 1.0f / 16.0f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float* u = v + 8 * c;
      dst[c] = f16x8_of(pack_f16(u[0], u[4]), pack_f16(u[1] * r16, u[5] * r16),
                        pack_f16(u[2], u[6]), pack_f16(u[3] * r16, u[7] * r16));
    }
  } else {
    constexpr float r4 = 0.25f, r16 = 1.0f / 16.0f, r64 = 1.0f / 64.0f, r256 = 1.0f / 256.0f;
    dst[0] = f16x8_of(pack_f16(v[0], v[8]), pack_f16(v[1] * r4, v[9] * r4),
                      pack_f16(v[2] * r16, v[10] * r16), pack_f16(v[3] * r64, v[11] * r64));
    dst[1] = f16x8_of(pack_f16(v[4] * r256, v[12] * r256), pack_f16(v[5], v[13]),
                      pack_f16(v[6] * r4, v[14] * r4), pack_f16(v[7] * r16, v[15] * r16));
  }
}

// Materializes a value in registers at this point (keeps the compiler from
// carrying the fp32 inputs of a packed operand further down).
__device__ __forceinline__ void pin(f16x8& v) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
  asm volatile("" : "+v"(u));
  v = __builtin_bit_cast(f16x8, u);
}

__device__ __forceinline__ float xor_lanes(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Exponent e with max|x| * 2^-e in [2^13, 2^14), or kNoExp for an all-zero range.
constexpr int kNoExp = -100000;
__device__ __forceinline__ int range_exp(float m) {
  if (!(m > 0.f) || !(m < INFINITY)) return kNoExp;
  int E = 0;
  frexpf(m, &E);
  return E - 14;
}

__device__ __forceinline__ uint32_t dup_lo(uint32_t w) { return (w & 0xFFFFu) | (w << 16); }
__device__ __forceinline__ uint32_t dup_hi(uint32_t w) { return (w >> 16) | (w & 0xFFFF0000u); }

__device__ __forceinline__ float half_of(const uint32_t* words, int h) {
  const uint32_t w = words[h >> 1];
  return f16_bits_to_f32((uint16_t)((h & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

template <int BITS, int FMT, int EPI>
__global__ __launch_bounds__(kThreads) void qmm_kernel(const MvParams p) {
  using G = MmGeo<BITS, FMT>;
  constexpr int CODES = G::kCodes, STEPS = G::kSteps, CPG = G::kCPG;
  constexpr int KW = kGW * CPG;  // chunks per wave range
  constexpr int IPB = KW / 4;    // items (4 chunks) per band
  constexpr int NACC = EPI == kEpiSwiglu ? 2 : 1;
  constexpr bool LUT = FMT == 1;
  constexpr int BACK_BIAS = LUT ? 0 : 24;
  // bands in flight per wave: about 8 KB of codes per wave
  constexpr int DB = (BITS == 2 && !LUT ? 4 : 2) / NACC;

  __shared__ float red[2][NACC][kWaves][kTok][kBand];
  __shared__ float ssq[kWaves][kTok];
  __shared__ float bk[kWaves][kTok];
  __shared__ uint16_t luts[LUT ? kWaves : 1][kBand * kLutStride];
  __shared__ int last_flag;

  const int slice = blockIdx.x / p.grid_x;
  const int tile = blockIdx.x - slice * p.grid_x;
  const int nbands = (p.N + kBand - 1) / kBand;
  if (tile >= nbands) return;  // padding workgroup (same tiles are idle in every slice)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;    // row of the wave: chunk loaded, word held, D rows 4q..4q+3
  const int col = lane & 15;  // A row (token) / B column (weight row) of this lane
  const int M = p.M;
  const int C = p.K / CODES;
  const int cw0 = (slice * kWaves + wave) * KW;  // first chunk of this wave's range
  const int gw0 = cw0 / CPG;                     // first group of this wave's range
  const bool norm = p.norm_w != nullptr;

  QMat mats[2] = {p.A[0], EPI == kEpiSwiglu ? p.B[0] : p.A[0]};
  MatRsrc rs_[NACC];
  __amdgpu_buffer_rsrc_t rl[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) {
    rs_[a] = mat_rsrc(mats[a], p.N, p.wpr, p.gpr);
    if constexpr (LUT) rl[a] = make_rsrc(mats[a].lut, (uint32_t)p.N * 32u);
  }

  // ---- loads ----------------------------------------------------------------
  // DB bands in flight per wave, in a ring of slots indexed at compile time.
  u32x4 cq[NACC][DB][IPB];   // codes: one 16-byte chunk per lane per item
  uint32_t sq[NACC][DB][4];  // scales of groups gw0..gw0+7 of the lane's row (8 halves)
  uint32_t bq[NACC][DB][2];  // biases of groups gw0+4q..gw0+4q+3 (rows q < 2), or
                             // table entries 4q..4q+3 of the row (table format)
  const bool range_ok = gw0 < p.gpr;  // wave-uniform: this wave has codes in this slice

  auto issue_item = [&](int band, int it, int a, int d) {
    const int ch = cw0 + 4 * it + q;
    const bool ok = band < nbands && ch < C;
    const uint32_t n = (uint32_t)(band * kBand + col);
    const uint32_t off = ok ? n * (uint32_t)p.wpr * 4u + (uint32_t)ch * 16u : kOOB;
    cq[a][d][it] = __builtin_amdgcn_raw_buffer_load_b128(rs_[a].q, off, 0, 2);
  };
  auto issue_rowdata = [&](int band, int a, int d) {
    const bool okb = band < nbands;
    const uint32_t n = (uint32_t)(band * kBand + col);
    if constexpr (LUT) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rl[a], okb ? n * 32u + (uint32_t)q * 8u : kOOB, 0, 0);
      bq[a][d][0] = v[0];
      bq[a][d][1] = v[1];
    } else {
      const uint32_t off = (okb && range_ok) ? n * (uint32_t)p.gpr * 2u + (uint32_t)gw0 * 2u : kOOB;
      const u32x4 sv = __builtin_amdgcn_raw_buffer_load_b128(rs_[a].s, off, 0, 0);
      sq[a][d][0] = sv.x;
      sq[a][d][1] = sv.y;
      sq[a][d][2] = sv.z;
      sq[a][d][3] = sv.w;
      const auto bv = __builtin_amdgcn_raw_buffer_load_b64(rs_[a].b, q < 2 ? off + 8u * q : kOOB, 0, 0);
      bq[a][d][0] = bv[0];
      bq[a][d][1] = bv[1];
    }
  };
  auto issue_band = [&](int band, int a, int d) {
#pragma unroll
    for (int it = 0; it < IPB; ++it) issue_item(band, it, a, d);
    issue_rowdata(band, a, d);
  };

  int band = tile;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int a = 0; a < NACC; ++a) issue_band(band + d * p.grid_x, a, d);
  asm volatile("" ::: "memory");

  // ---- stage this wave's share of X into registers --------------------------
  // Lane (q, col) holds token col; for group g its 16 values are elements
  // 8q..8q+7 of chunks 2g, 2g+1 (4-bit, table) or 16q..16q+15 of chunk g (2-bit).
  f16x8 xa[KW * STEPS];
  float gsum[kGW];
  int ge[kGW];
  float ssum = 0.f;
  const bool tok_ok = col < M;
  const char* xrow = static_cast<const char*>(p.x) + (size_t)(tok_ok ? col : 0) * p.K * (p.x_f32 ? 4 : 2);
#pragma unroll
  for (int g = 0; g < kGW; ++g) {
    float v[16];
    const bool ok = tok_ok && gw0 + g < p.gpr;
    int k0[2];
    if constexpr (BITS == 2 && !LUT) {
      k0[0] = (gw0 + g) * 64 + 16 * q;
      k0[1] = k0[0] + 8;
    } else {
      k0[0] = (cw0 + 2 * g) * 32 + 8 * q;
      k0[1] = k0[0] + 32;
    }
    if (ok) {
      load_x<8>(xrow, p.x_f32, k0[0], v);
      load_x<8>(xrow, p.x_f32, k0[1], v + 8);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.f;
    }
    if (norm) {
      float gv[16];
      if (ok) {
        load_f16<8>(p.norm_w, k0[0], gv);
        load_f16<8>(p.norm_w, k0[1], gv + 8);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ssum = fmaf(v[i], v[i], ssum);
        if (ok) v[i] *= gv[i];
      }
    }
    float s = 0.f, m = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s += v[i];
      m = fmaxf(m, fabsf(v[i]));
    }
    s += xor_lanes(s, 16);
    s += xor_lanes(s, 32);
    m = fmaxf(m, xor_lanes(m, 16));
    m = fmaxf(m, xor_lanes(m, 32));
    gsum[g] = s;
    ge[g] = range_exp(m);
    const float inv = ldexpf(1.0f, ge[g] == kNoExp ? 0 : -ge[g]);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= inv;
    group_operands<BITS, FMT>(v, &xa[g * 2]);
    pin(xa[g * 2]);
    pin(xa[g * 2 + 1]);
    if (g & 1) asm volatile("" ::: "memory");  // bound the loads in flight
  }
  // one exponent per token over the range: rescale each group's operands by
  // 2^(e_g - E) (a power of two <= 1, exact unless it drops into subnormals)
  int E = kNoExp;
#pragma unroll
  for (int g = 0; g < kGW; ++g) E = max(E, ge[g]);
  if (E == kNoExp) E = 0;
#pragma unroll
  for (int g = 0; g < kGW; ++g) {
    const int d = ge[g] == kNoExp ? 0 : ge[g] - E;
    if (d != 0) {
      const _Float16 f = (_Float16)ldexpf(1.0f, max(d, -30));
      xa[2 * g] *= f;
      xa[2 * g + 1] *= f;
    }
  }
  // bias operand: lane row q < 2 carries groups 4q..4q+3 as (hi, lo) pairs of
  // sum_x * 2^-(24+E), the units of D
  f16x8 xb = f16x8_of(0u, 0u, 0u, 0u);
  if constexpr (!LUT) {
    uint32_t d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float t = ldexpf(q == 0 ? gsum[j] : gsum[4 + j], -(BACK_BIAS + E));
      const _Float16 hi = (_Float16)t;
      const _Float16 lo = (_Float16)(t - (float)hi);
      d[j] = q < 2 ? ((uint32_t)__builtin_bit_cast(uint16_t, hi) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16))
                   : 0u;
    }
    xb = f16x8_of(d[0], d[1], d[2], d[3]);
  }
  // factor that undoes this wave's scaling of token col (applied in the band sums)
  if (q == 0 && col < kTok) bk[wave][col] = ldexpf(1.0f, BACK_BIAS + E);

  // sum of squares per token for the norm: this slice's share, or all of K
  // when the row is split over several workgroups
  if (norm) {
    if (p.splits > 1) {
      for (int j = 0; j < M; ++j) {
        float part = 0.f;
        const char* xj = static_cast<const char*>(p.x) + (size_t)j * p.K * (p.x_f32 ? 4 : 2);
        for (int k = threadIdx.x * 8; k < p.K; k += kThreads * 8) {
          float v[8];
          load_x<8>(xj, p.x_f32, k, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) part = fmaf(v[i], v[i], part);
        }
        part = wave_sum(part);
        if (lane == 0) ssq[wave][j] = part;
      }
    } else {
      ssum += xor_lanes(ssum, 16);
      ssum += xor_lanes(ssum, 32);
      if (q == 0 && col < M) ssq[wave][col] = ssum;
    }
  }
  __syncthreads();
  // the thread that finishes output (token ot, row orow) of each band
  const int ot = threadIdx.x >> 4, orow = threadIdx.x & 15;
  const bool out_thread = threadIdx.x < kBand * M;
  float rs = 1.f;
  if (norm && out_thread) {
    float t = 0.f;
    for (int w = 0; w < kWaves; ++w) t += ssq[w][ot];
    rs = 1.0f / sqrtf(t / (float)p.K + p.eps);
  }

  auto finish = [&](int n, const float* v) {
    const size_t o = (size_t)ot * p.N + n;
    if constexpr (EPI == kEpiSwiglu) {
      p.y[o] = silu(v[0] * rs) * (v[1] * rs);
    } else {
      const float r = v[0] * rs;
      p.y[o] = p.residual ? p.residual[o] + r : r;
    }
  };

  // ---- bands ------------------------------------------------------------------
  const uint16_t* trow = LUT ? &luts[LUT ? wave : 0][col * kLutStride] : nullptr;
  int slot = 0;
  auto run_band = [&](int d) {
    const int ahead = band + DB * p.grid_x;  // the band that reuses slot d
    f32x4 acc[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (LUT) {
        // this band's table rows into the wave's LDS copy
        wave_sync_lds();
        uint32_t* t32 = reinterpret_cast<uint32_t*>(&luts[wave][col * kLutStride + 4 * q]);
        t32[0] = bq[a][d][0];
        t32[1] = bq[a][d][1];
        wave_sync_lds();
      }
#pragma unroll
      for (int it = 0; it < IPB; ++it) {
        uint32_t w[4] = {cq[a][d][it].x, cq[a][d][it].y, cq[a][d][it].z, cq[a][d][it].w};
        issue_item(ahead, it, a, d);
        asm volatile("" ::: "memory");
        cross_rows_4x4(w[0], w[1], w[2], w[3]);
        f32x4 dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int k = 4 * it + c;  // chunk within the wave range
          if constexpr (LUT) {
            acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[k], lut_operand(w[c], trow), acc[a], 0, 0, 0);
          } else {
            if (k % CPG == 0) dacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int h = 0; h < STEPS; ++h)
              dacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[k * STEPS + h], code_operand<BITS>(w[c], h), dacc, 0, 0, 0);
            if (k % CPG == CPG - 1) {
              const float sg = half_of(sq[a][d], k / CPG);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[a][i] = fmaf(sg, dacc[i], acc[a][i]);
            }
          }
        }
      }
      if constexpr (!LUT) {
        const f16x8 bb = f16x8_of(dup_lo(bq[a][d][0]), dup_hi(bq[a][d][0]), dup_lo(bq[a][d][1]),
                                  dup_hi(bq[a][d][1]));
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xb, bb, acc[a], 0, 0, 0);
      }
      issue_rowdata(ahead, a, d);
      asm volatile("" ::: "memory");
    }

    // sum the eight waves' shares of this band in a fixed order
    if (q < 2) {
#pragma unroll
      for (int a = 0; a < NACC; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[slot][a][wave][4 * q + i][col] = acc[a][i];
    }
    __syncthreads();
    if (out_thread) {
      const int n = band * kBand + orow;
      if (n < p.N) {
        float v[NACC];
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
          float t = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) t = fmaf(red[slot][a][w][ot][orow], bk[w][ot], t);
          v[a] = t;
        }
        if (p.splits > 1) {
#pragma unroll
          for (int a = 0; a < NACC; ++a)
            p.partials[(((size_t)slice * NACC + a) * M + ot) * p.N + n] = v[a];
        } else {
          finish(n, v);
        }
      }
    }
    slot ^= 1;
    band += p.grid_x;
  };
  while (band < nbands) {
#pragma unroll
    for (int d = 0; d < DB; ++d)
      if (band < nbands) run_band(d);
  }

  if (p.splits > 1) {
    __syncthreads();
    if (threadIdx.x == 0) {
      __threadfence();
      const uint32_t prev = atomicAdd(&p.tickets[tile], 1u);
      last_flag = (prev == (uint32_t)(p.splits - 1));
      if (last_flag) __threadfence();
    }
    __syncthreads();
    if (!last_flag) return;
    if (out_thread) {
      for (int b = tile; b < nbands; b += p.grid_x) {
        const int n = b * kBand + orow;
        if (n >= p.N) continue;
        float v[NACC];
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
          float t = 0.f;
          for (int s = 0; s < p.splits; ++s)
            t += __builtin_nontemporal_load(&p.partials[(((size_t)s * NACC + a) * M + ot) * p.N + n]);
          v[a] = t;
        }
        finish(n, v);
      }
    }
    if (threadIdx.x == 0) p.tickets[tile] = 0u;
  }
}

}  // namespace

int mm_slice_codes() { return kWaves * kGW * 64; }

hipError_t launch_mm(int bits, int fmt, int epi, const MvPlan& plan, const MvParams& p,
                     hipStream_t stream) {
  void (*fn)(const MvParams) = nullptr;
  const bool sw = epi == kEpiSwiglu;
  if (fmt == 1) fn = sw ? qmm_kernel<4, 1, kEpiSwiglu> : qmm_kernel<4, 1, kEpiStore>;
  else if (bits == 4) fn = sw ? qmm_kernel<4, 0, kEpiSwiglu> : qmm_kernel<4, 0, kEpiStore>;
  else if (bits == 2) fn = sw ? qmm_kernel<2, 0, kEpiSwiglu> : qmm_kernel<2, 0, kEpiStore>;
  if (!fn) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3((unsigned)(plan.grid_x * plan.splits)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace qg
