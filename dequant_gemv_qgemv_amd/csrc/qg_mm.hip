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
// of X (M x 512 values) is converted once, spread evenly over the wave's 64
// lanes, and handed through LDS into registers as fp16 MFMA operands, so the
// inner loop reads no activations at all. For each band the wave
// streams its 16 x 512 codes in loads of 8 rows x 128 bytes (whole cache
// lines), regroups them with a DPP half-row rotation and a 4 x 4 exchange
// across the four 16-lane rows (v_permlane32_swap / v_permlane16_swap, no
// LDS) so that each lane holds one row's words, and issues one MFMA per 32
// codes. The eight waves' results for a band are summed
// in LDS in a fixed order. K longer than one slice is split across
// workgroups, combined by the last one to finish (integer ticket), which
// also takes the norm from every slice's sums of squares.
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

// The value of lane (i + 8) % 16 of the same 16-lane row (DPP row_ror:8).
__device__ __forceinline__ uint32_t row_ror8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over the 4 lanes of a quad (every lane gets the same bits).
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  return v + dpp<0x4E>(v);  // quad_perm [2,3,0,1]
}
// Max over the 32 lanes of each wave half (rows 0-1, rows 2-3).
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp<0x140>(v));  // row_mirror
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
// Sum over the 32 lanes of each wave half; exact in lane 0 / 32 of the half.
__device__ __forceinline__ float half_sum(float v) {
  v = quad_sum(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// The two operand pieces of one conversion job (16 activations of one group,
// already scaled): 4-bit and table format: elements 8q'..8q'+7 of one chunk for
// two consecutive q'; 2-bit: steps 0 and 1 of one q.
template <int BITS, int FMT>
__device__ __forceinline__ void job_pieces(const float* v, u32x4* out) {
  if constexpr (FMT == 1) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float* u = v + 8 * c;
      out[c] = u32x4{pack_f16(u[0], u[1]), pack_f16(u[2], u[3]), pack_f16(u[4], u[5]),
                     pack_f16(u[6], u[7])};
    }
  } else if constexpr (BITS == 4) {
    constexpr float r16 = 1.0f / 16.0f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float* u = v + 8 * c;
      out[c] = u32x4{pack_f16(u[0], u[4]), pack_f16(u[1] * r16, u[5] * r16),
                     pack_f16(u[2], u[6]), pack_f16(u[3] * r16, u[7] * r16)};
    }
  } else {
    constexpr float r4 = 0.25f, r16 = 1.0f / 16.0f, r64 = 1.0f / 64.0f, r256 = 1.0f / 256.0f;
    out[0] = u32x4{pack_f16(v[0], v[8]), pack_f16(v[1] * r4, v[9] * r4),
                   pack_f16(v[2] * r16, v[10] * r16), pack_f16(v[3] * r64, v[11] * r64)};
    out[1] = u32x4{pack_f16(v[4] * r256, v[12] * r256), pack_f16(v[5], v[13]),
                   pack_f16(v[6] * r4, v[14] * r4), pack_f16(v[7] * r16, v[15] * r16)};
  }
}
// Operand index within the half range (P) and lane row (q) of a job's two
// pieces, for group gl (0..3 within the half) and quarter r.
template <int BITS, int FMT>
__device__ __forceinline__ void job_slots(int gl, int r, int* P0, int* q0, int* P1, int* q1) {
  if constexpr (BITS == 2 && FMT == 0) {  // chunk = group; steps 0, 1 of row r
    *P0 = 2 * gl;
    *P1 = 2 * gl + 1;
    *q0 = *q1 = r;
  } else {  // chunk 2gl + r/2; rows 2(r&1), 2(r&1)+1
    *P0 = *P1 = 2 * gl + (r >> 1);
    *q0 = 2 * (r & 1);
    *q1 = *q0 + 1;
  }
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
  constexpr int NLI = KW / 8;    // line items (8 chunks = one 128-byte line per row) per band
  constexpr int NACC = EPI == kEpiSwiglu ? 2 : 1;
  constexpr bool LUT = FMT == 1;
  constexpr int BACK_BIAS = LUT ? 0 : 24;
  // bands in flight per wave: about 8 KB of codes per wave
  constexpr int DB = (BITS == 2 && !LUT ? 4 : 2) / NACC;

  __shared__ float red[2][NACC][kWaves][kTok][kBand];
  __shared__ float ssq[kWaves][kTok];            // per wave range: sum of squares per token
  __shared__ float bk[kWaves][kTok];             // per wave range: back scale per token
  __shared__ float xsq[kWaves][kTok][kGW];       // per wave range: group sums of x per token
  __shared__ u32x4 xst[kWaves][8 * 4 * kTok];    // staged pieces, half a range
  __shared__ uint16_t luts[LUT ? kWaves : 1][kBand * kLutStride];
  __shared__ int last_flag;

  params_now(p);
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
  const int gw0 = cw0 / CPG;                   // first group of this wave's range
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
  u32x4 cq[NACC][DB][NLI][2];  // codes: two 16-byte chunks per lane per line item
  uint32_t sq[NACC][DB][4];  // scales of groups gw0..gw0+7 of the lane's row (8 halves)
  uint32_t bq[NACC][DB][2];  // biases of groups gw0+4q..gw0+4q+3 (rows q < 2), or
                             // table entries 4q..4q+3 of the row (table format)
  const bool range_ok = gw0 < p.gpr;  // wave-uniform: this wave has codes in this slice

  // Line item it of a band: chunks 8it..8it+7 of the 16 rows, in two loads of
  // 8 rows x 128 bytes (whole cache lines; 16 rows x 64 bytes per load halves
  // the achieved bandwidth). In load h, lane (q, col) takes row 8h + col % 8,
  // chunk 4 * (col / 8) + q of the line.
  auto issue_item = [&](int band, int it, int a, int d) {
    const int ch = cw0 + 8 * it + 4 * (col >> 3) + q;
    const bool ok = band < nbands && ch < C;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t n = (uint32_t)(band * kBand + 8 * h + (col & 7));
      const uint32_t off = ok ? n * (uint32_t)p.wpr * 4u + (uint32_t)ch * 16u : kOOB;
      cq[a][d][it][h] = __builtin_amdgcn_raw_buffer_load_b128(rs_[a].q, off, 0, 2);
    }
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
    for (int it = 0; it < NLI; ++it) issue_item(band, it, a, d);
    issue_rowdata(band, a, d);
  };

  int band = tile;

  // ---- stage this wave's share of X (M x 512 activations) ---------------------
  // Conversion jobs: (token t, group g, quarter r) = 16 activations, elements
  // 16r..16r+15 of group g of the range. Job 32t + 4g + r runs on lane
  // (32t + 4g + r) % 64 in round t / 2: a group's quarters sit on one quad and a
  // token's eight groups on 32 lanes, so the group sums and the token maximum
  // are DPP / row-swap reductions, and the work grows with M only.
  const int jt = lane >> 5, jg = (lane >> 2) & 7, jr = lane & 3;
  const int k0 = (gw0 + jg) * 64 + 16 * jr;  // the job's first column (same in every round)
  const bool gok = gw0 + jg < p.gpr;
  // Every round's activations and the norm weights first, as buffer loads of
  // raw bits (a masked job reads zeros; only wave-uniform branches, so the
  // conversion of each round waits for its own loads alone): one memory
  // round trip for the range.
  const uint32_t elem = p.x_f32 ? 4u : 2u;
  const uint32_t tok_bytes = (uint32_t)p.K * elem;
  const uint32_t job_bytes = 16u * elem;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)M * tok_bytes);
  u32x4 xr[kTok / 2][4];
  u32x4 gr[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
  if (norm) {
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.norm_w, (uint32_t)p.K * 2u);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      gr[h] = __builtin_amdgcn_raw_buffer_load_b128(rg, gok ? (uint32_t)k0 * 2u + 16u * h : kOOB, 0, 0);
  }
#pragma unroll
  for (int rd = 0; rd < kTok / 2; ++rd) {
    xr[rd][0] = xr[rd][1] = xr[rd][2] = xr[rd][3] = u32x4{0u, 0u, 0u, 0u};
    if (2 * rd >= M) continue;  // wave-uniform
    const int t = 2 * rd + jt;
    const bool ok = t < M && gok;
    const uint32_t base = (uint32_t)t * tok_bytes + (uint32_t)k0 * elem;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      xr[rd][h] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? base + 16u * h : kOOB, 0, 0);
    if (p.x_f32) {  // wave-uniform
#pragma unroll
      for (int h = 2; h < 4; ++h)
        xr[rd][h] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? base + 16u * h : kOOB, 0, 0);
    }
  }
  // then the first bands' codes: they stream in while the activations, which
  // return first, are converted
  asm volatile("" ::: "memory");
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int a = 0; a < NACC; ++a) issue_band(band + d * p.grid_x, a, d);
  asm volatile("" ::: "memory");
  float gv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w = i < 8 ? gr[0][(i >> 1) & 3] : gr[1][(i >> 1) & 3];
    gv[i] = f16_bits_to_f32((uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFFu)));
  }
  u32x4 pc[kTok / 2][2];  // converted pieces of each round's job
#pragma unroll
  for (int rd = 0; rd < kTok / 2; ++rd) {
    pc[rd][0] = pc[rd][1] = u32x4{0u, 0u, 0u, 0u};
    if (2 * rd >= M) continue;  // wave-uniform
    const int t = 2 * rd + jt;
    float v[16];
    if (p.x_f32) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = __uint_as_float(xr[rd][i >> 2][i & 3]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t w = xr[rd][i >> 3][(i >> 1) & 3];
        v[i] = f16_bits_to_f32((uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFFu)));
      }
    }
    if (norm) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ss = fmaf(v[i], v[i], ss);
        v[i] *= gv[i];
      }
      ss = half_sum(ss);  // over the token's 32 lanes
      if ((lane & 31) == 0 && t < M) ssq[wave][t] = ss;
    }
    float sm = 0.f, mx = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sm += v[i];
      mx = fmaxf(mx, fabsf(v[i]));
    }
    sm = quad_sum(sm);
    mx = half_max(mx);
    int E = range_exp(mx);
    if (E == kNoExp) E = 0;
    if (jr == 0 && t < M) xsq[wave][t][jg] = sm;
    if ((lane & 31) == 0 && t < M) bk[wave][t] = ldexpf(1.0f, BACK_BIAS + E);
    const float inv = ldexpf(1.0f, -E);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= inv;
    job_pieces<BITS, FMT>(v, pc[rd]);
  }
  // pieces -> LDS -> operands, one half of the range (groups 0-3, then 4-7) at a
  // time: operand P of lane (q, col) is piece (P, q) of token col
  f16x8 xa[KW * STEPS];
  u32x4* xs = xst[wave];
  const int lane_half = jg >> 2;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    wave_sync_lds();
#pragma unroll
    for (int rd = 0; rd < kTok / 2; ++rd) {
      const int t = 2 * rd + jt;
      if (2 * rd < M && t < M && lane_half == hf) {
        int P0, q0, P1, q1;
        job_slots<BITS, FMT>(jg & 3, jr, &P0, &q0, &P1, &q1);
        xs[(P0 * 4 + q0) * kTok + t] = pc[rd][0];
        xs[(P1 * 4 + q1) * kTok + t] = pc[rd][1];
      }
    }
    wave_sync_lds();
#pragma unroll
    for (int P = 0; P < 8; ++P) {
      const u32x4 u = col < M ? xs[(P * 4 + q) * kTok + col] : u32x4{0u, 0u, 0u, 0u};
      xa[hf * 8 + P] = __builtin_bit_cast(f16x8, u);
    }
  }
  wave_sync_lds();
  // bias operand: lane row q < 2 carries groups 4q..4q+3 as (hi, lo) pairs of
  // sum_x * 2^-(24+E), the units of D
  f16x8 xb = f16x8_of(0u, 0u, 0u, 0u);
  if constexpr (!LUT) {
    if (q < 2 && col < M) {
      const float binv = 1.0f / bk[wave][col];  // a power of two: exact
      uint32_t d[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float t = xsq[wave][col][4 * q + j] * binv;
        const _Float16 hi = (_Float16)t;
        const _Float16 lo = (_Float16)(t - (float)hi);
        d[j] = (uint32_t)__builtin_bit_cast(uint16_t, hi) |
               ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
      }
      xb = f16x8_of(d[0], d[1], d[2], d[3]);
    }
  }
  __syncthreads();
  // the thread that finishes output (token ot, row orow) of each band
  const int ot = threadIdx.x >> 4, orow = threadIdx.x & 15;
  const bool out_thread = threadIdx.x < kBand * M;
  // Sum of squares of the slice per token (the waves' ranges in order); when
  // the row is cut into slices, the workgroup that adds them takes the norm
  // over all of K from every slice's sum.
  float rs = 1.f;
  if (norm && out_thread) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += ssq[w][ot];
    if (p.splits > 1) {
      if (orow == 0) handoff_store(&p.mm_ssq[slice * kTok + ot], t);
    } else {
      rs = 1.0f / sqrtf(t / (float)p.K + p.eps);
    }
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
      for (int it = 0; it < NLI; ++it) {
        const u32x4 X = cq[a][d][it][0], Y = cq[a][d][it][1];
        issue_item(ahead, it, a, d);
        asm volatile("" ::: "memory");
        // back to one row per column: lane (q, col) gets chunk q (w[0..3]) and
        // chunk 4 + q (w[4..7]) of row col, then the 4 x 4 exchanges give it
        // word q of chunks 0..3 and of chunks 4..7
        const bool lo = col < 8;
        uint32_t w[8];
        const uint32_t xs4[4] = {X.x, X.y, X.z, X.w}, ys4[4] = {Y.x, Y.y, Y.z, Y.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t xr4 = row_ror8(xs4[j]), yr4 = row_ror8(ys4[j]);
          w[j] = lo ? xs4[j] : yr4;
          w[4 + j] = lo ? xr4 : ys4[j];
        }
        cross_rows_4x4(w[0], w[1], w[2], w[3]);
        cross_rows_4x4(w[4], w[5], w[6], w[7]);
        f32x4 dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int k = 8 * it + c;  // chunk within the wave range
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
            handoff_store(&p.partials[(((size_t)slice * NACC + a) * M + ot) * p.N + n], v[a]);
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
    // the partial stores are complete before the barrier, then one thread
    // takes the ticket; the last workgroup of the tile adds the slices
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) last_flag = take_ticket(&p.tickets[tile]) == (uint32_t)(p.splits - 1);
    __syncthreads();
    if (!last_flag) return;
    if (out_thread) {
      if (norm) {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.mm_ssq, (uint32_t)(p.splits * kTok * 4));
        const float t = coherent_sum(rq, (uint32_t)(ot * 4), (uint32_t)(kTok * 4), p.splits);
        rs = 1.0f / sqrtf(t / (float)p.K + p.eps);
      }
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.partials, (uint32_t)(p.splits * NACC * M * p.N * 4));
      const uint32_t sstride = (uint32_t)(NACC * M * p.N * 4);
      for (int b = tile; b < nbands; b += p.grid_x) {
        const int n = b * kBand + orow;
        if (n >= p.N) continue;
        float v[NACC];
#pragma unroll
        for (int a = 0; a < NACC; ++a)
          v[a] = coherent_sum(rp, (uint32_t)(((a * M + ot) * p.N + n) * 4), sstride, p.splits);
        finish(n, v);
      }
    }
    if (threadIdx.x == 0) handoff_store(&p.tickets[tile], 0u);
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
