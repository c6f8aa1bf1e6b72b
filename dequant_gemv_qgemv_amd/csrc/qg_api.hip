// qg_api.hip -- the extern "C" entry points declared in include/qgemv.h:
// argument validation, variant selection (lanes per row, rows per lane,
// split-K) from the shape and the device's compute-unit count, and launches.
// Nothing here allocates, frees or synchronizes.
#include <cfloat>
#include <atomic>
#include <mutex>
#include <string.h>

#include "../../include/qgemv.h"
#include "qg_internal.h"

namespace qg {
int plan_and_launch_moe(const qg_qmat* gate_all, const qg_qmat* up_all, const qg_qmat* down_all,
                        int n_experts, int F, int H, int bits, int fmt, const qg_qmat* shared3,
                        const float* router_logits, int top_k, const uint16_t* norm_w, float eps,
                        const float* x, float* y, int32_t* sel_ids, float* sel_w, void* ws,
                        size_t ws_bytes, hipStream_t stream, int M);
size_t moe_workspace_bytes(int F, int H, int top_k, int M);
}  // namespace qg

using namespace qg;

namespace {

// ---- tuning knobs (tests and benchmarks; 0 = automatic) --------------------
std::atomic<int> g_knob[8];

struct DevInfo {
  int ok;
  int cus;
};

DevInfo device_info() {
  static std::mutex mu;
  static DevInfo cache[64];
  static bool have[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return {0, 0};
  std::lock_guard<std::mutex> lk(mu);
  if (!have[dev]) {
    hipDeviceProp_t prop;
    DevInfo d{0, 0};
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      d.ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      d.cus = prop.multiProcessorCount;
    }
    cache[dev] = d;
    have[dev] = true;
  }
  return cache[dev];
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The scale and bias arrays of W start 16-byte aligned (staged scale/bias
// rows load them 16 bytes at a time). NULL matrices do not count.
bool sb_aligned16(const qg_qmat* W) {
  return !W || (aligned(W->scales, 16) && aligned(W->biases, 16));
}

// [a, a+na) and [b, b+nb) overlap (byte ranges)
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_common(int N, int K, int M, int group, int bits, int fmt, int x_dtype) {
  if (N < 0 || K <= 0 || M < 1) return QG_EINVAL;
  if (x_dtype != QG_F16 && x_dtype != QG_F32) return QG_EINVAL;
  if (fmt != QG_AFFINE && fmt != QG_LUT && fmt != QG_DENSE) return QG_EINVAL;
  if (group != 64) return QG_EUNSUPPORTED;
  if (fmt == QG_AFFINE && bits != 4 && bits != 2 && bits != 8) return QG_EUNSUPPORTED;
  if (fmt == QG_LUT && bits != 4) return QG_EUNSUPPORTED;
  if (fmt == QG_DENSE && bits != 16) return QG_EUNSUPPORTED;
  if (K % 64) return QG_EINVAL;
  if (K > QG_MAX_K) return QG_EUNSUPPORTED;
  if (M > QG_MAX_M) return QG_EUNSUPPORTED;
  if ((size_t)N * (size_t)K * (size_t)bits / 8 >= ((size_t)1 << 31)) return QG_EUNSUPPORTED;
  return QG_OK;
}

int check_qmat(const qg_qmat* W, int fmt) {
  if (!W || !W->q || !aligned(W->q, 16)) return QG_EINVAL;
  if (fmt == QG_AFFINE) {
    if (!W->scales || !W->biases || !aligned(W->scales, 2) || !aligned(W->biases, 2))
      return QG_EINVAL;
  } else if (fmt == QG_LUT) {
    if (!W->lut || !aligned(W->lut, 2)) return QG_EINVAL;
  }
  return QG_OK;
}

QMat to_dev(const qg_qmat* W) {
  QMat m{nullptr, nullptr, nullptr, nullptr};
  if (W) {
    m.q = W->q;
    m.s = W->scales;
    m.b = W->biases;
    m.lut = W->lut;
  }
  return m;
}

constexpr int kMaxSplits = 16;
constexpr size_t kLdsBudget = 64 * 1024;

int codes_per_chunk(int bits) { return 128 / bits; }
// 16-byte pieces of staged x per chunk: fp16 pairs for the affine and dense
// formats, fp32 for the LUT format.
int pieces_per_chunk(int bits, int fmt) {
  if (fmt == QG_LUT) return 4;
  return bits == 16 ? 1 : bits == 8 ? 2 : bits == 4 ? 4 : 8;
}

// Lanes per row: the widest of 64/32/16 that leaves no lane idle in any pass,
// else the one that idles the fewest; with two exceptions measured on MI355X.
// Rows of 17..32 chunks: two passes of 16 lanes (one row reduction per two
// items instead of one per item: 151936 x 1024 logits 18.1 us against 20.4,
// 3072 x 1024 gate.up 4.57 against 4.74). Rows of 96..127 chunks: 64 lanes
// with a partly empty last pass, which keeps twice the bands of 32 lanes for
// short matrices (1024 x 3072: 3.64 us against 4.27). Rows of 33..64 chunks:
// two passes of 32 lanes up to 8192 rows (4096 x 4096 2-bit 4.46 us against
// 4.52 with one pass of 64; 4096 x 1792 4-bit 4.35 against 4.96), and beyond
// that 16 lanes unless they idle more lanes (more rows per band, fewer
// bands: 14336 x 4096 2-bit gate.up 11.60 against 11.97 with 32 lanes,
// 14336 x 2048 4-bit 6.22 against 6.39).
int pick_lpr(int C, int N) {
  if (C > 16 && C <= 32) return 16;
  if (C > 32 && C <= 64) {
    const double e32 = (double)C / (double)(((C + 31) / 32) * 32);
    const double e16 = (double)C / (double)(((C + 15) / 16) * 16);
    return (N > 8192 && e16 >= e32) ? 16 : 32;
  }
  if (C >= 96 && C < 128) return 64;
  const int cands[3] = {64, 32, 16};
  int best = 64;
  double best_eff = -1.0;
  for (int l : cands) {
    const int passes = (C + l - 1) / l;
    const double eff = (double)C / (double)(passes * l);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = l;
    }
  }
  return best;
}

struct MvShape {
  int N, K, bits, fmt, epi;
  int col_seg_chunks;  // K-segment length in chunks (0: one matrix along K)
  int seg;             // SegMode of the launch
  bool sb_aligned;     // every scale/bias array starts 16-byte aligned
};

// Chooses lanes per row, rows per lane, split-K and grid for one launch.
MvPlan plan_mv(const MvShape& s, int cus, bool have_ws) {
  MvPlan pl{};
  const int C = s.K / codes_per_chunk(s.bits);
  pl.lpr = g_knob[2].load() ? g_knob[2].load() : pick_lpr(C, s.N);
  if (s.col_seg_chunks > 0 && !g_knob[2].load()) {
    // keep every pass inside one K segment when the segments allow it
    for (int l : {64, 32, 16})
      if (s.col_seg_chunks % l == 0) {
        pl.lpr = l;
        break;
      }
  }
  // Two rows per lane for long 4-bit affine rows: half the workgroups, so
  // half the copies of a 56 KB x staged from L2 (measured on the 4096 x 14336
  // down projection: 11.5 -> 10.9 us). Measured slower for 2-bit codes (whose
  // kernels already hold one workgroup per CU: 9.2 -> 11.6 us) and for the
  // table format (per-band tables).
  pl.rows = g_knob[1].load()
                ? g_knob[1].load()
                : (s.bits == 4 && s.fmt == QG_AFFINE && s.seg == kSegNone && s.K >= 8192 ? 2 : 1);
  if (s.epi == kEpiTopk) pl.rows = 1;  // the fused top-k keeps one row per lane slot
  pl.depth = g_knob[4].load() ? g_knob[4].load() : 2;
  const int nacc = s.epi == kEpiSwiglu ? 2 : 1;
  if (s.fmt == QG_LUT) {
    // the table format keeps a 1 KB pair table per row in flight: wider rows
    // (fewer rows per band) where the tables would take more than three
    // quarters of the LDS budget (the rest stages x)
    while (pl.lpr < 64 &&
           (size_t)kWaves * (64 / pl.lpr) * pl.rows * nacc * kLutRowWords * 4 > kLdsBudget * 3 / 4)
      pl.lpr *= 2;
  }
  const int rpb = (64 / pl.lpr) * pl.rows;
  const int nbands = (s.N + rpb - 1) / rpb;
  const int tiles = (nbands + kWaves - 1) / kWaves;
  const size_t per_chunk = (size_t)pieces_per_chunk(s.bits, s.fmt) * 16 + 16;  // + ChunkInfo
  const size_t lut_bytes = (s.fmt == QG_LUT) ? (size_t)kWaves * rpb * nacc * kLutRowWords * 4 : 0;
  int max_chunks = (int)((kLdsBudget - lut_bytes) / per_chunk);
  max_chunks = (max_chunks / pl.lpr) * pl.lpr;
  const int passes = (C + pl.lpr - 1) / pl.lpr;
  int splits = (C + max_chunks - 1) / max_chunks;
  // K is split only when one slice would not fit in LDS: measured on MI355X,
  // splitting a launch to put more workgroups in flight made every shape slower
  // (a tail of the waves runs three times longer), so small-N launches keep
  // their tiles.
  if (g_knob[0].load()) splits = g_knob[0].load();
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits > passes) splits = passes;
  if (splits < 1) splits = 1;
  if (!have_ws) splits = 1;
  int slice_passes = (passes + splits - 1) / splits;
  pl.slice_chunks = slice_passes * pl.lpr;
  pl.splits = (C + pl.slice_chunks - 1) / pl.slice_chunks;
  const int slice_npass = slice_passes;
  pl.lds_bytes = (size_t)slice_npass * pl.lpr * per_chunk + lut_bytes;
  // Staged scale/bias rows (affine formats, one K segment), on request (knob
  // 6 = 1): each band's row segments over the slice come with one or two
  // 16-byte loads per lane into the wave's LDS area, and every pass reads its
  // two values per row there. Needs 16-byte aligned row segments (K and the
  // slice a multiple of 512 codes' groups) and the room in LDS. Not the
  // default: measured on MI355X it halves the load instructions per wave but
  // makes the Llama-3-8B-shaped layer slower (41.7 against 38.4 us; qkv 7.06
  // against 6.12, o 6.33 against 5.55), the MoE layer unchanged (20.2 us).
  pl.sbl = 0;
  pl.sb_segp = 0;
  if (s.fmt == QG_AFFINE && s.seg != kSegCols && s.sb_aligned && g_knob[6].load() == 1 &&
      !(pl.rows == 2 && s.epi == kEpiSwiglu)) {
    const int cpg = 64 / codes_per_chunk(s.bits);
    const int gpr = s.K / 64;
    const int gsl = (pl.slice_chunks < C ? pl.slice_chunks : C) / cpg;  // groups per slice
    const int want = pl.rows == 2 ? 2 : 1;  // loads per lane and band the kernels provide
    if ((gpr * 2) % 16 == 0 && (gsl * 2) % 16 == 0 && pl.slice_chunks % cpg == 0) {
      const int segp = gsl * 2 / 16;
      const int pieces = rpb * nacc * 2 * segp;
      const size_t sb_bytes = (size_t)kWaves * pieces * 16;
      if (pieces <= 64 * want && pl.lds_bytes + sb_bytes <= kLdsBudget) {
        pl.sbl = want;
        pl.sb_segp = segp;
        pl.lds_bytes += sb_bytes;
      }
    }
  }
  // Resident workgroups per CU: two 8-wave groups keep 16 waves in flight
  // where the kernel's registers allow it. 2-bit codes take one: measured on
  // MI355X, a second group slows them down (4096 x 14336 down 10.22 us
  // against 8.96 at 64 lanes, 14336 x 4096 gate.up 12.14 against 11.40 at
  // 32), while the 4-bit kernels gain from it (gate.up 14.22 against 14.88).
  const int resident = mv_resident_per_cu(s.bits, s.fmt, s.epi, s.seg, pl);
  const int wg_cap = s.bits == 2 ? 1 : 2;
  const int wg_per_cu = g_knob[3].load() ? g_knob[3].load() : (resident < wg_cap ? resident : wg_cap);
  int gx = tiles;
  const int cap = (cus * wg_per_cu + pl.splits - 1) / pl.splits;
  if (gx > cap) gx = cap;
  gx = ((gx + 7) / 8) * 8;  // slices of one tile share an XCD (workgroups go round-robin over 8)
  pl.grid_x = gx;
  return pl;
}

// Tickets, then the fp32 partials of every slice; several vectors (the
// matrix-core kernels) add each slice's per-vector sums of squares.
constexpr size_t kMmSsqBytes = (size_t)kMaxSplits * 8 * 4;
size_t mv_ws_bytes(int N, int M, int epi) {
  const size_t tickets = ((size_t)(N + 7) / 8 + 64) * 4;
  const size_t tickets_al = (tickets + 255) / 256 * 256;
  return tickets_al + (size_t)kMaxSplits * (epi == kEpiSwiglu ? 2 : 1) * M * N * 4 +
         (M > 1 ? kMmSsqBytes : 0);
}

// Work to enqueue right before a call's first kernel, once every check has
// passed (so that a refused call still enqueues nothing).
struct PreLaunch {
  int (*fn)(void* arg, hipStream_t stream);
  void* arg;
};

int run_pre(const PreLaunch* pre, hipStream_t stream) { return pre ? pre->fn(pre->arg, stream) : QG_OK; }

// Extra requirements of the M = 2..8 kernels: each wave loads whole
// 512-code ranges of a row's scales/biases (or its table) with 16-byte loads.
int check_mm(const qg_qmat* A, const qg_qmat* B, int K, int fmt) {
  if (K % 512) return QG_EUNSUPPORTED;
  const qg_qmat* mats[2] = {A, B};
  for (const qg_qmat* W : mats) {
    if (!W) continue;
    if (fmt == QG_AFFINE && (!aligned(W->scales, 16) || !aligned(W->biases, 16)))
      return QG_EUNSUPPORTED;
    if (fmt == QG_LUT && !aligned(W->lut, 16)) return QG_EUNSUPPORTED;
  }
  return QG_OK;
}

// M = 2..8: matrix-core kernels. K is cut into slices of mm_slice_codes()
// codes (one workgroup each per band set); more than one slice needs the
// workspace for the fp32 partials (and, with a norm, each slice's sums of
// squares).
int run_mm(const qg_qmat* A, const qg_qmat* B, int N, int K, int M, int bits, int fmt, int epi,
           const void* x, int x_dtype, const uint16_t* norm_w, float eps, const float* residual,
           float* y, void* ws, bool have_ws, int cus, hipStream_t stream, const PreLaunch* pre) {
  const int slice = mm_slice_codes();
  const int splits = (K + slice - 1) / slice;
  if (splits > 1 && !have_ws) return QG_EWORKSPACE;
  if (int rc = run_pre(pre, stream)) return rc;
  const int nbands = (N + 15) / 16;
  // one 8-wave workgroup per compute unit: the waves hold their activations
  // and two to four bands of codes in registers
  const int wg_per_cu = g_knob[3].load() ? g_knob[3].load() : 1;
  int gx = nbands;
  const int cap = (cus * wg_per_cu + splits - 1) / splits;
  if (gx > cap) gx = cap;
  gx = ((gx + 7) / 8) * 8;  // slices of one tile share an XCD
  MvPlan pl{};
  pl.splits = splits;
  pl.grid_x = gx;
  MvParams p;
  memset(&p, 0, sizeof(p));
  p.A[0] = to_dev(A);
  p.B[0] = to_dev(B);
  p.nseg = 1;
  p.seg_mode = kSegNone;
  p.N = N;
  p.K = K;
  p.M = M;
  p.wpr = K * bits / 32;
  p.gpr = K / 64;
  p.x = x;
  p.x_f32 = x_dtype == QG_F32;
  p.norm_w = norm_w;
  p.eps = eps;
  p.residual = residual;
  p.y = y;
  p.splits = splits;
  p.slice_chunks = slice / (128 / bits);
  p.grid_x = gx;
  if (splits > 1) {
    const size_t tickets = ((size_t)(N + 7) / 8 + 64) * 4;
    const size_t tickets_al = (tickets + 255) / 256 * 256;
    const size_t partial_bytes = (size_t)kMaxSplits * (epi == kEpiSwiglu ? 2 : 1) * M * N * 4;
    p.tickets = static_cast<uint32_t*>(ws);
    p.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + tickets_al);
    p.mm_ssq = reinterpret_cast<float*>(static_cast<char*>(ws) + tickets_al + partial_bytes);
  }
  const hipError_t e = launch_mm(bits, fmt, epi, pl, p, stream);
  return e == hipSuccess ? QG_OK : QG_ELAUNCH;
}

// Outputs and workspace regions of a matvec launch that also takes the top-k
// of its rows (kEpiTopk).
struct TopkOut {
  int k;
  int32_t* idx;
  float* vals;
  DrawParams dp;      // dp.token set: draw one token from the top-k too
  uint32_t* tickets;  // [kTkMaxGroups + 1], zero at rest
  uint64_t* cand;     // [grid_x + groups][kTkList]
};
// run_mv with kEpiTopk: the plan does not allow the one-launch top-k (nothing
// was enqueued; the caller takes the two-launch path).
constexpr int kNotFused = 1;

// The one-launch top-k takes a plan where each wave's rows fit its key list,
// the groups of workgroups fit the last merge, and K is one slice.
bool topk_fits(const MvPlan& pl, int N, int k) {
  const int rpb = 64 / pl.lpr;
  const int nbands = (N + rpb - 1) / rpb;
  const int waves = pl.grid_x * kWaves;
  const int per_wave = (nbands + waves - 1) / waves;
  return k <= kTkList && pl.splits == 1 && pl.rows == 1 && pl.grid_x <= kTkMaxGroups * kTkGroup &&
         per_wave * rpb <= kTkList;
}

int run_mv(const qg_qmat* A, const qg_qmat* B, int N, int K, int M, int group, int bits, int fmt,
           int epi, const void* x, int x_dtype, const uint16_t* norm_w, float eps,
           const float* residual, float* y, void* ws, size_t ws_bytes, hipStream_t stream,
           const PreLaunch* pre = nullptr, const TopkOut* tko = nullptr) {
  int rc = check_common(N, K, M, group, bits, fmt, x_dtype);
  if (rc) return rc;
  if ((rc = check_qmat(A, fmt))) return rc;
  if (epi == kEpiSwiglu && (rc = check_qmat(B, fmt))) return rc;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 4)) return QG_EINVAL;
  if (norm_w && !aligned(norm_w, 16)) return QG_EINVAL;
  if (residual && !aligned(residual, 4)) return QG_EINVAL;
  const size_t xbytes = (size_t)M * K * (x_dtype == QG_F32 ? 4 : 2);
  const size_t ybytes = (size_t)M * N * 4;
  if (overlaps(x, xbytes, y, ybytes)) return QG_EINVAL;
  if (residual && residual != y && overlaps(residual, ybytes, y, ybytes)) return QG_EINVAL;
  // Several vectors: 2- and 4-bit codes on the matrix cores; 8-bit and dense
  // weights through the streaming kernel, one workgroup row per vector.
  const bool on_mfma = M > 1 && bits != 8 && fmt != QG_DENSE;
  if (on_mfma && (rc = check_mm(A, epi == kEpiSwiglu ? B : nullptr, K, fmt))) return rc;
  if (N == 0) return QG_OK;
  const DevInfo dev = device_info();
  if (!dev.ok) return QG_EDEVICE;
  const bool have_ws = ws && ws_bytes >= mv_ws_bytes(N, M, epi) && aligned(ws, 256);
  if (on_mfma)
    return run_mm(A, B, N, K, M, bits, fmt, epi, x, x_dtype, norm_w, eps, residual, y, ws,
                  have_ws, dev.cus, stream, pre);
  // Several vectors keep each vector's K in one slice (per-vector split-K
  // partials are not provided): planned as if a workspace were there, so a
  // K that needs slices is refused whatever workspace came with the call.
  const bool sb_al = sb_aligned16(A) && (epi != kEpiSwiglu || sb_aligned16(B));
  MvPlan pl = plan_mv({N, K, bits, fmt, epi, 0, kSegNone, sb_al}, dev.cus, M > 1 || have_ws);
  if (M > 1 && pl.splits > 1) return QG_EUNSUPPORTED;
  if (pl.lds_bytes > kLdsBudget) return QG_EWORKSPACE;  // K too long for one slice: needs ws
  if (epi == kEpiTopk && (!tko || M != 1 || residual || !topk_fits(pl, N, tko->k))) return kNotFused;
  pl.tokens = M;
  MvParams p;
  memset(&p, 0, sizeof(p));
  p.A[0] = to_dev(A);
  p.B[0] = to_dev(B);
  p.nseg = 1;
  p.seg_mode = kSegNone;
  p.seg_len = 0;
  p.N = N;
  p.K = K;
  p.wpr = K * bits / 32;
  p.gpr = K / 64;
  p.M = 1;
  p.x = x;
  p.x_f32 = x_dtype == QG_F32;
  p.norm_w = norm_w;
  p.eps = eps;
  p.residual = residual;
  p.y = y;
  p.splits = pl.splits;
  p.slice_chunks = pl.slice_chunks;
  p.grid_x = pl.grid_x;
  p.tokens = M;
  p.sb_segp = pl.sb_segp;
  if (epi == kEpiTopk) {
    p.tk_k = tko->k;
    p.tk_idx = tko->idx;
    p.tk_vals = tko->vals;
    p.tk_tickets = tko->tickets;
    p.tk_cand = tko->cand;
    p.tk_draw = tko->dp;
  }
  if (pl.splits > 1) {
    const size_t tickets = ((size_t)(N + 7) / 8 + 64) * 4;
    const size_t tickets_al = (tickets + 255) / 256 * 256;
    p.tickets = static_cast<uint32_t*>(ws);
    p.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + tickets_al);
  }
  if ((rc = run_pre(pre, stream))) return rc;
  const hipError_t e = launch_mv(bits, fmt, epi, pl, p, stream);
  return e == hipSuccess ? QG_OK : QG_ELAUNCH;
}

}  // namespace

namespace qg {
// Shared with the MoE launcher: plans one launch (variant, split-K, grid,
// workspace regions) into *p and *plan without enqueueing anything, so a
// caller with several launches can validate all of them first.
int mv_plan_internal(int bits, int fmt, int epi, MvParams* p, bool have_ws, void* ws,
                     size_t ws_bytes, size_t ws_offset, int tokens, MvPlan* plan) {
  const DevInfo dev = device_info();
  if (!dev.ok) return QG_EDEVICE;
  bool sb_al = true;
  auto al16 = [](const void* q) { return ((uintptr_t)q % 16) == 0; };
  for (int i = 0; i < p->nseg && i < kMaxSeg; ++i)
    sb_al = sb_al && al16(p->A[i].s) && al16(p->A[i].b) && al16(p->B[i].s) && al16(p->B[i].b);
  sb_al = sb_al && al16(p->route.all_A.s) && al16(p->route.all_A.b) && al16(p->route.all_B.s) &&
          al16(p->route.all_B.b);
  const MvPlan pl = plan_mv({p->N, p->K, bits, fmt, epi, p->seg_mode == kSegCols ? p->seg_len : 0,
                             p->seg_mode, sb_al}, dev.cus, have_ws);
  if (pl.lds_bytes > kLdsBudget) return QG_EWORKSPACE;
  // a batched launch keeps each token's K in one slice (its split-K partials
  // and tickets would need one workspace region per token)
  if (tokens > 1 && pl.splits > 1) return QG_EUNSUPPORTED;
  p->splits = pl.splits;
  p->slice_chunks = pl.slice_chunks;
  p->grid_x = pl.grid_x;
  p->sb_segp = pl.sb_segp;
  *plan = pl;
  plan->tokens = tokens;
  p->tokens = tokens;
  if (pl.splits > 1) {
    const size_t tickets = ((size_t)(p->N + 7) / 8 + 64) * 4;
    const size_t tickets_al = (tickets + 255) / 256 * 256;
    if (ws_offset + mv_ws_bytes(p->N, 1, epi) > ws_bytes) return QG_EWORKSPACE;
    char* base = static_cast<char*>(ws) + ws_offset;
    p->tickets = reinterpret_cast<uint32_t*>(base);
    p->partials = reinterpret_cast<float*>(base + tickets_al);
  }
  return QG_OK;
}
int mv_launch_planned(int bits, int fmt, int epi, const MvPlan& plan, const MvParams& p,
                      hipStream_t stream) {
  return launch_mv(bits, fmt, epi, plan, p, stream) == hipSuccess ? QG_OK : QG_ELAUNCH;
}
size_t mv_workspace_bytes(int N, int epi) { return mv_ws_bytes(N, 1, epi); }
int device_ok() { return device_info().ok; }
}  // namespace qg

namespace {
// Argument checks shared by the logits entry points (those that run_mv does
// not make itself).
int check_logits(int V, int K, int group, int bits, int fmt, int x_dtype, const uint16_t* norm_w,
                 float eps, const float* logits, int k, const int32_t* idx, const float* vals) {
  int rc = check_common(V, K, 1, group, bits, fmt, x_dtype);
  if (rc) return rc;
  if (V < 1) return QG_EINVAL;
  if (k < 1 || k > V) return QG_EINVAL;
  if (k > QG_MAX_TOPK) return QG_EUNSUPPORTED;
  if (!logits || !idx || !vals || !aligned(logits, 4) || !aligned(idx, 4) || !aligned(vals, 4))
    return QG_EINVAL;
  if (norm_w && !(eps >= 0.f)) return QG_EINVAL;
  return QG_OK;
}

// The logits matvec and its top-k ([F] section 1: both on the GPU, only the
// chosen entries, or the drawn token, come back). Where the plan allows it,
// one launch: the matvec's workgroups merge their rows' keys themselves and
// the last merger draws the token (kEpiTopk). Otherwise the matvec, then the
// top-k kernel (which also draws).
// ws starts with the top-k region (topk_workspace_bytes), the matvec's follows.
int run_logits(const qg_qmat* W, int V, int K, int group, int bits, int fmt, const void* x,
               int x_dtype, const uint16_t* norm_w, float eps, float* logits, int k, int32_t* idx,
               float* vals, void* ws, size_t ws_bytes, const DrawParams& dp, hipStream_t stream,
               const PreLaunch* pre) {
  const size_t tk = topk_workspace_bytes(V, k);
  char* const base = static_cast<char*>(ws);
  if (!g_knob[5].load()) {
    const TopkOut tko{k, idx, vals, dp, reinterpret_cast<uint32_t*>(base + kTkFusedTicketOffset),
                      reinterpret_cast<uint64_t*>(base + kTkTicketBytes)};
    const int rc = run_mv(W, nullptr, V, K, 1, group, bits, fmt, kEpiTopk, x, x_dtype, norm_w, eps,
                          nullptr, logits, base + tk, ws_bytes - tk, stream, pre, &tko);
    if (rc != kNotFused) return rc;
  }
  int rc = run_mv(W, nullptr, V, K, 1, group, bits, fmt, kEpiStore, x, x_dtype, norm_w, eps,
                  nullptr, logits, base + tk, ws_bytes - tk, stream, pre);
  if (rc) return rc;
  return plan_and_launch_topk(logits, V, k, idx, vals, ws, tk, dp, stream);  // 0, -3 or -4 = QG_ codes
}

// ---- library-held scratch for qlogits_topk_noalloc -------------------------
// One array per GPU, held until the process ends; its device address comes
// from hipGetSymbolAddress once per device (the array's name in host code is
// not a device address). Every call on a GPU shares it, so calls that overlap
// on one GPU race.
constexpr size_t kStaticScratchBytes = (size_t)24 << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
struct StaticScratch {
  void* ptr;     // device address of this device's copy of `scratch`
  bool cleared;  // its integer tickets are known to be zero
};
std::mutex g_static_mu;
StaticScratch g_static[kMaxDevices];

// This device's scratch address (taken once, with the device current).
int static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QG_EDEVICE;
  std::lock_guard<std::mutex> lk(g_static_mu);
  StaticScratch& s = g_static[dev];
  if (!s.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QG_ELAUNCH;
    s.ptr = p;
  }
  *out = s.ptr;
  return QG_OK;
}

// Pre-launch step of the first call on a device: clears the whole array with
// the fill kernel on the call's stream (ahead of the call's kernels; no
// memset node, so it may be captured). A clear recorded into a graph under
// capture does not count: the next uncaptured call clears again. Every call
// leaves the tickets at zero, so later calls need no clear.
int clear_static_once(void* arg, hipStream_t stream) {
  (void)arg;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QG_EDEVICE;
  std::lock_guard<std::mutex> lk(g_static_mu);
  StaticScratch& s = g_static[dev];
  if (s.cleared) return QG_OK;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) return QG_ELAUNCH;
  if (launch_fill_u32(static_cast<uint32_t*>(s.ptr), kStaticScratchBytes / 4, 0u, stream) != hipSuccess)
    return QG_ELAUNCH;
  if (st == hipStreamCaptureStatusNone) s.cleared = true;
  return QG_OK;
}

// Validates the draw arguments and fills dp. QG_OK or QG_EINVAL.
int make_draw(float temperature, float top_p, uint64_t seed, uint64_t* counter, int32_t* token,
              DrawParams* dp) {
  if (!(temperature >= 0.f) || !(temperature <= FLT_MAX)) return QG_EINVAL;
  if (!(top_p > 0.f) || !(top_p <= 1.f)) return QG_EINVAL;
  if (!token || !aligned(token, 4) || (counter && !aligned(counter, 8))) return QG_EINVAL;
  dp->temperature = temperature;
  dp->top_p = top_p;
  dp->seed = seed;
  dp->counter = counter;
  dp->token = token;
  return QG_OK;
}
}  // namespace

extern "C" {

const char* qg_status_str(int status) {
  switch (status) {
    case QG_OK: return "QG_OK";
    case QG_EINVAL: return "QG_EINVAL: invalid argument (NULL pointer, size, alignment or aliasing)";
    case QG_EUNSUPPORTED: return "QG_EUNSUPPORTED: valid but not provided (group, bits, format, M, K or k)";
    case QG_EWORKSPACE: return "QG_EWORKSPACE: workspace missing or too small";
    case QG_ELAUNCH: return "QG_ELAUNCH: the HIP runtime reported an error while enqueueing";
    case QG_EDEVICE: return "QG_EDEVICE: the current HIP device is not a usable gfx950";
    default: return "unknown qgemv status";
  }
}

int qg_workspace_bytes(int op, int N, int K, int M, int bits, int fmt, int k, size_t* bytes) {
  if (!bytes) return QG_EINVAL;
  if (N < 0 || K < 0 || M < 1) return QG_EINVAL;
  (void)bits;
  (void)fmt;
  switch (op) {
    case QG_OP_GEMV:
    case QG_OP_GEMV_RMSNORM: *bytes = mv_ws_bytes(N, M, kEpiStore); return QG_OK;
    case QG_OP_SWIGLU: *bytes = mv_ws_bytes(N, M, kEpiSwiglu); return QG_OK;
    case QG_OP_MOE:
      if (k < 1 || k > kMaxRoutes) return QG_EUNSUPPORTED;
      if (M < 1 || M > QG_MAX_M) return QG_EUNSUPPORTED;
      *bytes = moe_workspace_bytes(K, N, k, M);
      return QG_OK;
    case QG_OP_LOGITS_TOPK:
      if (k < 1 || k > QG_MAX_TOPK) return QG_EUNSUPPORTED;
      *bytes = topk_workspace_bytes(N, k) + mv_ws_bytes(N, 1, kEpiStore);
      return QG_OK;
    case QG_OP_ATTN:
      if (N < 1 || N % M) return QG_EINVAL;
      if ((k != 64 && k != 128) || (N / M != 1 && N / M != 2 && N / M != 4 && N / M != 8))
        return QG_EUNSUPPORTED;
      *bytes = attn_ws_bytes(N, M, k);
      return QG_OK;
    default: return QG_EINVAL;
  }
}

int qg_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || ws_bytes % 4 || !aligned(ws, 4)) return QG_EINVAL;
  const hipError_t e = launch_fill_u32(static_cast<uint32_t*>(ws), ws_bytes / 4, 0u, stream);
  return e == hipSuccess ? QG_OK : QG_ELAUNCH;
}

// Tuning override for tests and benchmarks: knob 0 = split count, 1 = rows per
// lane, 2 = lanes per row, 3 = workgroups per CU, 4 = pipeline depth, 5 = 1
// for the two-launch logits top-k, 6 = 1 for staged scale/bias rows instead
// of per-pass loads; value 0 restores automatic.
int qg_tune(int knob, int value) {
  if (knob < 0 || knob > 6 || value < 0) return QG_EINVAL;
  if ((knob == 5 || knob == 6) && value > 1) return QG_EINVAL;
  if (knob == 4 && value != 0 && value != 2 && value != 4) return QG_EINVAL;
  if (knob == 1 && value != 0 && value != 1 && value != 2) return QG_EINVAL;
  if (knob == 2 && value != 0 && value != 16 && value != 32 && value != 64) return QG_EINVAL;
  if (knob == 0 && value > kMaxSplits) return QG_EINVAL;
  g_knob[knob].store(value);
  return QG_OK;
}

int qgemv(const qg_qmat* W, int N, int K, int M, int group, int bits, int fmt, const void* x,
          int x_dtype, const float* residual, float* y, void* ws, size_t ws_bytes,
          hipStream_t stream) {
  return run_mv(W, nullptr, N, K, M, group, bits, fmt, kEpiStore, x, x_dtype, nullptr, 0.f,
                residual, y, ws, ws_bytes, stream);
}

int qgemv_rmsnorm(const qg_qmat* W, int N, int K, int M, int group, int bits, int fmt,
                  const void* x, int x_dtype, const uint16_t* norm_w, float eps,
                  const float* residual, float* y, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  if (!norm_w || !(eps >= 0.f)) return QG_EINVAL;
  return run_mv(W, nullptr, N, K, M, group, bits, fmt, kEpiStore, x, x_dtype, norm_w, eps,
                residual, y, ws, ws_bytes, stream);
}

int qswiglu(const qg_qmat* Wgate, const qg_qmat* Wup, int F, int K, int M, int group, int bits,
            int fmt, const void* x, int x_dtype, const uint16_t* norm_w, float eps, float* u,
            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (norm_w && !(eps >= 0.f)) return QG_EINVAL;
  return run_mv(Wgate, Wup, F, K, M, group, bits, fmt, kEpiSwiglu, x, x_dtype, norm_w, eps,
                nullptr, u, ws, ws_bytes, stream);
}

int qmoe_experts(const qg_qmat* gate_all, const qg_qmat* up_all, const qg_qmat* down_all,
                 int n_experts, int F, int H, int group, int bits, int fmt,
                 const qg_qmat* shared3, const float* router_logits, int top_k,
                 const uint16_t* norm_w, float eps, const float* x, float* y, int32_t* sel_ids,
                 float* sel_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  return qmoe_experts_batch(gate_all, up_all, down_all, n_experts, F, H, 1, group, bits, fmt,
                            shared3, router_logits, top_k, norm_w, eps, x, y, sel_ids, sel_w, ws,
                            ws_bytes, stream);
}

int qmoe_experts_batch(const qg_qmat* gate_all, const qg_qmat* up_all, const qg_qmat* down_all,
                       int n_experts, int F, int H, int M, int group, int bits, int fmt,
                       const qg_qmat* shared3, const float* router_logits, int top_k,
                       const uint16_t* norm_w, float eps, const float* x, float* y,
                       int32_t* sel_ids, float* sel_w, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  if (M < 1) return QG_EINVAL;
  if (M > QG_MAX_M) return QG_EUNSUPPORTED;
  int rc = check_common(F, H, 1, group, bits, fmt, QG_F32);
  if (rc) return rc;
  if ((rc = check_common(H, F, 1, group, bits, fmt, QG_F32))) return rc;
  if (n_experts < 1 || F < 1 || H < 1) return QG_EINVAL;
  if (top_k < 1 || top_k > kMaxRoutes || top_k > n_experts) return QG_EUNSUPPORTED;
  if (fmt != QG_AFFINE) return QG_EUNSUPPORTED;  // expert layers take the affine format
  return plan_and_launch_moe(gate_all, up_all, down_all, n_experts, F, H, bits, fmt, shared3,
                             router_logits, top_k, norm_w, eps, x, y, sel_ids, sel_w, ws,
                             ws_bytes, stream, M);
}

int qlogits_topk(const qg_qmat* W, int V, int K, int group, int bits, int fmt, const void* x,
                 int x_dtype, const uint16_t* norm_w, float eps, float* logits, int k,
                 int32_t* idx, float* vals, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_logits(V, K, group, bits, fmt, x_dtype, norm_w, eps, logits, k, idx, vals);
  if (rc) return rc;
  const size_t need = topk_workspace_bytes(V, k) + mv_ws_bytes(V, 1, kEpiStore);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return QG_EWORKSPACE;
  return run_logits(W, V, K, group, bits, fmt, x, x_dtype, norm_w, eps, logits, k, idx, vals, ws,
                    ws_bytes, DrawParams{}, stream, nullptr);
}

int qlogits_topk_noalloc(const qg_qmat* W, int V, int K, int group, int bits, int fmt,
                         const void* x, int x_dtype, const uint16_t* norm_w, float eps,
                         float* logits, int k, int32_t* idx, float* vals, hipStream_t stream) {
  int rc = check_logits(V, K, group, bits, fmt, x_dtype, norm_w, eps, logits, k, idx, vals);
  if (rc) return rc;
  const size_t need = topk_workspace_bytes(V, k) + mv_ws_bytes(V, 1, kEpiStore);
  if (need > kStaticScratchBytes) return QG_EUNSUPPORTED;
  if (!device_info().ok) return QG_EDEVICE;
  void* ws = nullptr;
  if ((rc = static_scratch(&ws))) return rc;
  const PreLaunch pre{clear_static_once, nullptr};
  return run_logits(W, V, K, group, bits, fmt, x, x_dtype, norm_w, eps, logits, k, idx, vals, ws,
                    need, DrawParams{}, stream, &pre);
}

int qg_logits_topk_launches(const qg_qmat* W, int V, int K, int group, int bits, int fmt, int k,
                            int* launches) {
  if (!launches) return QG_EINVAL;
  int rc = check_common(V, K, 1, group, bits, fmt, QG_F32);
  if (rc) return rc;
  if (V < 1 || k < 1 || k > V) return QG_EINVAL;
  if (k > QG_MAX_TOPK) return QG_EUNSUPPORTED;
  const DevInfo dev = device_info();
  if (!dev.ok) return QG_EDEVICE;
  const MvPlan pl = plan_mv({V, K, bits, fmt, kEpiTopk, 0, kSegNone, sb_aligned16(W)}, dev.cus, true);
  *launches = (!g_knob[5].load() && topk_fits(pl, V, k)) ? 1 : 2;
  return QG_OK;
}

int qlogits_sample(const qg_qmat* W, int V, int K, int group, int bits, int fmt, const void* x,
                   int x_dtype, const uint16_t* norm_w, float eps, float* logits, int k,
                   int32_t* idx, float* vals, float temperature, float top_p, uint64_t seed,
                   uint64_t* counter, int32_t* token, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  DrawParams dp;
  int rc = make_draw(temperature, top_p, seed, counter, token, &dp);
  if (rc) return rc;
  rc = check_logits(V, K, group, bits, fmt, x_dtype, norm_w, eps, logits, k, idx, vals);
  if (rc) return rc;
  const size_t need = topk_workspace_bytes(V, k) + mv_ws_bytes(V, 1, kEpiStore);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return QG_EWORKSPACE;
  return run_logits(W, V, K, group, bits, fmt, x, x_dtype, norm_w, eps, logits, k, idx, vals, ws,
                    ws_bytes, dp, stream, nullptr);
}

int qattn_decode(const float* q, const float* k_new, const float* v_new, uint16_t* k_cache,
                 uint16_t* v_cache, int H, int Hkv, int d, int T_max, int pos, float scale,
                 float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (H < 1 || Hkv < 1 || H % Hkv || T_max < 1 || pos < 0 || pos >= T_max) return QG_EINVAL;
  if (!(scale == scale) || scale > FLT_MAX || scale < -FLT_MAX) return QG_EINVAL;
  const int G = H / Hkv;
  if ((d != 64 && d != 128) || (G != 1 && G != 2 && G != 4 && G != 8)) return QG_EUNSUPPORTED;
  if (!q || !k_cache || !v_cache || !out || !aligned(q, 16) || !aligned(out, 4) ||
      !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return QG_EINVAL;
  if ((k_new == nullptr) != (v_new == nullptr)) return QG_EINVAL;
  if (k_new && (!aligned(k_new, 4) || !aligned(v_new, 4))) return QG_EINVAL;
  if ((size_t)Hkv * T_max * d * 2 > 0x7fffffffull) return QG_EUNSUPPORTED;  // 32-bit buffer offsets
  if (!ws || ws_bytes < attn_ws_bytes(H, Hkv, d) || !aligned(ws, 256)) return QG_EWORKSPACE;
  const hipError_t e = launch_attn(q, k_new, v_new, k_cache, v_cache, H, Hkv, d, T_max, pos,
                                   scale, out, ws, stream);
  return e == hipSuccess ? QG_OK : QG_ELAUNCH;
}

int qg_sample_topk(const int32_t* idx, const float* vals, int k, float temperature, float top_p,
                   uint64_t seed, uint64_t* counter, int32_t* token, hipStream_t stream) {
  DrawParams dp;
  const int rc = make_draw(temperature, top_p, seed, counter, token, &dp);
  if (rc) return rc;
  if (k < 1) return QG_EINVAL;
  if (k > QG_MAX_TOPK) return QG_EUNSUPPORTED;
  if (!idx || !vals || !aligned(idx, 4) || !aligned(vals, 4)) return QG_EINVAL;
  return launch_sample(idx, vals, k, dp, stream) == hipSuccess ? QG_OK : QG_ELAUNCH;
}

}  // extern "C"
