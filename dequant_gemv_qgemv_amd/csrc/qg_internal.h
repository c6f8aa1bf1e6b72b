// qg_internal.h -- types shared by the kernels and the C-ABI layer of the
// gfx950 quantized matvec library. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

constexpr int kThreads = 512;          // threads per workgroup (8 wave64s)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxRoutes = 8;          // routed experts per token
constexpr int kMaxSeg = kMaxRoutes + 1; // matrices one launch can gather: the routed experts + the shared one
static_assert(kMaxSeg >= kMaxRoutes + 1, "an expert launch gathers every routed expert and the shared one");

// Device pointers of one planar quantized matrix.
struct QMat {
  const uint32_t* q;
  const uint16_t* s;
  const uint16_t* b;
  const uint16_t* lut;
};

enum Epi : int {
  kEpiStore = 0,   // y = acc (+ residual)
  kEpiSwiglu = 1,  // y = silu(acc_A) * acc_B
  kEpiTopk = 2,    // y = acc, and the k largest (y, row) of the launch into tk_idx / tk_vals
};

// Top-k fused into the logits matvec: every workgroup sorts its rows' keys
// and keeps its 64 largest; groups of kTkGroup workgroups and then the groups
// are merged by the last to finish (integer tickets). Limits of the fused
// form (the host falls back to a separate top-k launch beyond them).
// Table format: per row in flight, a table of the 256 code pairs (lut[lo],
// lut[hi]) as fp16 pairs (indexed by the byte of a code word holding two
// codes) plus the row's 16 entries it is built from.
constexpr int kLutPairWords = 256;
constexpr int kLutRowWords = kLutPairWords + 8;  // + 16 fp16 entries
constexpr int kTkList = 64;       // keys per list (k <= kTkList)
constexpr int kTkGroup = 16;      // workgroups per first-level group (the last may be short)
constexpr int kTkMaxGroups = 32;  // so at most 512 workgroups
// Top-k workspace (topk_workspace_bytes): a ticket region, then the
// candidate lists of whichever form runs. The two-launch top-k's ticket is at
// offset 0, the fused form's kTkMaxGroups + 1 tickets at kTkFusedTicketOffset.
constexpr size_t kTkTicketBytes = 1024;
constexpr size_t kTkFusedTicketOffset = 512;
static_assert(kTkFusedTicketOffset + (kTkMaxGroups + 1) * 4 <= kTkTicketBytes, "fused tickets fit");

// Where the rows / columns of the logical matrix come from.
//  kSegNone: one matrix, A[0] (and B[0] for SwiGLU).
//  kSegRows: logical row r belongs to matrix A[r / seg_len] (local row r % seg_len).
//  kSegCols: logical chunk c belongs to matrix A[c / seg_len] (local chunk c % seg_len),
//            all matrices having the same N; x is the concatenation of the segments' inputs.
enum SegMode : int { kSegNone = 0, kSegRows = 1, kSegCols = 2 };

// Routing input: when `ids` is set, segments [0, n_routed) are expert ids[i]
// of a stacked tensor whose expert e starts at row e * expert_rows of
// `all_A`/`all_B`; segment n_routed (if any) is the fixed A[n_routed].
// With `logits` set, every workgroup picks the experts itself (top n_routed
// of n_experts logits, softmax over the chosen) before its first weight load,
// and workgroup 0 stores the choice in ids_store / w_store (and sel_ids /
// sel_w when set) for the launches that follow.
struct Routing {
  const int32_t* ids;     // device [n_routed] or nullptr
  const float* weights;   // device [n_routed] (K-segment input scaling) or nullptr
  int n_routed;
  int expert_rows;
  QMat all_A, all_B;
  const float* logits;    // device [n_experts] or nullptr
  int n_experts;
  int32_t* ids_store;
  float* w_store;
  int32_t* sel_ids;
  float* sel_w;
};

// One token drawn from a sorted top-k list (temperature, top-p, a uniform
// number from draw `*counter` of SplitMix64 started at `seed`).
struct DrawParams {
  float temperature;  // 0: greedy
  float top_p;        // in (0, 1]
  uint64_t seed;
  uint64_t* counter;  // device; read, then advanced by one; nullptr: draw 0
  int32_t* token;     // device; nullptr: no draw
};

struct MvParams {
  QMat A[kMaxSeg];
  QMat B[kMaxSeg];
  int nseg;
  int seg_mode;
  int seg_len;        // rows (kSegRows) or chunks (kSegCols) per segment
  int N;              // logical rows
  int K;              // logical columns (sum over K segments)
  int M;              // activation vectors (x is [M][K], y is [M][N])
  int wpr;            // uint32 words per row of each underlying matrix
  int gpr;            // groups of 64 per row of each underlying matrix
  const void* x;      // [K] activations (fp16 or fp32)
  int x_f32;
  const uint16_t* norm_w;  // [K] fp16 or nullptr
  float eps;
  const float* residual;   // [N] or nullptr
  float* y;                // [N]
  Routing route;
  // split-K
  int splits;         // number of K slices (1 = none)
  int slice_chunks;   // chunks per slice (multiple of the lanes per row)
  int grid_x;         // workgroups per slice (multiple of 8: slice s of tile t lands on XCD t%8)
  float* partials;    // [splits][n_acc][N] when splits > 1
  uint32_t* tickets;  // [grid_x] zero-initialized when splits > 1
  int tokens;         // vectors served by one launch (0 or 1: one; more: splits == 1)
  int sb_segp;        // staged scale/bias rows: 16-byte pieces per row segment of the K slice
  float* mm_ssq;      // M = 2..8 kernels: [splits][8] per-slice sums of squares per vector (norm, splits > 1)
  // fused top-k (kEpiTopk)
  int tk_k;
  uint64_t* tk_cand;     // [grid_x][kTkList] workgroup lists, then [groups][kTkList] group lists
  uint32_t* tk_tickets;  // [kTkMaxGroups + 1], zero between calls
  int32_t* tk_idx;       // [tk_k]
  float* tk_vals;        // [tk_k]
  DrawParams tk_draw;    // a token drawn from the top-k as well (tk_draw.token set)
};

// Launch configuration chosen on the host.
struct MvPlan {
  int lpr;            // lanes per row: 64, 32 or 16
  int rows;           // rows per lane slot (R)
  int splits;
  int slice_chunks;
  int grid_x;
  int depth;          // (band, pass) items in flight per wave: 2 or 4
  int sbl;            // staged scale/bias rows: 0 (per-pass loads), or 16-byte loads per lane and band
  int sb_segp;        // 16-byte pieces per staged row segment
  size_t lds_bytes;
  int tokens;         // expert launches: tokens in the batch (grid y; 0 or 1 = one)
};

hipError_t launch_mv(int bits, int fmt, int epi, const MvPlan& plan, const MvParams& p,
                     hipStream_t stream);
// Workgroups of the kernel launch_mv would pick that fit on one compute unit.
int mv_resident_per_cu(int bits, int fmt, int epi, int seg, const MvPlan& plan);

// Small-M (2..8) matrix-core kernels: plain / normed store, SwiGLU; one
// matrix (seg_mode kSegNone). K slices of mm_slice_codes() codes.
hipError_t launch_mm(int bits, int fmt, int epi, const MvPlan& plan, const MvParams& p,
                     hipStream_t stream);
int mm_slice_codes();

size_t topk_workspace_bytes(int V, int k);
// Top-k of logits[V] into idx/vals; with dp.token set, the last workgroup
// also draws the token. Returns 0, -3 (workspace too small) or -4 (launch).
int plan_and_launch_topk(const float* logits, int V, int k, int32_t* idx, float* vals, void* ws,
                         size_t ws_bytes, const DrawParams& dp, hipStream_t stream);
// The draw alone, from idx/vals as the top-k writes them.
hipError_t launch_sample(const int32_t* idx, const float* vals, int k, const DrawParams& dp,
                         hipStream_t stream);

// Decode attention against a [Hkv][T_max][d] fp16 KV cache.
size_t attn_ws_bytes(int H, int Hkv, int d);
hipError_t launch_attn(const float* q, const float* k_new, const float* v_new, uint16_t* k_cache,
                       uint16_t* v_cache, int H, int Hkv, int d, int T_max, int pos, float scale,
                       float* out, void* ws, hipStream_t stream);

// Fill kernel (graph-safe replacement for hipMemsetAsync).
hipError_t launch_fill_u32(uint32_t* dst, size_t n, uint32_t value, hipStream_t stream);

}  // namespace qg
