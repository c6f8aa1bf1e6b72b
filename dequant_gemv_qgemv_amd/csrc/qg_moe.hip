// qg_moe.hip -- one MoE expert layer per token, entirely on the device
// (GeekNews item on the 397B MoE engine: "Architecture du modele" -- 512
// experts, 4 active per token of which one is shared; "Deferred GPU Expert
// Compute" -- the combine, norm and residual run on the GPU and go straight to
// the next layer, with no host round trip).
//
// A batch of M tokens (1..8) runs in the same two launches: workgroup row
// blockIdx.y serves token blockIdx.y, with its own routing, expert rows and
// vectors (tokens do not interact).
//
// Two launches on one stream:
//  1. gate.up SwiGLU over the chosen experts plus the shared one, as one
//     matvec over (top_k+1)*F gathered rows: every workgroup first picks the
//     experts itself (top_k of the router logits, softmax over the chosen
//     ones; 512 logits cost less than a launch) and points its row segments
//     at them; workgroup 0 stores the choice in the workspace (and in sel_ids /
//     sel_w when given);
//  2. down + combine + residual, as one matvec over the K-concatenation
//     [Down_e0 | Down_e1 | ... | Down_shared] against [w0*u0, w1*u1, ..., u_sh]:
//     sum_e w_e (Down_e u_e) is that single row-by-row dot product, so the
//     weighted combine costs no extra pass.
#include <string.h>

#include "../../include/qgemv.h"
#include "qg_internal.h"

namespace qg {

int mv_plan_internal(int bits, int fmt, int epi, MvParams* p, bool have_ws, void* ws,
                     size_t ws_bytes, size_t ws_offset, int tokens, MvPlan* plan);
int mv_launch_planned(int bits, int fmt, int epi, const MvPlan& plan, const MvParams& p,
                      hipStream_t stream);
size_t mv_workspace_bytes(int N, int epi);
int device_ok();

namespace {
size_t align256(size_t v) { return (v + 255) / 256 * 256; }
// Stored routes of M tokens: ids [M][kMaxRoutes] int32, then weights
// [M][kMaxRoutes] fp32.
size_t route_bytes(int M) { return align256((size_t)M * kMaxRoutes * 8); }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_mat(const qg_qmat* W, int fmt) {
  if (!W || !W->q || !aligned(W->q, 16)) return QG_EINVAL;
  if (fmt == QG_AFFINE) {
    if (!W->scales || !W->biases || !aligned(W->scales, 2) || !aligned(W->biases, 2))
      return QG_EINVAL;
  } else if (!W->lut || !aligned(W->lut, 2)) {
    return QG_EINVAL;
  }
  return QG_OK;
}

QMat dev(const qg_qmat* W) { return QMat{W->q, W->scales, W->biases, W->lut}; }
}  // namespace

size_t moe_workspace_bytes(int F, int H, int top_k, int M) {
  const int nseg = top_k + 1;
  const size_t u = align256((size_t)M * nseg * F * 4);
  const size_t gu = mv_workspace_bytes(nseg * F, kEpiSwiglu);
  const size_t dn = mv_workspace_bytes(H, kEpiStore);
  return route_bytes(M) + u + (gu > dn ? gu : dn);
}

int plan_and_launch_moe(const qg_qmat* gate_all, const qg_qmat* up_all, const qg_qmat* down_all,
                        int n_experts, int F, int H, int bits, int fmt, const qg_qmat* shared3,
                        const float* router_logits, int top_k, const uint16_t* norm_w, float eps,
                        const float* x, float* y, int32_t* sel_ids, float* sel_w, void* ws,
                        size_t ws_bytes, hipStream_t stream, int M) {
  int rc;
  if ((rc = check_mat(gate_all, fmt)) || (rc = check_mat(up_all, fmt)) ||
      (rc = check_mat(down_all, fmt)))
    return rc;
  if (shared3) {
    for (int i = 0; i < 3; ++i)
      if ((rc = check_mat(&shared3[i], fmt))) return rc;
  }
  if (!router_logits || !x || !y || !aligned(router_logits, 4) || !aligned(x, 16) ||
      !aligned(y, 4))
    return QG_EINVAL;
  if (norm_w && (!aligned(norm_w, 16) || !(eps >= 0.f))) return QG_EINVAL;
  if ((sel_ids && !aligned(sel_ids, 4)) || (sel_w && !aligned(sel_w, 4))) return QG_EINVAL;
  if (x != y) {
    const uintptr_t a = (uintptr_t)x, b = (uintptr_t)y, n = (uintptr_t)M * H * 4;
    if (a < b + n && b < a + n) return QG_EINVAL;
  }
  if (!ws || !aligned(ws, 256) || ws_bytes < moe_workspace_bytes(F, H, top_k, M))
    return QG_EWORKSPACE;
  if (!device_ok()) return QG_EDEVICE;

  const int nseg = top_k + (shared3 ? 1 : 0);
  char* base = static_cast<char*>(ws);
  int32_t* ids_ws = reinterpret_cast<int32_t*>(base);
  float* w_ws = reinterpret_cast<float*>(base + (size_t)M * kMaxRoutes * 4);
  float* u = reinterpret_cast<float*>(base + route_bytes(M));
  const size_t mv_off = route_bytes(M) + align256((size_t)M * (top_k + 1) * F * 4);

  // 1. routing + gate.up SwiGLU over the chosen experts' rows (+ shared)
  MvParams p;
  memset(&p, 0, sizeof(p));
  p.M = 1;
  p.nseg = nseg;
  p.seg_mode = kSegRows;
  p.seg_len = F;
  if (shared3) {
    p.A[top_k] = dev(&shared3[0]);
    p.B[top_k] = dev(&shared3[1]);
  }
  p.route.ids = nullptr;
  p.route.weights = nullptr;
  p.route.n_routed = top_k;
  p.route.expert_rows = F;
  p.route.logits = router_logits;
  p.route.n_experts = n_experts;
  p.route.ids_store = ids_ws;
  p.route.w_store = w_ws;
  p.route.sel_ids = sel_ids;
  p.route.sel_w = sel_w;
  p.route.all_A = dev(gate_all);
  p.route.all_B = dev(up_all);
  p.N = nseg * F;
  p.K = H;
  p.wpr = H * bits / 32;
  p.gpr = H / 64;
  p.x = x;
  p.x_f32 = 1;
  p.norm_w = norm_w;
  p.eps = eps;
  p.residual = nullptr;
  p.y = u;

  // 2. down over the K-concatenated experts, weighted, + residual
  MvParams d;
  memset(&d, 0, sizeof(d));
  d.M = 1;
  d.nseg = nseg;
  d.seg_mode = kSegCols;
  d.seg_len = F / (128 / bits);  // chunks per expert segment
  if (shared3) d.A[top_k] = dev(&shared3[2]);
  d.route.ids = ids_ws;
  d.route.weights = w_ws;
  d.route.n_routed = top_k;
  d.route.expert_rows = H;
  d.route.all_A = dev(down_all);
  d.route.all_B = QMat{nullptr, nullptr, nullptr, nullptr};
  d.N = H;
  d.K = nseg * F;
  d.wpr = F * bits / 32;
  d.gpr = F / 64;
  d.x = u;
  d.x_f32 = 1;
  d.norm_w = nullptr;
  d.residual = x;
  d.y = y;
  // Both launches are planned before either is enqueued: a down projection
  // that cannot run (K beyond one LDS slice for a batch, workspace too small)
  // must not leave the gate.up launch's routes and u behind.
  MvPlan plan_gu, plan_dn;
  if ((rc = mv_plan_internal(bits, fmt, kEpiSwiglu, &p, true, ws, ws_bytes, mv_off, M, &plan_gu)))
    return rc;
  if ((rc = mv_plan_internal(bits, fmt, kEpiStore, &d, true, ws, ws_bytes, mv_off, M, &plan_dn)))
    return rc;
  if ((rc = mv_launch_planned(bits, fmt, kEpiSwiglu, plan_gu, p, stream))) return rc;
  return mv_launch_planned(bits, fmt, kEpiStore, plan_dn, d, stream);
}

}  // namespace qg
