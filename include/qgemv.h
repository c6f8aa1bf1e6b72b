/*
 * qgemv.h -- C ABI of the MI355X (gfx950) quantized decode matrix-vector
 * library: batch-1 (and small-M) matvecs over planar 4-bit / 2-bit
 * group-quantized weights, dequantized inside the inner loop, with the decode
 * fusions around them.
 *
 * Sources (page title, then the section that defines each operation):
 *  [F] "Booster la vitesse d'inference sur Apple Silicon -- avec le format
 *      .forge" (web research report, August 2026):
 *        TL;DR -- decode is bandwidth bound: time per token is about the
 *                 bytes read divided by the memory bandwidth;
 *        section 1 "Le chemin de decodage rapide" -- the matvec that
 *                 dequantizes inside its inner loop; the fusions rmsnorm +
 *                 QKV matvec, residual + norm, gate.up SwiGLU in one kernel,
 *                 logits matvec + top-k on the GPU returning only the chosen
 *                 entries; a decode loop that allocates nothing;
 *        section 3 item 4 -- planar quantization: 4-bit codes packed in
 *                 uint32 with separate scale and bias tensors (group 64);
 *                 a palettized type with 4-bit indices into a 16-entry fp16
 *                 table.
 *  [G] GeekNews item on a C/Metal engine running a 397B MoE on a 48 GB
 *      MacBook Pro (fr.news.hada.io topic 27758):
 *        "Architecture du modele" -- 512 experts per layer, 4 active per
 *                 token including one shared expert, hidden size 4096;
 *        "Noyau de dequantification optimise FMA" -- the weight is
 *                 nibble*scale + bias, and the product with x is rewritten
 *                 as fma(nibble, scale*x, bias*x);
 *        "Shaders de calcul Metal" / "Deferred GPU Expert Compute" -- 4-bit
 *                 and 2-bit dequant matvecs, SwiGLU, RMS norm, and the MoE
 *                 combine + residual on the GPU, handed straight to the next
 *                 layer.
 *  [B] gist.science explainer of the BaseRT paper ("BaseRT: Best-in-Class LLM
 *      Inference on Apple Silicon via Native Metal"):
 *        "Methodologie" -- one matvec variant per quantization format from
 *                 Q2 to FP16, each dequantizing inside its inner loop.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument except the qg_qmat descriptor itself is a DEVICE
 *    pointer owned by the caller. The descriptor (qg_qmat) is a HOST struct
 *    read during the call only. Buffers must stay alive until the work queued
 *    on `stream` has finished.
 *  - Calls are asynchronous: they validate, enqueue kernels on `stream`
 *    (NULL = the device's default stream) and return. They never allocate,
 *    free or synchronize, and print nothing.
 *  - Return value: QG_OK (0) or a negative status. Validation happens before
 *    anything is enqueued; a call that fails validation enqueues nothing.
 *    QG_ELAUNCH reports an error from the HIP runtime after enqueueing.
 *  - Weight layout (planar, [F] section 3 item 4): row n of an N x K matrix
 *    is contiguous along K. Codes: q[n][K*bits/32] uint32; element k sits in
 *    word k/(32/bits) at bit offset bits*(k mod 32/bits), least significant
 *    field first. Affine format: scales[n][K/64], biases[n][K/64] fp16, and
 *    W[n][k] = code*scale + bias for the group of 64 consecutive k that holds
 *    k; bits = 2, 4 or 8 ([B] Methodologie: Q2 to Q8). LUT format (bits = 4
 *    only): lut[n][16] fp16 and W[n][k] = lut[n][code]. Dense format (bits =
 *    16, [B] Methodologie: FP16): each 16-bit field is the fp16 weight itself,
 *    so q is the row-major fp16 matrix [N][K] read as words; no scales,
 *    biases or table. group must be 64 and K a multiple of 64 for every
 *    format.
 *  - fp16 arrays are passed as uint16_t bit patterns (IEEE 754 binary16).
 *  - Activations x are [M][K] row-major (fp16 or fp32); outputs are fp32.
 *  - Accumulation is fp32. Results are deterministic: the same call on the
 *    same inputs gives bitwise the same outputs (no floating-point atomics).
 *  - Alignment: q and x must be 16-byte aligned; fp16 arrays 2-byte aligned;
 *    fp32 arrays 4-byte aligned. Otherwise QG_EINVAL.
 *  - Several activation vectors (M = 2..8; qgemv, qgemv_rmsnorm, qswiglu):
 *    2- and 4-bit codes run on the matrix cores ([F] section 1: the
 *    dispatcher's choice by M) and additionally need K % 512 == 0 and
 *    16-byte aligned scales/biases (affine) or lut (LUT format), otherwise
 *    QG_EUNSUPPORTED. 8-bit and dense weights run the one-vector kernel once
 *    per vector in the same launch (each vector's weight pass after the first
 *    mostly hits the last-level cache) and need K within one LDS slice
 *    (QG_EUNSUPPORTED otherwise). With
 *    K > 4096 they need the workspace (QG_EWORKSPACE without it).
 *  - Workspace: calls that need scratch device memory take (ws, ws_bytes);
 *    qg_workspace_bytes() sizes it. The caller allocates it once, clears it
 *    once with qg_workspace_init(), and may then reuse it for every call on
 *    one stream (each call leaves it ready for the next). Two calls that run
 *    at the same time must not share a workspace.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define QG_OK 0
#define QG_EINVAL (-1)        /* NULL required pointer, bad size, misalignment, bad aliasing */
#define QG_EUNSUPPORTED (-2)  /* valid but not provided: group != 64, affine bits not 2/4/8,
                                 LUT with bits != 4, dense with bits != 16, M outside [1,8],
                                 K or k beyond the limits below, M > 1 with 2/4-bit codes
                                 and K % 512 != 0 or scales/biases/lut not 16-byte aligned,
                                 M > 1 with 8-bit/dense weights and K beyond one slice */
#define QG_EWORKSPACE (-3)    /* ws NULL or smaller than qg_workspace_bytes() */
#define QG_ELAUNCH (-4)       /* the HIP runtime reported an error while enqueueing */
#define QG_EDEVICE (-5)       /* no usable gfx950 device for the current HIP device */

/* ---- enums ------------------------------------------------------------- */
#define QG_AFFINE 0 /* W = code*scale + bias per group of 64 */
#define QG_LUT 1    /* W = lut[row][code], 16 fp16 entries per row, bits = 4 */
#define QG_DENSE 2  /* W = the fp16 value of each 16-bit field, bits = 16 ([B] FP16 variant) */

#define QG_F16 0 /* activation dtype: IEEE binary16 */
#define QG_F32 1 /* activation dtype: IEEE binary32 */

#define QG_OP_GEMV 0
#define QG_OP_GEMV_RMSNORM 1
#define QG_OP_SWIGLU 2
#define QG_OP_MOE 3
#define QG_OP_LOGITS_TOPK 4
#define QG_OP_ATTN 5

/* Limits. K counts columns of one matrix (for qmoe_experts: the hidden size
 * and the expert FFN size); k counts top-k entries. */
#define QG_MAX_K 65536
#define QG_MAX_M 8
#define QG_MAX_TOPK 1024
/* One matrix (or one expert's rows) may hold at most 2^31 - 1 bytes of codes. */

/* A planar quantized matrix ([F] section 3 item 4). Host struct holding
 * device pointers; see the layout above. Unused members must be NULL. */
typedef struct qg_qmat {
    const uint32_t *q;      /* [N][K*bits/32] code words (dense: fp16 [N][K]), 16-byte aligned */
    const uint16_t *scales; /* [N][K/64] fp16 (QG_AFFINE) */
    const uint16_t *biases; /* [N][K/64] fp16 (QG_AFFINE) */
    const uint16_t *lut;    /* [N][16] fp16 (QG_LUT) */
} qg_qmat;

/* Human-readable name of a status code (static string, never NULL). */
const char *qg_status_str(int status);

/* Bytes of workspace that `op` needs for these sizes (0 if none). For
 * QG_OP_MOE, N is the hidden size, K the expert FFN size, M the tokens of a
 * batch (1 for qmoe_experts) and k the number of
 * routed experts; for QG_OP_LOGITS_TOPK, N is the vocabulary size and k the
 * number of entries returned; for QG_OP_ATTN, N is the number of query heads
 * H, M the number of kv heads Hkv and k the head dimension d (K, bits and fmt
 * are not used; the size does not depend on the cache length). Returns a
 * status; *bytes is set on QG_OK. */
int qg_workspace_bytes(int op, int N, int K, int M, int bits, int fmt, int k, size_t *bytes);

/* Clears a workspace before its first use (a fill kernel on `stream`, safe to
 * record in a HIP graph). ws_bytes must be a multiple of 4. */
int qg_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* Variant override for tests and benchmarks; normal callers never need it.
 * knob 0 = number of K slices (split-K, needs a workspace), 1 = rows per lane
 * (1 or 2), 2 = lanes per row (16, 32 or 64), 3 = resident workgroups per
 * compute unit, 4 = (band, pass) items in flight per wave (2 or 4), 5 = 1 for
 * the two-launch form of qlogits_topk, 6 = 1 for scale/bias rows staged in
 * LDS once per band (affine formats, 16-byte aligned rows) in place of two
 * 2-byte loads per pass; value 0 restores the automatic choice.
 * Process-wide; affects calls made after it returns. QG_EINVAL for an unknown
 * knob or value. */
int qg_tune(int knob, int value);

/* qgemv -- y[m][n] = residual[m][n] + sum_k W[n][k] * x[m][k]
 * The decode matvec that dequantizes inside its inner loop ([F] section 1;
 * the weight form and the fma(code, scale*x, bias*x) rewrite: [G] FMA
 * section). residual may be NULL; it may be the same pointer as y (in-place
 * residual add) but must not overlap it otherwise. x must not overlap y.
 *   W      quantized N x K matrix (fmt, bits as above; group must be 64)
 *   x      [M][K] activations of dtype x_dtype
 *   y      [M][N] fp32 output
 *   M      number of activation vectors, 1..8 */
int qgemv(const qg_qmat *W, int N, int K, int M, int group, int bits, int fmt,
          const void *x, int x_dtype, const float *residual, float *y,
          void *ws, size_t ws_bytes, hipStream_t stream);

/* qgemv_rmsnorm -- y = residual + W . rmsnorm(x), with
 *   rmsnorm(x)_k = x_k * norm_w[k] / sqrt((1/K) sum_j x_j^2 + eps)
 * per activation vector ([F] section 1: rmsnorm fused into the QKV matvec).
 * norm_w: [K] fp16. Other arguments as qgemv. */
int qgemv_rmsnorm(const qg_qmat *W, int N, int K, int M, int group, int bits, int fmt,
                  const void *x, int x_dtype, const uint16_t *norm_w, float eps,
                  const float *residual, float *y, void *ws, size_t ws_bytes,
                  hipStream_t stream);

/* qswiglu -- u[m][j] = silu((Wgate x')_j) * (Wup x')_j, silu(z) = z/(1+e^-z),
 * where x' = rmsnorm(x) when norm_w is non-NULL and x otherwise ([F]
 * section 1: gate.up SwiGLU in one kernel, residual + norm). Wgate and Wup
 * are both F x K with the same bits/fmt. u: [M][F] fp32, must not overlap x. */
int qswiglu(const qg_qmat *Wgate, const qg_qmat *Wup, int F, int K, int M, int group,
            int bits, int fmt, const void *x, int x_dtype, const uint16_t *norm_w, float eps,
            float *u, void *ws, size_t ws_bytes, hipStream_t stream);

/* qmoe_experts -- one MoE expert layer for one token ([G] "Architecture du
 * modele", "Deferred GPU Expert Compute"):
 *   ids   = the top_k router logits (larger first, equal values by lower
 *           index); w_i = softmax over the chosen logits only;
 *   x'    = rmsnorm(x; norm_w) (x itself when norm_w is NULL);
 *   y     = x + sum_i w_i * Down_{ids_i}(SwiGLU_{ids_i}(x'))
 *             + Down_sh(SwiGLU_sh(x'))            (shared expert, weight 1)
 * Expert e's gate/up are rows [e*F, (e+1)*F) of gate_all/up_all (each
 * (n_experts*F) x H), its down is rows [e*H, (e+1)*H) of down_all
 * ((n_experts*H) x F). shared3 = {gate, up, down} of the always-on expert
 * (F x H, F x H, H x F) or NULL for none. Routing, expert selection and the
 * combine all stay on the device. x, y: [H] fp32, y may equal x. Expert
 * weights take the affine format (2-, 4- or 8-bit codes).
 * router_logits: [n_experts] fp32. sel_ids/sel_w (device, [top_k], int32 /
 * fp32) receive the routing decision when non-NULL. 1 <= top_k <= 8. */
int qmoe_experts(const qg_qmat *gate_all, const qg_qmat *up_all, const qg_qmat *down_all,
                 int n_experts, int F, int H, int group, int bits, int fmt,
                 const qg_qmat *shared3, const float *router_logits, int top_k,
                 const uint16_t *norm_w, float eps, const float *x, float *y,
                 int32_t *sel_ids, float *sel_w, void *ws, size_t ws_bytes,
                 hipStream_t stream);

/* qmoe_experts_batch -- qmoe_experts for M tokens at once (1 <= M <= QG_MAX_M;
 * [F] section 1: several vectors per step), in the same two launches. Each
 * token routes, runs its chosen experts and combines on its own; tokens do
 * not interact. x, y: [M][H] fp32 row-major (y may equal x, otherwise they
 * must not overlap); router_logits: [M][n_experts] fp32; sel_ids / sel_w:
 * NULL or [M][top_k]. Workspace: qg_workspace_bytes(QG_OP_MOE, H, F, M, bits,
 * fmt, top_k, ...). QG_EUNSUPPORTED when a token's hidden size or
 * concatenated expert width would need split-K (beyond one LDS slice). Other
 * arguments and conditions as qmoe_experts, which is this call with M = 1. */
int qmoe_experts_batch(const qg_qmat *gate_all, const qg_qmat *up_all, const qg_qmat *down_all,
                       int n_experts, int F, int H, int M, int group, int bits, int fmt,
                       const qg_qmat *shared3, const float *router_logits, int top_k,
                       const uint16_t *norm_w, float eps, const float *x, float *y,
                       int32_t *sel_ids, float *sel_w, void *ws, size_t ws_bytes,
                       hipStream_t stream);

/* qlogits_topk -- z = W . x' (x' = rmsnorm(x; norm_w), or x when norm_w is
 * NULL), written to logits[V]; then the k largest entries of z, larger first
 * and equal values by lower index, into idx[k] (int32) and vals[k] (fp32)
 * ([F] section 1: logits matvec + top-k on the GPU, only the chosen entries
 * need to come back). M must be 1 (x is [K]). 1 <= k <= min(V, QG_MAX_TOPK).
 * For k <= 64 one launch where the shape allows it: each matvec workgroup
 * keeps its rows' 64 largest and the last workgroups to finish merge the
 * lists; otherwise the matvec and then a separate top-k launch. Both forms
 * return the same bits. Calls that overlap on one workspace race. */
int qlogits_topk(const qg_qmat *W, int V, int K, int group, int bits, int fmt,
                 const void *x, int x_dtype, const uint16_t *norm_w, float eps,
                 float *logits, int k, int32_t *idx, float *vals,
                 void *ws, size_t ws_bytes, hipStream_t stream);

/* qg_logits_topk_launches -- *launches = the number of kernels (1 or 2) that
 * qlogits_topk and qlogits_topk_noalloc enqueue for this head (W may be NULL:
 * then its scale/bias arrays are taken as 16-byte aligned) on the current
 * device under the current tuning (for profilers and graph budgets;
 * qlogits_sample takes the same number). Enqueues nothing. Statuses as qlogits_topk;
 * QG_EDEVICE without a usable gfx950. */
int qg_logits_topk_launches(const qg_qmat *W, int V, int K, int group, int bits, int fmt, int k,
                            int *launches);

/* qlogits_topk_noalloc -- qlogits_topk without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments (minus
 * ws / ws_bytes), results, kernels and errors as qlogits_topk. Its scratch
 * memory (top-k candidates, split-K partials and tickets) is a
 * library-held device array of 24 MiB per GPU, kept until the process ends;
 * a call whose workspace need (qg_workspace_bytes(QG_OP_LOGITS_TOPK, V, K, 1,
 * bits, fmt, k)) exceeds it returns QG_EUNSUPPORTED (this is V <= 385828
 * for k = 40). The call itself allocates and frees nothing; its first call on
 * a device clears the array with a fill kernel on `stream`, ahead of its own
 * kernels. Every call on one GPU shares that GPU's array and leaves it ready
 * for the next call, so calls that may overlap on one GPU (different streams
 * without ordering between them) race and must not be made. */
int qlogits_topk_noalloc(const qg_qmat *W, int V, int K, int group, int bits, int fmt,
                         const void *x, int x_dtype, const uint16_t *norm_w, float eps,
                         float *logits, int k, int32_t *idx, float *vals, hipStream_t stream);

/* Sampling after top-k ([F] section 1: logits matvec + top-k sampling on the
 * GPU, only the token comes back). The page names the step, not its rule;
 * the rule implemented:
 *   temperature == 0: the token is idx[0] (greedy);
 *   otherwise w_i = exp((vals_i - vals_0) / temperature) over the k
 *   candidates in their order (vals_0 is the largest); top_p keeps the
 *   shortest prefix whose weight sum reaches top_p times the total (at least
 *   one candidate); the token is idx[i] for the first i whose running sum
 *   w_0 + ... + w_i exceeds u times that prefix sum.
 * u = (splitmix64(seed, c) >> 11) * 2^-53 in [0, 1): output number c of the
 * SplitMix64 generator started at state `seed` (Steele, Lea and Flood,
 * OOPSLA 2014). c = *counter, and the call then stores c + 1 there, so every
 * call (greedy ones too) consumes one number and a captured graph replayed n
 * times draws n successive numbers; counter NULL means c = 0 on every call.
 * Evaluated in double precision, sums in index order.
 *   temperature  >= 0 and finite;   top_p  in (0, 1]
 *   counter      device uint64, 8-byte aligned, or NULL
 *   token        device int32 (receives the token id)
 * QG_EINVAL for an argument outside these ranges. */

/* qlogits_sample -- qlogits_topk (same arguments, workspace and results)
 * followed by the draw from its k candidates, in the launch that finishes the
 * top-k (the matvec's own launch where qlogits_topk takes one). */
int qlogits_sample(const qg_qmat *W, int V, int K, int group, int bits, int fmt,
                   const void *x, int x_dtype, const uint16_t *norm_w, float eps,
                   float *logits, int k, int32_t *idx, float *vals,
                   float temperature, float top_p, uint64_t seed, uint64_t *counter,
                   int32_t *token, void *ws, size_t ws_bytes, hipStream_t stream);

/* qg_sample_topk -- the draw alone, from a top-k list in the form
 * qlogits_topk writes it: idx[k] (int32), vals[k] (fp32, larger first), both
 * device pointers. 1 <= k <= QG_MAX_TOPK. One small launch on `stream`. */
int qg_sample_topk(const int32_t *idx, const float *vals, int k, float temperature,
                   float top_p, uint64_t seed, uint64_t *counter, int32_t *token,
                   hipStream_t stream);

/* qattn_decode -- one decode step of attention against a KV cache ([F]
 * section 2 "KV cache": preallocated at its maximum length, laid out along the
 * time axis per head, fp16; one query per head; split along the cache for
 * long contexts; GQA).
 *   k_cache, v_cache  [Hkv][T_max][d] fp16, device, 16-byte aligned
 *   q                 [H][d] fp32 (16-byte aligned), out [H][d] fp32
 *   k_new, v_new      [Hkv][d] fp32 or both NULL: when given, they are first
 *                     written (rounded to nearest fp16) at position pos
 * Then, for query head h and kv head g = h / (H / Hkv), over t = 0..pos:
 *   out[h] = sum_t softmax_t(scale * q[h] . K[g][t]) V[g][t].
 * d must be 64 or 128 and H / Hkv one of 1, 2, 4, 8 (QG_EUNSUPPORTED
 * otherwise); 0 <= pos < T_max. The workspace (QG_OP_ATTN) holds the
 * slices' partial results and one ticket per kv head; cleared once with
 * qg_workspace_init, it is left clear by every call. out must not overlap q
 * or the caches. */
int qattn_decode(const float *q, const float *k_new, const float *v_new, uint16_t *k_cache,
                 uint16_t *v_cache, int H, int Hkv, int d, int T_max, int pos, float scale,
                 float *out, void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- bandwidth probes (measurement only) ---------------------------------
 * The decode matvec is bound by HBM bandwidth ([F] TL;DR: time per token is
 * about the bytes read divided by the bandwidth); these give the achievable
 * figures to compare against. Both stream `bytes` (a multiple of 16, 16-byte
 * aligned) with 16-byte non-temporal accesses over `blocks` workgroups of 256
 * threads. qg_probe_read reads src once and writes one uint32 per thread to
 * out (out must hold blocks*256 entries); flags bit 0 = ordinary (cached)
 * loads instead of non-temporal ones. qg_probe_copy copies src to dst (no
 * overlap). QG_EINVAL on bad arguments. */
int qg_probe_read(const void *src, size_t bytes, uint32_t *out, int blocks, int flags,
                  hipStream_t stream);
int qg_probe_copy(void *dst, const void *src, size_t bytes, int blocks, hipStream_t stream);

/* qg_probe_phases -- one launch of `blocks` workgroups of 512 threads that
 * reads nphases byte ranges of src in order, the way a persistent kernel
 * would stream a whole token's matvecs ([F] TL;DR lever 3 and section 1:
 * per-token overhead). ranges: device array [2 * nphases] uint64 of
 * (byte offset, byte count), each a multiple of 16; a range is clipped to
 * src_bytes. barrier = 1 adds a device-wide barrier between ranges (each
 * workgroup publishes one coherent word, raises flags[block] to the range
 * number and waits for every flag); barrier = 2 does the same and issues
 * each thread's first loads of the next range before the wait (as a
 * persistent kernel would fetch the next matvec's weights, which do not
 * depend on the barrier). With a barrier, flags [blocks] must be zero at launch,
 * err [1] counts workgroups whose wait exceeded
 * spin_limit polls (1 <= spin_limit <= 2^22; the launch then ends early and
 * its timing is void). With barrier = 1, blocks must not exceed 1024 nor
 * the workgroups that fit on the device at once (QG_EUNSUPPORTED). out
 * [blocks * 512] receives one uint32 per thread. Measurement only. */
int qg_probe_phases(const void *src, size_t src_bytes, const uint64_t *ranges, int nphases,
                    int barrier, uint32_t *flags, uint32_t *out, uint32_t *err, int blocks,
                    int spin_limit, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
