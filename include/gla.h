/*
 * gla.h -- C ABI of the MI355X (gfx950) chunk-parallel gated linear attention.
 *
 * The operation (per batch row b and head h) is the gated linear-attention
 * recurrence
 *
 *     S_t = diag(alpha_t) S_{t-1} + k_t v_t^T,      o_t = S_t^T q_t,
 *
 * with S_{-1} = h0 and hT = S_{T-1}, as written on the FLAT page ("FLAT: Flash
 * Linear Attention on TPUs", section Linear Attention > Forward Recurrence and
 * the table of gated forms, whose notation F_t = prod_{s<=t} f_s covers both
 * gate forms here):
 *
 *   - GLA_GATE_SCALAR: one gate per (b, t, h), the Mamba-2 / SSD form;
 *   - GLA_GATE_VECTOR: one gate per key channel, f_t in R^{d_k}, the GLA form.
 *
 * g holds the natural logarithm of the gate, alpha_t = exp(g_t).  For every
 * finite g <= 0 (a decay; the pages' gate forms are all of this kind) the
 * results are those of the recurrence up to rounding, however strong the decay:
 * inside a chunk whose |g| all stay within 1.875 the vector gate's decays are
 * factored around one reference row (every factor within exp(+-60)); a chunk
 * with a stronger gate forms each exp(beta_r - beta_s) of its score pairs
 * directly, and its log-gate gradient from the non-cancelling terms only.
 * Positive g are accepted and computed by the same formulas; their results stay
 * finite while the growth they describe stays within float32's range.  There
 * is no internal 1/sqrt(d) scale: callers pre-scale q and k.
 *
 * Document resets (JLA page, "JLA: JAX Linear Attention", the segment_ids
 * paragraph): wherever segment_ids[b,t] differs from segment_ids[b,t-1] the
 * carried state is dropped before token t is added (alpha_t is then unused),
 * so a packed row computes exactly what its documents would compute one by
 * one; h0 seeds only the row's first document and hT is the state after the
 * row's last token.
 *
 * gla_bwd returns the gradients of a scalar loss L given dO = dL/do and
 * dhT = dL/dhT (FLAT page, Linear Attention > Backward Recurrence: the state
 * gradient runs backwards in time with the gate scaling it at each step, and
 * the log-gate gradient is f_t * (grad_{H_t} (.) H_{t-1}) 1_V).  dg is the
 * gradient with respect to the log gate g; it is 0 at reset tokens.  When
 * H_qk < H, each q/k head is read by H / H_qk consecutive heads (head h reads
 * q/k head h / (H / H_qk)) and dq, dk are summed over those heads (FLAT page,
 * Pallas Kernels > Gated Linear Attention, the paragraph on head sharing).
 *
 * Layouts: all tensors are row-major; q, k, v, dq, dk, dv may have token rows
 * further apart than packed (see the row strides below), every other tensor is
 * contiguous.
 *     q, k, dq, dk           [B, T, H_qk, d_k]   dtype
 *     v, o, dO, dv           [B, T, H, d_v]      dtype
 *     g, dg  scalar gate     [B, T, H]           dtype
 *            vector gate     [B, T, H, d_k]      dtype
 *     h0, hT, dhT, dh0       [B, H, d_k, d_v]    float32 always
 *     segment_ids            [B, T]              int32
 * dtype is GLA_F32 (IEEE float32) or GLA_BF16 (bfloat16).  bf16 products run
 * on the bf16 matrix cores with float32 accumulation.  float32 inputs with the
 * scalar gate and d_k = d_v = 128 run every product as three bf16 products of
 * operands split into high and low bf16 halves (x = hi + lo), float32
 * accumulation (about 2^-16 relative error per product, the dropped lo * lo
 * term); other float32 shapes use the float32 matrix cores.  Every state, gate
 * prefix and gate-gradient sum is carried in float32.  Outputs in bf16 are
 * rounded to nearest even.
 *
 * Pointers: every tensor pointer is a device pointer on the current HIP
 * device, 16-byte aligned.  Nullable pointers: h0 (zeros), segment_ids (one
 * document per row), hT (not written), dhT (zeros), dh0 (not written), and the
 * activation and gradient pointers when T == 0 (then hT = h0 and dh0 = dhT, or
 * zeros).  All others are required.  ws is a device workspace of ws_bytes bytes, at least
 * gla_workspace_size(); it may be NULL when that size is 0.
 *
 * Ownership and ordering: the caller allocates and frees every buffer; the
 * library allocates nothing, frees nothing, never synchronises and keeps no
 * state between calls.  Work is enqueued on `stream` (a hipStream_t; NULL is
 * the default stream) and the call returns before it completes.  Inputs are
 * read only.  Outputs are fully overwritten (never accumulated into) and must
 * not overlap inputs, each other or the workspace (dq, dk and dv may interleave
 * in one buffer, as in the fused layout below; elements outside them are not
 * touched).  Two calls that share a
 * workspace must be ordered on one stream.
 *
 * Errors: every argument is checked on the host before anything is launched;
 * a failed check returns a negative gla_status and enqueues nothing.  Sizes:
 * B >= 1, T >= 0, H >= 1, 1 <= H_qk <= H with H % H_qk == 0, d_k and d_v in
 * {64, 128}, chunk == 64, split >= 0.  A launch failure returns GLA_E_LAUNCH.  There is no
 * fallback path: a shape the kernels do not cover is an error.
 */
#ifndef GLA_H
#define GLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GLA_OK = 0,
    GLA_E_NULL = -1,        /* a required pointer is NULL */
    GLA_E_SHAPE = -2,       /* sizes inconsistent or out of range */
    GLA_E_DTYPE = -3,       /* unknown dtype or gate kind */
    GLA_E_UNSUPPORTED = -4, /* valid, but no kernel for this d_k / d_v / chunk (convolution: K, C; norm: d) */
    GLA_E_ALIGN = -5,       /* a pointer is not 16-byte aligned */
    GLA_E_WORKSPACE = -6,   /* workspace missing or smaller than required */
    GLA_E_DEVICE = -7,      /* no HIP device, or the current device is not gfx950 */
    GLA_E_LAUNCH = -8,      /* a kernel launch failed */
    GLA_E_SCRATCH = -9      /* gla_fwd_noalloc: the problem needs more than its fixed scratch */
} gla_status;

typedef enum { GLA_F32 = 0, GLA_BF16 = 1 } gla_dtype;
typedef enum { GLA_GATE_SCALAR = 0, GLA_GATE_VECTOR = 1 } gla_gate;

/* Problem description, passed by pointer (host memory, read during the call). */
typedef struct {
    int64_t B, T, H, H_qk, d_k, d_v;
    int32_t chunk;  /* tokens per chunk; 64 */
    int32_t gate;   /* gla_gate */
    int32_t dtype;  /* gla_dtype */
    int32_t split;  /* sequence pieces per (b, h): 0 = chosen from the sizes; >= 1 forces
                       that many (fewer if the row has fewer chunks); see below */
    /* Row strides: elements from token (b, t) to token (b, t + 1) (and from the
     * last token of row b to the first of row b + 1) of q and k (ld_qk), v
     * (ld_v), dq and dk (ld_dqk) and dv (ld_dv); 0 = packed (H_qk * d_k, or
     * H * d_v).  Head h of token (b, t) of q starts at q + (b * T + t) * ld_qk
     * + h * d_k.  A non-zero stride is at least the packed one and a multiple of
     * 16 bytes.  o, dO, g and dg are always packed. */
    int64_t ld_qk, ld_v, ld_dqk, ld_dv;
    int32_t flags;      /* 0, or GLA_SAVE_STATES; other bits: GLA_E_UNSUPPORTED */
    int32_t reserved;   /* 0 */
    int64_t generation; /* with GLA_SAVE_STATES: the caller's count of changes to the inputs */
} gla_problem;

/* Saved states (flags = GLA_SAVE_STATES, given to both calls of a forward /
 * backward pair that share one workspace).  The backward needs the state
 * entering every chunk; without this flag it recomputes them with a state
 * pass over k, v and g (and, for split rows, a summary pass over the same
 * inputs).  With it, gla_fwd also stores those states (in the input dtype) in
 * ws, as the forward kernel passes through them, together with a stamp of what
 * they were computed from: the problem's sizes, dtype, gate and strides, the q,
 * k, v, g, h0 and segment_ids pointers and p->generation.  gla_bwd compares the
 * stamp with its own call's on the device: when they are equal its state passes
 * exit at once and it uses the stored states; otherwise it recomputes them (and
 * stamps the workspace for its own inputs).  The caller's part: give both calls
 * the same generation only while the inputs' contents are unchanged (change it
 * whenever they are written in place).  The workspace size is the same for both
 * calls with this flag (gla_workspace_size(p, 0) == gla_workspace_size(p, 1)).
 * The forward stores states for the scalar gate with d_k = d_v = 128, bf16 or
 * fp32: there the backward's state pass is skipped (bf16: it runs alone before
 * a walk over the chunks; fp32: the state-gradient pass then runs alone, over
 * the backward's own split).  For every other problem (the vector gate, other
 * head sizes) the flag only sets the workspace size: there the state pass runs
 * beside the state-gradient pass, so skipping it would gain less than the
 * forward's store of every state costs, and the backward recomputes the states
 * as without the flag.  Results equal the recomputing backward's up to float
 * rounding order. */
#define GLA_SAVE_STATES 1

/* Fused projection.  The FLAT page ("FLAT: Flash Linear Attention on TPUs",
 * sections Gated Linear Attention (the data-movement paragraph) and Full Linear
 * Attention Layer) has the kernels read q, k and v straight out of the one
 * projection output and write one fused gradient, so that no layout copies,
 * splits or concatenations run around them.  With the projection output X of
 * shape [B, T, W], W = 2 * H_qk * d_k + H * d_v, holding q | k | v along its
 * last axis, pass q = X, k = X + H_qk * d_k, v = X + 2 * H_qk * d_k and
 * ld_qk = ld_v = W; with a gradient buffer dX of the same shape, pass dq = dX,
 * dk = dX + H_qk * d_k, dv = dX + 2 * H_qk * d_k and ld_dqk = ld_dv = W, and
 * gla_bwd fills dX completely. */

/* Sequence split.  The time axis of every (b, h) can be cut into pieces of
 * whole chunks that run in parallel: a piece maps the state entering it to the
 * state leaving it by S -> D S + L (D diagonal, the product of the gates over
 * the piece, 0 once a document starts inside it; L the state the piece builds
 * from zero), and these maps compose exactly, so a short pass computes (L, D)
 * per piece, a P-step combine gives each piece its entry state (the state
 * gradient at its exit, in the backward) and the main kernels then run the
 * pieces side by side.  The JLA page ("JLA: JAX Linear Attention", the case
 * of long single sequences among those where it is slower) contrasts such an
 * exact split with starting each piece early from a zero state, which only
 * approximates; the chunkwise state passing on the FLAT page (Linear Attention
 * > Forward Recurrence) is the same identity between chunks.  Results equal
 * the unsplit ones up to float32 rounding order.  With split == 0 the library splits only when B * H is too
 * small to occupy the device.  The workspace depends on the split. */

/* Bytes of device workspace gla_fwd (for_backward == 0) or gla_bwd
 * (for_backward != 0) needs for this problem.  Writes it to *bytes and returns
 * GLA_OK, or returns a negative status for an invalid problem. */
int gla_workspace_size(const gla_problem* p, int for_backward, size_t* bytes);

/* Forward: o (and hT if non-NULL) from q, k, v, g, h0, segment_ids. */
int gla_fwd(const gla_problem* p, const void* q, const void* k, const void* v, const void* g,
            const float* h0, const int32_t* segment_ids, void* o, float* hT, void* ws,
            size_t ws_bytes, void* stream);

/* Forward for callers that cannot allocate: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid allocation.  The same
 * computation and kernels as gla_fwd (results identical bit for bit), without a
 * workspace argument: the workspace gla_fwd would take (only sequence-split
 * problems need one: the per-piece summaries and entry states) is a fixed
 * device array inside the library, gla_fwd_noalloc_max_scratch() bytes (64 MiB),
 * one per device for the life of the process.  A problem whose
 * gla_workspace_size(p, 0) exceeds it returns GLA_E_SCRATCH before anything is
 * enqueued.  The call allocates and frees nothing (the array's address is looked
 * up once per device, on the first call made with that device current).  Every
 * call on one device shares that device's array, which keeps the last call's
 * contents: calls that may overlap on one device (different streams, no
 * ordering between them) race, so order them on one stream.  Nothing in the
 * array needs to start at zero.  Other arguments, ownership and errors as for
 * gla_fwd. */
int gla_fwd_noalloc(const gla_problem* p, const void* q, const void* k, const void* v, const void* g,
                    const float* h0, const int32_t* segment_ids, void* o, float* hT, void* stream);

/* Bytes of the fixed scratch gla_fwd_noalloc works in. */
size_t gla_fwd_noalloc_max_scratch(void);

/* Backward: dq, dk, dv, dg (and dh0 if non-NULL) from the forward's inputs and
 * the upstream gradients dO and dhT.  Recomputes whatever it needs from the
 * inputs; it does not read anything gla_fwd produced. */
int gla_bwd(const gla_problem* p, const void* q, const void* k, const void* v, const void* g,
            const float* h0, const int32_t* segment_ids, const void* dO, const float* dhT,
            void* dq, void* dk, void* dv, void* dg, float* dh0, void* ws, size_t ws_bytes,
            void* stream);

/* ---- Short depthwise causal convolution (the step before the recurrence)
 *
 * FLAT page ("FLAT: Flash Linear Attention on TPUs"), section Depthwise Causal
 * Short Convolution: per batch row b, time step t and channel c, with K taps
 * w[k][c] and a bias[c],
 *
 *     z_t = bias + sum_{k=0}^{K-1} w_k * x_{t-(K-1-k)}     (x before t = 0 is 0),
 *     y_t = SiLU(z_t) = z_t * sigmoid(z_t),
 *
 * so tap K-1 multiplies the current input.  The backward takes dy = dL/dy and
 * returns dx = sum_k w_k * dz_{t+(K-1-k)} (dz past the end is 0), dw[k][c] =
 * sum over all b, t of x_{t-(K-1-k)} * dz_t and db[c] = sum of dz_t, where
 * dz = dy * SiLU'(z), SiLU'(z) = s (1 + z (1 - s)), s = sigmoid(z).  The
 * convolution has no document resets (the page's has none).
 *
 * Layouts (row-major, contiguous): x, y, dy, dx [B, T, C] in the problem's
 * dtype; w, dw [K, C], bias, db [C] float32.  Sums run in float32; bf16
 * outputs are rounded to nearest even.  Sizes: B >= 1, T >= 0, K == 4, C a
 * multiple of 8.  Pointers are device pointers on the current HIP device,
 * 16-byte aligned; bias and db may be NULL (no bias; bias gradient not
 * written), and x, y, dy, dx may be NULL when T == 0; all others are required.  ws is a device workspace of at least
 * gla_conv_workspace_size() bytes (the backward's per-block partial sums of dw
 * and db, reduced in a fixed order, so results are the same on every run).
 * Ownership, ordering and errors are as for gla_fwd / gla_bwd above: the caller
 * owns every buffer, work is enqueued on `stream`, every argument is checked
 * before anything is launched, outputs are overwritten and must not alias the
 * inputs. */
typedef struct {
    int64_t B, T, C;  /* batch rows, time steps, channels */
    int32_t K;        /* taps; 4 */
    int32_t dtype;    /* gla_dtype of x, y, dy, dx */
} gla_conv_problem;

/* Bytes of device workspace gla_conv_bwd needs (gla_conv_fwd needs none). */
int gla_conv_workspace_size(const gla_conv_problem* p, size_t* bytes);

/* Forward: y = SiLU(causal depthwise convolution of x with w, plus bias). */
int gla_conv_fwd(const gla_conv_problem* p, const void* x, const float* w, const float* bias,
                 void* y, void* stream);

/* Backward: dx, dw (and db if non-NULL) from x, w, bias and dy; recomputes z. */
int gla_conv_bwd(const gla_conv_problem* p, const void* x, const float* w, const float* bias,
                 const void* dy, void* dx, float* dw, float* db, void* ws, size_t ws_bytes,
                 void* stream);

/* ---- Gated delta rule (Gated DeltaNet)
 *
 * The pages name the delta-rule layers (FLAT page, "FLAT: Flash Linear
 * Attention on TPUs", Conclusion, future work 1: DeltaNet, Gated DeltaNet and
 * Kimi Delta Attention, whose state update is not a plain sum of outer
 * products; probjax page, "GPU kernels", section Gated DeltaNet: a token-by-
 * token reference and a chunked WY/UT form whose backward keeps only
 * chunk-boundary states) without writing the update out.  The update computed
 * here is the published Gated DeltaNet one, in this library's orientation:
 *
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
 *
 * per batch row b and head h, with alpha_t = exp(g_t) (g: natural-log gate, one
 * per (b, t, h)) and beta_t the write strength (one per (b, t, h), any finite
 * value; usually in (0, 1)).  S_{-1} = h0, hT = S_{T-1}; segment_ids resets as
 * for gla_fwd.  There is no internal normalisation of q or k.  gla_delta_bwd
 * returns dq, dk, dv, dg (dL/dg, 0 at reset tokens), dbeta and dh0.
 *
 * Layouts (row-major, contiguous): q, k, dq, dk [B, T, H, d_k]; v, o, dO, dv
 * [B, T, H, d_v]; g, dg, beta, dbeta [B, T, H]; h0, hT, dhT, dh0 [B, H, d_k, d_v]
 * float32; segment_ids [B, T] int32.  dtype as for gla_fwd (all products and
 * sums in float32).  Sizes: B >= 1, T >= 0, H >= 1, d_k and d_v in {64, 128}.
 * Nullable: h0, segment_ids, hT, dhT, dh0 (as for gla_fwd / gla_bwd), and the
 * activation pointers when T == 0.  Ownership, ordering and errors are as for
 * gla_fwd / gla_bwd.
 *
 * Workspaces.  ws (both calls): gla_delta_workspace_size(p, 0) bytes, the
 * per-chunk factors the chunked form builds from the inputs (the inverse T, U,
 * W, the masked scores, gamma Q, the decayed keys and the chunk carries, fp32)
 * behind a small header; with GLA_DELTA_WS_FROM_FWD also the state entering
 * each chunk and its effective writes.  scratch (the backward only):
 * gla_delta_workspace_size(p, 1) bytes, the backward's own per-chunk
 * intermediates (the state gradients at the chunk boundaries, the gradient
 * blocks, and without the flag the states); nothing of it outlives the call.
 * Both sizes depend on the flag. */
typedef struct {
    int64_t B, T, H, d_k, d_v;
    int32_t dtype;    /* gla_dtype */
    int32_t flags;    /* 0, or GLA_DELTA_WS_FROM_FWD; other bits: GLA_E_UNSUPPORTED */
    int64_t generation; /* the caller's count of changes to the inputs' contents; see below */
} gla_delta_problem;

/* Given to both calls of a forward / backward pair that share ws: gla_delta_fwd
 * also stores in ws the state entering every chunk and the chunk's effective
 * writes, and gla_delta_bwd reuses them and the per-chunk factors instead of
 * recomputing them.  Every ws carries a stamp of what it holds: the problem's
 * sizes, dtype and flags, the q, k, v, g, beta and segment_ids pointers and
 * p->generation (gla_delta_fwd's last pass writes it; a backward that
 * recomputes rewrites it).  The backward's prepare and state passes compare the
 * stamp with their own call's on the device and recompute unless they are equal,
 * so a ws from another problem, other inputs, another layer or a forward without
 * the flag is never used.  The caller's part: give gla_delta_fwd and
 * gla_delta_bwd the same generation only while the inputs' contents are
 * unchanged (change it whenever they are written in place). */
#define GLA_DELTA_WS_FROM_FWD 1

/* Bytes of ws (for_backward == 0) or of the backward's scratch (for_backward != 0). */
int gla_delta_workspace_size(const gla_delta_problem* p, int for_backward, size_t* bytes);

/* Forward: o (and hT if non-NULL). */
int gla_delta_fwd(const gla_delta_problem* p, const void* q, const void* k, const void* v,
                  const void* g, const void* beta, const float* h0, const int32_t* segment_ids,
                  void* o, float* hT, void* ws, size_t ws_bytes, void* stream);

/* Backward: dq, dk, dv, dg, dbeta (and dh0 if non-NULL).  Recomputes the
 * per-chunk factors and the states entering the chunks unless p->flags has
 * GLA_DELTA_WS_FROM_FWD and ws's stamp matches (above). */
int gla_delta_bwd(const gla_delta_problem* p, const void* q, const void* k, const void* v,
                  const void* g, const void* beta, const float* h0, const int32_t* segment_ids,
                  const void* dO, const float* dhT, void* dq, void* dk, void* dv, void* dg,
                  void* dbeta, float* dh0, void* ws, size_t ws_bytes, void* scratch,
                  size_t scratch_bytes, void* stream);

/* ---- Output norm and gate (the step after the recurrence)
 *
 * FLAT page ("FLAT: Flash Linear Attention on TPUs"), section Full Linear
 * Attention Layer: the layer output is the per-head RMSNorm of the recurrence
 * output o multiplied by a swish output gate.  Per row (b, t, h) of d channels,
 * with the gate's pre-activation z and one scale vector gamma[d] for every head:
 *
 *     r = 1 / sqrt(mean_j o_j^2 + eps),   n = o * r,
 *     y = gamma * n * swish(z),           swish(z) = z * sigmoid(z).
 *
 * The backward takes dy = dL/dy and returns
 *     dz     = dy * gamma * n * swish'(z),    swish'(z) = s (1 + z (1 - s)), s = sigmoid(z),
 *     do     = r * (dn - n * mean_j(dn_j n_j)),  dn = dy * gamma * swish(z),
 *     dgamma = sum over all rows of dy * n * swish(z).
 *
 * Layouts (row-major, contiguous): o, z, y, dy, do, dz [B, T, H, d] in the
 * problem's dtype; gamma, dgamma [d] float32.  Sums run in float32; bf16 outputs
 * are rounded to nearest even.  Sizes: B >= 1, T >= 0, H >= 1, d in {64, 128},
 * eps finite and >= 0 (a row of zeros with eps = 0 gives NaN, as the formula
 * does).  Pointers are device pointers on the current HIP device, 16-byte
 * aligned; the activation pointers may be NULL when T == 0, the others are
 * required.  ws is a device workspace of at least gla_norm_gate_workspace_size()
 * bytes (per-block partial sums of dgamma, reduced in a fixed order: results are
 * the same on every run).  Ownership, ordering and errors are as for gla_fwd /
 * gla_bwd above. */
typedef struct {
    int64_t B, T, H, d;  /* batch rows, time steps, heads, channels per head */
    float eps;           /* added to the mean square */
    int32_t dtype;       /* gla_dtype of o, z, y, dy, do, dz */
} gla_norm_gate_problem;

/* Bytes of device workspace gla_norm_gate_bwd needs (the forward needs none). */
int gla_norm_gate_workspace_size(const gla_norm_gate_problem* p, size_t* bytes);

/* Forward: y = gamma * RMSNorm(o) * swish(z), per head. */
int gla_norm_gate_fwd(const gla_norm_gate_problem* p, const void* o, const void* z,
                      const float* gamma, void* y, void* stream);

/* Backward: d_o, dz and dgamma from o, z, gamma and dy; recomputes the norm. */
int gla_norm_gate_bwd(const gla_norm_gate_problem* p, const void* o, const void* z,
                      const float* gamma, const void* dy, void* d_o, void* dz, float* dgamma,
                      void* ws, size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* gla_status_str(int status);

/* ABI version: major * 10000 + minor * 100 + patch. */
int gla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GLA_H */
