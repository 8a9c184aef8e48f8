/*
 * llops.h -- C ABI of the MI355X (gfx950) LLoPS linear-attention library.
 *
 * LLoPS ("Learnable Low-Rank Polynomial Sketch for Effective Linear
 * Attention", arXiv 2610.14219) replaces the exact degree-p monomial map
 * psi_p(x) = vec(x^{(x)p}) by the CP-factorised sketch
 *     phi(X) = sum_{r=1..t} prod_{j=1..p} X Theta_{j,r},   Theta_{j,r} in R^{d x m}
 * (papernotes.org notes, key design 2: psi_p(Q) W_hat = sum_r prod_j Q Theta_{j,r}),
 * optionally squared element-wise after the r-sum for non-negative weights
 * (notes, training strategy; paper Sec. 3 non-negativity paragraph), and
 * uses it in linear attention phi_Q(Q) (phi_K(K)^T V) (notes, overall
 * framework; paper Sec. 1 associativity).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    allocates nothing, frees nothing and keeps no pointer after returning.
 *  - Tensors are dense row-major:
 *        X, Q, K       [batch][heads][n][d]
 *        V             [batch][heads][n][dv]
 *        phi           [batch][heads][n][m]
 *        out           [batch][heads][n][dv]
 *        Theta         [heads][p][t][d][m] if theta_per_head, else [p][t][d][m];
 *                      Theta[..][j][r][:, i] is column i of Theta_{j+1,r+1}
 *        S             [batch][heads][m][dv]   (fp32 always)
 *        z             [batch][heads][m]       (fp32 always)
 *  - in_dtype applies to X/Q/K/V/Theta; out_dtype to phi/out. Supported:
 *        in BF16 -> MFMA path (bf16 products, fp32 accumulation);
 *        in F32  -> fp32 path (fp32 products and accumulation).
 *        out F32 everywhere; out BF16 for llops_featmap only.
 *  - Normaliser (normalize = 1): out_i = num_i / (phi_Q(q_i) . z_i + delta),
 *    delta added once per row after the dot product (the +delta stabiliser of
 *    the SLAY notes, key design 3; Performer's numerator/denominator form in
 *    the low-rank-attention blog). normalize = 0 returns num_i.
 *  - Causal mask is inclusive: key j reaches query i iff j <= i.
 *  - Calls are asynchronous on `stream` and perform no host synchronisation.
 *    Validation happens before any launch; on an error nothing is launched and
 *    nothing is written. Device faults surface at the caller's next sync.
 *  - n = 0 (or batch*heads = 0) is a successful no-op (state outputs are still
 *    written as S0/z0, or zeros, by the causal entry point); pointers to
 *    tensors with no elements may then be null.
 *  - Thread safety: calls hold no shared mutable state; concurrent calls on
 *    different streams with disjoint buffers are safe. llops_last_error() is
 *    per thread.
 */
#ifndef LLOPS_H
#define LLOPS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LLOPS_F32 = 0, LLOPS_BF16 = 1 } llops_dtype_t;

typedef enum {
  LLOPS_OK = 0,
  LLOPS_ERR_INVALID_ARG = 1,  /* null pointer, bad size, bad enum, bad delta */
  LLOPS_ERR_UNSUPPORTED = 2,  /* valid request with no kernel for its shape */
  LLOPS_ERR_WORKSPACE = 3,    /* ws_bytes smaller than llops_workspace_bytes() */
  LLOPS_ERR_HIP = 4           /* a HIP launch or query failed */
} llops_status_t;

typedef enum {
  LLOPS_ENTRY_FEATMAP = 0,
  LLOPS_ENTRY_LINATTN = 1,
  LLOPS_ENTRY_CAUSAL = 2,
  LLOPS_ENTRY_DECODE = 3,
  LLOPS_ENTRY_FEATMAP_BWD = 4,
  LLOPS_ENTRY_CAUSAL_BWD = 5,
  LLOPS_ENTRY_LINATTN_BWD = 6,
  LLOPS_ENTRY_GATED_CAUSAL = 7,
  LLOPS_ENTRY_GATED_DECODE = 8,
  LLOPS_ENTRY_GATED_CAUSAL_BWD = 9
} llops_entry_t;

typedef struct llops_shape {
  int64_t batch, heads, n;  /* n: tokens per sequence (ignored by decode) */
  int32_t d, dv, m, p, t;   /* head dim, value dim, features, degree, CP rank */
  int32_t square;           /* 0|1: phi <- phi * phi after the sum over r    */
  int32_t normalize;        /* 0|1: divide by phi_Q . z + delta              */
  float delta;              /* >= 0 and finite when normalize = 1            */
  int32_t chunk;            /* causal block length hint: 0 (default), 16, 32,
                               64 or 128; changes rounding order, not math   */
  int32_t theta_per_head;   /* 1: Theta [heads][p][t][d][m]; 0: shared      */
  int32_t in_dtype;         /* llops_dtype_t                                 */
  int32_t out_dtype;        /* llops_dtype_t                                 */
} llops_shape_t;

/* Size limits checked by validation (else LLOPS_ERR_UNSUPPORTED):
 *   1 <= p <= 8, 1 <= t <= 64, 1 <= d <= 256, 1 <= dv <= 256, 1 <= m <= 1024;
 *   BF16 in additionally needs d % 16 == 0, m % 16 == 0, dv % 16 == 0 and
 *   p * d <= 1024; the causal/linattn BF16 path needs m <= 256, dv <= 128.
 */

/* Bytes of scratch `ws` the entry point needs for this shape (0 if none). */
size_t llops_workspace_bytes(const llops_shape_t* shape, int32_t entry);

/*
 * llops_featmap -- phi = sum_r prod_j X Theta_{j,r}  [squared if shape->square]
 * (notes, key design 2; paper Sec. 3: p*t projections, Hadamard product over
 * j, sum over r). X [batch][heads][n][d] (in_dtype), Theta per the layout
 * above (in_dtype), phi [batch][heads][n][m] (out_dtype). normalize, delta,
 * dv and chunk are ignored. ws: llops_workspace_bytes(shape,
 * LLOPS_ENTRY_FEATMAP) bytes of device scratch (a repacked copy of Theta for
 * the bf16 shapes that have an unrolled kernel and more than 1024 rows per
 * head; 0 bytes otherwise, and ws may then be null).
 * Why a workspace here, where the plain definition needs only X, Theta and
 * phi: the 256-row-tile kernels stream Theta through LDS one (32-feature
 * block, rank) stage at a time, and a stage is one contiguous p*d*64-byte
 * block only in a fragment-order copy of Theta, written by a separate launch
 * (15 us for both Theta sets at 1 x 32 heads x 65536 rows, d = 128, m = 256,
 * p = 2, t = 4: 0.7% of the feature map). The library allocates nothing, so
 * that copy lives in caller memory. Up to 1024 rows per head the few-row
 * kernels read Theta in place and need no workspace.
 */
llops_status_t llops_featmap(const llops_shape_t* shape, const void* X,
                             const void* theta, void* phi, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * llops_featmap_bwd -- gradients of L = sum(dphi * phi) for phi = llops_featmap(X, Theta):
 *   Y_{j,r} = X Theta_{j,r},  s = sum_r prod_j Y_{j,r},  ds = dphi * 2s (square) or dphi,
 *   dY_{j,r} = ds * prod_{j' != j} Y_{j',r},
 *   dX = sum_{j,r} dY_{j,r} Theta_{j,r}^T,  dTheta_{j,r} = X^T dY_{j,r}
 * (the chain rule through key design 2 of the notes; Theta is learned end to
 * end, notes' training strategy). X and Theta as for llops_featmap (in_dtype
 * BF16 only); dphi [batch][heads][n][m] in out_dtype (F32 or BF16); dX fp32
 * [batch][heads][n][d]; dtheta fp32 in Theta's layout, summed over heads when
 * Theta is shared. Both outputs are overwritten (n = 0 with heads > 0 writes
 * a zero dtheta). Kernels exist for p = 2, t in {1, 4}, d in {64, 128},
 * m % 32 == 0 (else LLOPS_ERR_UNSUPPORTED). Y is recomputed from X on MFMA
 * and dY rounded to bf16 before its two products; the head and row sums run
 * in a fixed order, so results are deterministic. ws:
 * llops_workspace_bytes(shape, LLOPS_ENTRY_FEATMAP_BWD) bytes (partial dTheta
 * sums per row chunk). normalize, delta, dv and chunk are ignored.
 */
llops_status_t llops_featmap_bwd(const llops_shape_t* shape, const void* X,
                                 const void* theta, const void* dphi, float* dX,
                                 float* dtheta, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * llops_linattn_fwd -- non-causal linear attention
 *   out = phi_Q(Q) (phi_K(K)^T V)  [ / (phi_Q(Q) (phi_K(K)^T 1) + delta) ]
 * (notes, overall framework; paper Sec. 1; blog, Performer section).
 * Q, K, V, theta_q, theta_k in in_dtype; out fp32 [batch][heads][n][dv].
 * theta_q may equal theta_k. ws: llops_workspace_bytes(shape, LLOPS_ENTRY_LINATTN).
 * fp32 inputs with (d, m, p, t) = (16, 32, 2, 2), n <= 1024 and dv in
 * {4, 8, ..., 20} run as one launch (one workgroup per sequence); other
 * shapes run the feature map and the segment passes through the workspace.
 */
llops_status_t llops_linattn_fwd(const llops_shape_t* shape, const void* Q,
                                 const void* K, const void* V,
                                 const void* theta_q, const void* theta_k,
                                 void* out, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * llops_linattn_causal_fwd -- causal linear attention over a prefix state
 *   out_i = (phi_Q(q_i) S_i) [ / (phi_Q(q_i) z_i + delta) ],
 *   S_i = S0 + sum_{j<=i} phi_K(k_j) v_j^T,  z_i = z0 + sum_{j<=i} phi_K(k_j)
 * (paper Sec. 1: streaming form with a constant-size state; blog: causal
 * masking by incremental cumulative sums). S0/z0 (fp32, nullable = zeros)
 * continue an earlier call; S_final/z_final (fp32, nullable) receive the state
 * after the last token, so prefill(n1) then prefill(n2, S0=S_final) equals
 * prefill(n1+n2). S0/z0 may alias S_final/z_final.
 * ws: llops_workspace_bytes(shape, LLOPS_ENTRY_CAUSAL).
 * Two execution paths compute bit for bit the same result on bf16 inputs:
 * by default the feature maps of Q and K go through the workspace (HBM) and
 * the segment passes read them back; with the environment variable
 * LLOPS_FUSED_Q=1 (read at each call), shapes (m, dv, d, p, t) in
 * {(256, 128, 128, 2, 4), (128, 64, 64, 3, 8)} with more than 1024 rows per
 * head project phi_Q inside the output pass instead, so phi_Q never reaches
 * HBM (the fused feature map -> causal pass; the notes' key design 2 and the
 * paper's runtime paragraph attribute the method's cost to these
 * projections and element-wise products).
 */
llops_status_t llops_linattn_causal_fwd(const llops_shape_t* shape, const void* Q,
                                        const void* K, const void* V,
                                        const void* theta_q, const void* theta_k,
                                        const float* S0, const float* z0,
                                        void* out, float* S_final, float* z_final,
                                        void* ws, size_t ws_bytes,
                                        hipStream_t stream);

/*
 * llops_linattn_gated_causal_fwd -- causal linear attention with a decaying state
 *   S_i = exp(g_i) S_{i-1} + phi_K(k_i) v_i^T,  z_i = exp(g_i) z_{i-1} + phi_K(k_i),
 *   S_{-1} = S0, z_{-1} = z0,  out_i = (phi_Q(q_i) S_i) [ / (phi_Q(q_i) z_i + delta) ],
 * i.e. key j reaches query i >= j with weight exp(g_{j+1} + ... + g_i) (the
 * decay-masked, semiseparable form). The LLoPS notes name data-driven
 * forgetting gates (Mamba2's semiseparable matrix) as the way forward in
 * "limitations and outlook" and say the feature map drops into gated state
 * rules unchanged ("highlights"); the gate here is one scalar per token and
 * head, applied to the whole state before the token is added, which with
 * g = 0 is exactly llops_linattn_causal_fwd.
 * log_gate: fp32 [batch][heads][n], g_i = log of the decay (device, 4-byte
 * aligned). Values <= 0 keep every factor in (0, 1]; positive values grow the
 * state and can overflow. Other arguments as for llops_linattn_causal_fwd;
 * S_final/z_final include the decay of every token. in_dtype F32 runs the
 * fp32 kernels (any shape within the general limits); in_dtype BF16 needs
 * (m, dv) in {(256, 128), (128, 64), (64, 64)} (else LLOPS_ERR_UNSUPPORTED).
 * Decay factors are computed in fp32 from chunk-local sums of g; on the
 * bf16 path the decay-weighted phi_Q and V are rounded to bf16 before their
 * products.
 * ws: llops_workspace_bytes(shape, LLOPS_ENTRY_GATED_CAUSAL).
 */
llops_status_t llops_linattn_gated_causal_fwd(const llops_shape_t* shape, const void* Q,
                                              const void* K, const void* V,
                                              const void* theta_q, const void* theta_k,
                                              const float* log_gate,
                                              const float* S0, const float* z0,
                                              void* out, float* S_final, float* z_final,
                                              void* ws, size_t ws_bytes,
                                              hipStream_t stream);

/*
 * llops_linattn_causal_bwd -- gradients of L = sum(dO * out) for
 * out = llops_linattn_causal_fwd(Q, K, V, theta_q, theta_k) started from a
 * zero state: dQ, dK [batch][heads][n][d], dV [batch][heads][n][dv] and
 * dtheta_q, dtheta_k in Theta's layout (summed over heads when shared), all
 * fp32 and overwritten. dO is fp32 [batch][heads][n][dv] (out_dtype F32).
 * With M = tril(phi_Q phi_K^T), num = M V and den = M 1 + delta:
 *   dnum = dO / den, dden = -sum_v(dO * out) / den   (normalize = 0: dnum = dO, dden = 0)
 *   dM = tril(dnum V^T + dden 1^T), dphi_Q = dM phi_K, dphi_K = dM^T phi_Q, dV = M^T dnum,
 * then llops_featmap_bwd on each side (paper Sec. 1 attention form; blog,
 * Performer section, and SLAY notes key design 3 for the normaliser; Theta is
 * learned end to end, notes' training strategy). The three sums are run as
 * causal linear attentions over bf16 features (dphi_K and dV as suffix sums,
 * anti-causal passes), so they carry the forward's bf16 rounding. Where phi
 * is too long for a 32-bit view, or with LLOPS_BWD_REVERSED=1 in the
 * environment (read at each call and by the workspace query), the suffix sums
 * run as causal passes over reversed copies instead (a larger workspace; the
 * same gradients up to summation order). At m = 256, dv = 128 the dphi passes
 * read [dnum | dden | 0] from a dv + 8 wide copy and [V | 1 | 0] from V
 * itself (this entry point, the _state one and both gated ones);
 * LLOPS_BWD_PADDED=1 in the environment (read at each call) selects 256-wide
 * padded copies instead, with bit for bit the same gradients.
 * in_dtype BF16 only; kernels exist for p = 2, t in {1, 4}, d in {64, 128},
 * m in {64, 128, 256}, dv % 16 == 0 and dv <= 128 (else LLOPS_ERR_UNSUPPORTED).
 * theta_q and theta_k may alias; their gradients are still returned apart.
 * chunk is ignored. ws: llops_workspace_bytes(shape, LLOPS_ENTRY_CAUSAL_BWD).
 */
llops_status_t llops_linattn_causal_bwd(const llops_shape_t* shape, const void* Q,
                                        const void* K, const void* V,
                                        const void* theta_q, const void* theta_k,
                                        const float* dO, float* dQ, float* dK, float* dV,
                                        float* dtheta_q, float* dtheta_k,
                                        void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * llops_linattn_causal_bwd_state -- llops_linattn_causal_bwd for the forward
 * continued from an initial state, out = llops_linattn_causal_fwd(..., S0, z0):
 *   num = M V + phi_Q S0,  den = M 1 + phi_Q z0 + delta,
 *   dphi_Q = dM phi_K + dnum S0^T + dden z0^T,  dS0 = phi_Q^T dnum,  dz0 = phi_Q^T dden
 * (the streaming form of the paper's Sec. 1: a chunk's initial state is the
 * running sums of the chunks before it, so dS0, dz0 carry the gradient back
 * to them). S0 [batch][heads][m][dv] and z0 [batch][heads][m] fp32 inputs
 * (nullable = zeros); dS0, dz0 fp32 outputs of those shapes (nullable = not
 * wanted), overwritten. The other arguments, limits and the workspace
 * (LLOPS_ENTRY_CAUSAL_BWD) are those of llops_linattn_causal_bwd, which is
 * this call with all four null.
 */
llops_status_t llops_linattn_causal_bwd_state(const llops_shape_t* shape, const void* Q,
                                              const void* K, const void* V,
                                              const void* theta_q, const void* theta_k,
                                              const float* S0, const float* z0,
                                              const float* dO, float* dQ, float* dK, float* dV,
                                              float* dtheta_q, float* dtheta_k,
                                              float* dS0, float* dz0,
                                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * llops_linattn_bwd -- the same gradients for the non-causal
 * out = llops_linattn_fwd(Q, K, V, theta_q, theta_k): M = phi_Q phi_K^T without
 * the mask, so each of dphi_Q = dM phi_K, dphi_K = dM^T phi_Q, dV = M^T dnum is
 * a non-causal linear attention (paper Sec. 1 associativity). Arguments,
 * layouts, kernels and limits as for llops_linattn_causal_bwd.
 * ws: llops_workspace_bytes(shape, LLOPS_ENTRY_LINATTN_BWD).
 */
llops_status_t llops_linattn_bwd(const llops_shape_t* shape, const void* Q, const void* K,
                                 const void* V, const void* theta_q, const void* theta_k,
                                 const float* dO, float* dQ, float* dK, float* dV,
                                 float* dtheta_q, float* dtheta_k,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * llops_decode_step -- one new token per (batch, head) on the recurrent state:
 *   S += phi_K(k) v^T;  z += phi_K(k);  out = phi_Q(q)^T S [ / (phi_Q(q)^T z + delta) ]
 * (paper Sec. 1: recurrent memory state; the update precedes the read, which
 * matches the inclusive causal mask). q, k [batch][heads][d], v
 * [batch][heads][dv] (in_dtype); S [batch][heads][m][dv] and z
 * [batch][heads][m] fp32, updated in place; out fp32 [batch][heads][dv].
 * shape->n is ignored. ws: llops_workspace_bytes(shape, LLOPS_ENTRY_DECODE)
 * bytes: phi_q and phi_k in fp32, plus repacked copies of Theta_q and Theta_k
 * when batch > 1024 on a bf16 shape with an unrolled feature-map kernel.
 */
llops_status_t llops_decode_step(const llops_shape_t* shape, const void* q,
                                 const void* k, const void* v,
                                 const void* theta_q, const void* theta_k,
                                 float* S, float* z, void* out,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * llops_linattn_gated_causal_bwd -- gradients of L = sum(dO * out) for
 * out = llops_linattn_gated_causal_fwd(Q, K, V, theta_q, theta_k, log_gate)
 * started from a zero state: dQ, dK, dV, dtheta_q, dtheta_k as for
 * llops_linattn_causal_bwd, and dlog_gate fp32 [batch][heads][n]. With
 * W_ij = exp(c_i - c_j) (j <= i), c = cumsum(log_gate), M = W * (phi_Q phi_K^T):
 *   dM = tril(dnum V^T + dden 1^T),  dphi_Q = (dM * W) phi_K,  dphi_K = (dM * W)^T phi_Q,
 *   dV = M^T dnum,  dlog_gate_l = sum_{i >= l} (phi_Q,i . dphi_Q,i - phi_K,i . dphi_K,i)
 * (the chain rule through the decay-masked form; the gate after the LLoPS
 * notes' limitations and outlook, the attention of the paper's Sec. 1, the
 * normaliser of the SLAY notes' key design 3). The three sums are gated
 * causal linear attentions over bf16 features (dphi_K and dV as suffix sums,
 * gated anti-causal passes), so they carry the forward's bf16 rounding; the gate gradient's row dots are taken on the
 * fp32 pass outputs. in_dtype BF16 only; kernels exist for p = 2, t in
 * {1, 4}, d in {64, 128} and (m, dv) in {(256, 128), (128, 64), (64, 64)}
 * (else LLOPS_ERR_UNSUPPORTED). All outputs are overwritten. chunk is
 * ignored. ws: llops_workspace_bytes(shape, LLOPS_ENTRY_GATED_CAUSAL_BWD).
 */
llops_status_t llops_linattn_gated_causal_bwd(const llops_shape_t* shape, const void* Q,
                                              const void* K, const void* V,
                                              const void* theta_q, const void* theta_k,
                                              const float* log_gate, const float* dO,
                                              float* dQ, float* dK, float* dV,
                                              float* dtheta_q, float* dtheta_k,
                                              float* dlog_gate, void* ws, size_t ws_bytes,
                                              hipStream_t stream);

/*
 * llops_linattn_gated_causal_bwd_state -- llops_linattn_gated_causal_bwd for the
 * forward continued from an initial state, out =
 * llops_linattn_gated_causal_fwd(..., log_gate, S0, z0), where the state reaches
 * query i with weight exp(c_i):
 *   dphi_Q_i += exp(c_i) (S0 dnum_i + dden_i z0),
 *   dS0 = sum_i exp(c_i) phi_Q,i dnum_i^T,  dz0 = sum_i exp(c_i) dden_i phi_Q,i,
 * and the gate gradient includes the state's term (same passages). S0, z0 fp32
 * inputs (nullable = zeros); dS0, dz0 fp32 outputs (nullable = not wanted),
 * overwritten. Other arguments, limits and the workspace
 * (LLOPS_ENTRY_GATED_CAUSAL_BWD) as for llops_linattn_gated_causal_bwd, which
 * is this call with all four null.
 */
llops_status_t llops_linattn_gated_causal_bwd_state(const llops_shape_t* shape, const void* Q,
                                                    const void* K, const void* V,
                                                    const void* theta_q, const void* theta_k,
                                                    const float* log_gate, const float* S0,
                                                    const float* z0, const float* dO,
                                                    float* dQ, float* dK, float* dV,
                                                    float* dtheta_q, float* dtheta_k,
                                                    float* dlog_gate, float* dS0, float* dz0,
                                                    void* ws, size_t ws_bytes,
                                                    hipStream_t stream);

/*
 * llops_gated_decode_step -- llops_decode_step on a decaying state:
 *   S = exp(g) S + phi_K(k) v^T;  z = exp(g) z + phi_K(k);
 *   out = phi_Q(q)^T S [ / (phi_Q(q)^T z + delta) ]
 * with one log gate g per (batch, head): log_gate fp32 [batch][heads]
 * (device, 4-byte aligned). The recurrent step of
 * llops_linattn_gated_causal_fwd (same source passages); g = 0 is
 * llops_decode_step. Other arguments, layouts and limits as for
 * llops_decode_step. ws: llops_workspace_bytes(shape, LLOPS_ENTRY_GATED_DECODE).
 */
llops_status_t llops_gated_decode_step(const llops_shape_t* shape, const void* q,
                                       const void* k, const void* v,
                                       const void* theta_q, const void* theta_k,
                                       const float* log_gate,
                                       float* S, float* z, void* out,
                                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * llops_decode_step_noalloc -- llops_decode_step with no workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It computes
 * exactly what llops_decode_step computes, with the same kernels. Its scratch
 * (phi_q, phi_k, and repacked Theta copies when batch > 1024 on a bf16
 * shape with an unrolled feature-map kernel) lives in a static device array
 * of 16 MiB inside the library, one per GPU, held until the process ends; a
 * shape whose scratch (llops_workspace_bytes(shape, LLOPS_ENTRY_DECODE))
 * exceeds 16 MiB returns LLOPS_ERR_UNSUPPORTED before any launch (batch *
 * heads * m <= 2^21 fits, e.g. 4096 sequences x heads at m = 256). The call
 * allocates nothing and needs nothing zeroed: every scratch byte it reads was
 * written earlier in the same call. The first call on a device looks the
 * array's address up (hipGetSymbolAddress, with the stream's device
 * current); later calls reuse it. All calls on one GPU share that GPU's
 * array: calls that overlap in time on one GPU (different streams, or host
 * threads without ordering) race on it and must be serialised by the
 * caller. Other arguments, layouts and errors as for llops_decode_step.
 */
llops_status_t llops_decode_step_noalloc(const llops_shape_t* shape, const void* q,
                                         const void* k, const void* v,
                                         const void* theta_q, const void* theta_k,
                                         float* S, float* z, void* out, hipStream_t stream);

/*
 * Diagnostics: kernel-level timing. While armed on the calling thread, each
 * kernel launch made by the library on behalf of that thread records
 * events[2*i] just before and events[2*i+1] just after it on the launch
 * stream, and stores the kernel's static name in names[i] (names may be
 * null), for the first `capacity` launches. The caller creates and owns the
 * 2*capacity events and reads them with hipEventElapsedTime after syncing.
 * llops_profile_disarm() stops recording and returns the launches recorded.
 * Arming adds two event records per launch and changes nothing else.
 */
llops_status_t llops_profile_arm(hipEvent_t* events, const char** names, int32_t capacity);
int32_t llops_profile_disarm(void);

/* Static description of a status code. */
const char* llops_status_str(llops_status_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* llops_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LLOPS_H */
