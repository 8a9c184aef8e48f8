// Host-side launchers of the LLoPS kernels (internal to libllops.so).
// Each returns hipSuccess or the launch error; shapes were validated by the
// C ABI layer before these are called.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace llops {

// Kernels with more than 64 KiB of dynamic LDS must say so before launch
// (a CU has 160 KiB on gfx950).
template <typename F>
inline hipError_t allow_lds(F* kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

// Kernel-level timing hook behind llops_profile_arm(): while armed on the
// calling thread, each launch is bracketed by two recorded events.
void prof_before(const char* name, hipStream_t st);
void prof_after(hipStream_t st);

#define LLOPS_LAUNCH(name, st, ...)       \
  do {                                    \
    ::llops::prof_before(name, st);       \
    hipLaunchKernelGGL(__VA_ARGS__);      \
    ::llops::prof_after(st);              \
  } while (0)

// One feature-map job: X [B][H][n][d] -> phi [B][H][n][m].
struct FeatJob {
  const void* X;
  const void* theta;  // [H][p][t][d][m] or [p][t][d][m]
  void* phi;
  void* theta_pk;     // featmap_pack_bytes() of scratch for the repacked Theta (or null)
};

struct FeatShape {
  int64_t B, H, n;
  int d, m, p, t;
  int theta_per_head;
  int square;
  int out_bf16;  // phi storage: 1 = bf16, 0 = fp32
};

// Scratch bytes per job for the fragment-order copy of Theta that the
// unrolled bf16 kernels read (0 when the shape takes the generic kernel).
size_t featmap_pack_bytes(const FeatShape& s);

// Fragment-order copy of one Theta set (the layout the 256-row-tile kernels
// read) into pk (featmap_pack_bytes() bytes); hipErrorInvalidValue when the
// shape has no unrolled kernel or takes the few-row path.
hipError_t launch_pack_theta(const FeatShape& s, const void* theta, void* pk, hipStream_t st);
// bf16 inputs on MFMA; runs `njobs` (1 or 2) jobs of the same shape in one launch.
hipError_t launch_featmap_bf16(const FeatShape& s, const FeatJob* jobs, int njobs,
                               hipStream_t st);
// fp32 inputs, fp32 arithmetic, fp32 phi.
hipError_t launch_featmap_f32(const FeatShape& s, const FeatJob* jobs, int njobs,
                              hipStream_t st);

// Feature-map backward (bf16 X and Theta): dX [B][H][n][d] and dtheta in
// Theta's layout (fp32; summed over heads for a shared Theta) from dphi
// [B][H][n][m] (bf16 when dphi_bf16, else fp32). dtheta is overwritten.
bool featmap_bwd_supported(const FeatShape& s);
// Scratch bytes for the per-chunk partial dTheta sums.
size_t featmap_bwd_ws_bytes(const FeatShape& s);
hipError_t launch_featmap_bwd(const FeatShape& s, const void* X, const void* theta,
                              const void* dphi, int dphi_bf16, float* dX, float* dtheta,
                              void* ws, hipStream_t st);

// Causal-attention backward helpers (attn_bwd.hip). Rows are [rows][width]
// blocks of per-(b, h) sequences of n rows; rev = 1 writes row i of each
// sequence to row n-1-i.
hipError_t launch_rows_copy_bf16(const uint16_t* src, int sw, int soff, uint16_t* dst, int dw,
                                 int doff, int width, int64_t n, int64_t rows, int rev,
                                 hipStream_t st);
hipError_t launch_rows_copy_f32(const float* src, int sw, int soff, float* dst, int dw, int doff,
                                int width, int64_t n, int64_t rows, int rev, hipStream_t st);
hipError_t launch_rows_copy_f32_bf16(const float* src, int sw, int soff, uint16_t* dst, int dw,
                                     int doff, int width, int64_t n, int64_t rows, int rev,
                                     hipStream_t st);
hipError_t launch_fill_ones16(uint16_t* dst, int64_t rows, hipStream_t st);
hipError_t launch_make_ab(const float* num, const float* den1, const float* G, const uint16_t* V,
                          int dv, int MA, int64_t n, int64_t rows, int normalize, float delta,
                          uint16_t* a, uint16_t* ra, uint16_t* b, uint16_t* rb, uint16_t* rdnum,
                          int rev, int den_ld, hipStream_t st);
// The same for the narrow operands of launch_attn_out32_aug: dnum to rdnum
// [rows][dv] and an = [dnum | dden | 0 x 7] [rows][dv + 8] (bf16, rows in
// order) in place of the padded a and b (b is v with a one at column dv).
hipError_t launch_make_ab_aug(const float* num, const float* den1, const float* G, int dv,
                              int64_t rows, int normalize, float delta, uint16_t* an,
                              uint16_t* rdnum, int den_ld, hipStream_t st);
// Backward from an initial state (S0 [BH][m][dv], z0 [BH][m]): z0 broadcast
// over `width` columns, the transposed [S0^T; z0^T] slice that starts a dphi_Q
// pass, and one column of per-(b, h) totals.
hipError_t launch_state_bcast(const float* z0, int64_t BH, int m, int width, float* out,
                              hipStream_t st);
// dS0, dz0 columns p0 .. p0+W-1 from segment 0 of a dphi_Q slice's start-anchored
// suffix states U [BH][nseg][per] (gated backward; either output may be null).
hipError_t launch_state_grad_slice(const float* U, int nseg, int64_t per, int64_t BH, int m, int dv,
                                   int W, int p0, float* dS0, float* dz0, hipStream_t st);
hipError_t launch_build_p0(const float* S0, const float* z0, int64_t BH, int m, int dv, int MA,
                           int W, int p0, float* out, hipStream_t st);
hipError_t launch_col_extract(const float* tot, int64_t BH, int m, int64_t per, int ld, float* out,
                              hipStream_t st);
// Gated backward helpers: reversed-sequence gates (shifted by one), bf16
// ones, row dots of an fp32 block against bf16 feature columns accumulated
// per row (optionally into the reversed row).
hipError_t launch_gate_reverse_shift(const float* g, int64_t n, int64_t rows, float* out,
                                     hipStream_t st);
hipError_t launch_fill_ones_bf16(uint16_t* dst, int64_t count, hipStream_t st);
hipError_t launch_rowdot_acc(const float* x, int xw, const uint16_t* phi, int pw, int poff,
                             int width, int64_t n, int64_t rows, int rev, float sign, int init,
                             float* acc, hipStream_t st, uint16_t* out = nullptr);
// (out: also stores the x rows as bf16, RNE, at phi's rows and columns)
// Exact gate gradient at segment starts: segment sums anchored at the start
// (launch_seg_state32_anchored), their reverse scan into suffix states, the inner products with the forward pass's prefix
// states, and the bridged per-segment suffix sums of the per-token terms.
hipError_t launch_seg_rscan_gated(int64_t BH, int nseg, int64_t per, int64_t mdv, float* seg,
                                  const float* gseg, hipStream_t st);
hipError_t launch_seg_dot(int64_t BH, int nseg, int64_t per, int64_t mdv, const float* P,
                          const float* U, int init, float* dgb, hipStream_t st);
hipError_t launch_seg_bridge_dg(const float* dc, int64_t BH, int64_t n, int64_t seg_len, int nseg,
                                const float* dgb, float* dg, hipStream_t st);

// Linear-attention contraction over precomputed features.
struct AttnShape {
  int64_t BH, n;
  int m, dv;
  int chunk;      // tokens per intra-chunk block
  int nseg;       // sequence segments per (b, h)
  int64_t seg_len;  // tokens per segment (multiple of chunk)
  int causal;
  int normalize;
  float delta;
  // anti-causal (with causal set): row i reads keys j >= i, i.e. suffix sums.
  // The segment states are then scanned from the last segment back, and the
  // output pass walks each segment's chunks from the last to the first.
  int anti = 0;
};

// Per-segment partial state: seg[bh][g][0 : m*dv] = phi_K^T V, [m*dv : +m] = phi_K^T 1.
hipError_t launch_seg_state_bf16(const AttnShape& a, const uint16_t* phik,
                                 const uint16_t* v, float* seg, hipStream_t st);
hipError_t launch_seg_state_f32(const AttnShape& a, const float* phik, const float* v,
                                float* seg, hipStream_t st);
// Exclusive scan of seg over g starting from (S0, z0) (null = zeros). Writes the
// total into (S_tot, z_tot) when non-null. For non-causal (exclusive = 0) the
// slots are left untouched and only the total is produced. a.anti: the scan
// runs from the last segment to the first (exclusive suffix sums).
hipError_t launch_seg_scan(const AttnShape& a, float* seg, const float* S0,
                           const float* z0, float* S_tot, float* z_tot, int exclusive,
                           hipStream_t st);
// Output pass. Causal: segment g starts from seg[bh][g]. Non-causal: every
// segment reads the total state `tot` [bh][m*dv + m] (contiguous S then z).
hipError_t launch_attn_out_bf16(const AttnShape& a, const uint16_t* phiq,
                                const uint16_t* phik, const uint16_t* v,
                                const float* state, int64_t state_seg_stride,
                                int64_t state_bh_stride, float* out, hipStream_t st);
hipError_t launch_attn_out_f32(const AttnShape& a, const float* phiq, const float* phik,
                               const float* v, float* state, int64_t state_seg_stride,
                               int64_t state_bh_stride, float* out, hipStream_t st);

// 32x32x16-MFMA segment passes for (m, dv) in {(256, 128), (128, 64), (64, 64)}
// (same seg / state layouts as the kernels above).
bool attn32_supported(const AttnShape& a);
hipError_t launch_seg_state32(const AttnShape& a, const uint16_t* phik, const uint16_t* v,
                              float* seg, hipStream_t st);
hipError_t launch_attn_out32(const AttnShape& a, const uint16_t* phiq, const uint16_t* phik,
                             const uint16_t* v, const float* state, int64_t state_seg_stride,
                             int64_t state_bh_stride, float* out, hipStream_t st);
// The causal output pass with phi_Q projected inside it (phi_Q never leaves
// the chip): X_Q [BH][n][d] bf16 and Theta_Q in fragment order (pack_theta's
// layout, heads pk_hstride elements apart, 0 = shared) replace phi_Q. Shapes:
// (m, dv, d, p, t) in {(256, 128, 128, 2, 4), (128, 64, 64, 3, 8)}.
bool attn32_fq_supported(const AttnShape& a, int d, int p, int t);
hipError_t launch_attn_out32_fq(const AttnShape& a, int d, int p, int t, const uint16_t* xq,
                                const uint16_t* thpk, int64_t pk_hstride, int64_t H, int square,
                                const uint16_t* phik, const uint16_t* v, const float* state,
                                int64_t state_seg_stride, int64_t state_bh_stride, float* out,
                                hipStream_t st);
// The same pass writing its rows elsewhere: to outb (bf16, RNE; rows ldo
// elements apart, e.g. a column slice of a wider row) when outb is set, else
// to out; rev = 1 (causal only): row t of the pass goes to row n - 1 - t.
hipError_t launch_attn_out32_to(const AttnShape& a, const uint16_t* phiq, const uint16_t* phik,
                                const uint16_t* v, const float* state, int64_t state_seg_stride,
                                int64_t state_bh_stride, float* out, uint16_t* outb, int ldo,
                                int rev, hipStream_t st, int vld = 0);
// vld != 0 (the backward's bf16 passes): value rows vld elements apart, v at
// the slice's first column; launch_seg_state32_v is the matching state pass.
hipError_t launch_seg_state32_v(const AttnShape& a, const uint16_t* phik, const uint16_t* v,
                                int vld, float* seg, hipStream_t st);
// The backward's chain-rule passes on narrow operands (m = 256, dv = 128
// kernels only): each feature row of phi_Q (phi_K) is stored as qald (kald)
// bf16 (row stride the same, a multiple of 8; qald + qone <= 160) and read
// as 256: those values, a bf16 one at column qald (kald) if qone (kone), then
// zeros (features past 160 take no products). So the passes
// read [dnum | dden | 0] (stored [dnum | dden | 0 x 7]) and [v | 1 | 0] (v
// itself) without padded copies. Values are a column slice (vld, as
// launch_seg_state32_v); rows go to outb (bf16, ldo apart). a.anti selects
// the suffix form.
bool aug32_supported(const AttnShape& a);
hipError_t launch_seg_state32_aug(const AttnShape& a, const uint16_t* phik, int kald, int kone,
                                  const uint16_t* v, int vld, float* seg, hipStream_t st);
hipError_t launch_attn_out32_aug(const AttnShape& a, const uint16_t* phiq, int qald, int qone,
                                 const uint16_t* phik, int kald, int kone, const uint16_t* v,
                                 int vld, const float* state, int64_t state_seg_stride,
                                 int64_t state_bh_stride, uint16_t* outb, int ldo, hipStream_t st);
// The gated backward's passes on narrow operands: the decayed (or, anchored,
// start-anchored) state pass, and the causal or (a.anti) suffix output pass
// writing fp32 rows to out [rows][128].
hipError_t launch_seg_state32_gated_aug(const AttnShape& a, const uint16_t* phik, int kald, int kone,
                                        const uint16_t* v, int vld, const float* gl, float* gseg,
                                        float* seg, bool anchored, hipStream_t st);
hipError_t launch_attn_out32_gated_aug(const AttnShape& a, const uint16_t* phiq, int qald, int qone,
                                       const uint16_t* phik, int kald, int kone,
                                       const uint16_t* v, int vld, const float* gl,
                                       const float* state, float* out, hipStream_t st);
// The same pass with a.normalize set, writing the unnormalised rows to out
// and each row's denominator phi_Q,i . z_i (no delta) to den [BH][n].
hipError_t launch_attn_out32_den(const AttnShape& a, const uint16_t* phiq, const uint16_t* phik,
                                 const uint16_t* v, const float* state, int64_t state_seg_stride,
                                 int64_t state_bh_stride, float* out, float* den, hipStream_t st);

// Gated causal passes (per-token log gates g [BH][n], decay exp(g)), on the
// 32x32x16 kernels' shapes. gate_cumsum32 writes L = the inclusive sum of g
// inside each 32-token chunk; pass 1 writes the per-segment sums of g to
// gseg [BH][nseg] next to the decayed segment states; launch_seg_scan with
// gseg carries the prefix through each segment's decay; pass 2 reads seg.
hipError_t launch_gate_cumsum32(int64_t BH, int64_t n, const float* g, float* L, hipStream_t st);
hipError_t launch_seg_state32_gated(const AttnShape& a, const uint16_t* phik, const uint16_t* v,
                                    const float* gl, float* gseg, float* seg, hipStream_t st);
hipError_t launch_attn_out32_gated(const AttnShape& a, const uint16_t* phiq, const uint16_t* phik,
                                   const uint16_t* v, const float* gl, const float* state,
                                   float* out, hipStream_t st);
// Gated backward passes: value rows vld apart (vld != 0; anchored: the
// start-anchored state pass), or (output) rows written in reversed order.
hipError_t launch_seg_state32_gated_v(const AttnShape& a, const uint16_t* phik, const uint16_t* v,
                                      int vld, const float* gl, float* gseg, float* seg,
                                      bool anchored, hipStream_t st);
hipError_t launch_attn_out32_gated_to(const AttnShape& a, const uint16_t* phiq,
                                      const uint16_t* phik, const uint16_t* v, const float* gl,
                                      const float* state, float* out, int rev, int vld,
                                      hipStream_t st);
hipError_t launch_attn_out32_gated_den(const AttnShape& a, const uint16_t* phiq,
                                       const uint16_t* phik, const uint16_t* v, const float* gl,
                                       const float* state, float* out, float* den,
                                       hipStream_t st);
// fp32 gated passes over the raw log gates g [BH][n] (any chunk, m, dv).
// Non-causal fp32 attention of small sequences in one launch (one workgroup
// per (b, h)): Q, K [B][H][n][d], V and out [B][H][n][dv], Theta [H'][p][t][d][m]
// (th_hstride elements apart, 0 = shared). ok() says whether the shape takes it.
bool linattn_small_f32_ok(int64_t BH, int64_t n, int d, int dv, int m, int p, int t);
hipError_t launch_linattn_small_f32(int64_t B, int64_t H, int64_t n, int d, int dv, int m, int p,
                                    int t, const float* Q, const float* K, const float* V,
                                    const float* tq, const float* tk, int64_t th_hstride,
                                    int square, int normalize, float delta, float* out,
                                    hipStream_t st);
hipError_t launch_seg_state_f32_gated(const AttnShape& a, const float* phik, const float* v,
                                      const float* log_gate, float* gseg, float* seg,
                                      hipStream_t st);
hipError_t launch_attn_out_f32_gated(const AttnShape& a, const float* phiq, const float* phik,
                                     const float* v, const float* log_gate, float* state,
                                     float* out, hipStream_t st);
// Segment sums anchored at the segment start, sum_k exp(c_k - c_{t0-1}) phik_k v_k^T
// (gate gradient of the backward; same seg layout).
hipError_t launch_seg_state32_anchored(const AttnShape& a, const uint16_t* phik,
                                      const uint16_t* v, const float* gl, float* gseg, float* seg,
                                      hipStream_t st);
// Causal scan with per-segment decays: prefix_{g+1} = exp(gseg[g]) prefix_g + seg[g].
hipError_t launch_seg_scan_gated(const AttnShape& a, float* seg, const float* gseg,
                                 const float* S0, const float* z0, float* S_tot, float* z_tot,
                                 hipStream_t st);

// Decode: per (b, h): S = a S + phik v^T; z = a z + phik; out = phiq^T S [/(phiq^T z + delta)]
// with a = exp(log_gate[b, h]), or a = 1 when log_gate is null.
hipError_t launch_decode_state(int64_t BH, int m, int dv, const float* phiq,
                               const float* phik, const void* v, int v_bf16, float* S,
                               float* z, float* out, int normalize, float delta,
                               const float* log_gate, hipStream_t st);

// Copies (S0, z0) or zeros into (S, z): used when n = 0.
hipError_t launch_state_init(int64_t BH, int m, int dv, const float* S0, const float* z0,
                             float* S, float* z, hipStream_t st);

}  // namespace llops
