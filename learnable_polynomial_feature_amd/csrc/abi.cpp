// C ABI of libllops: argument validation, workspace layout and kernel dispatch.
// No allocation, no host synchronisation; every check runs before the first launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kernels.h"
#include "llops.h"

namespace {

thread_local char g_err[512] = "";

llops_status_t fail(llops_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

llops_status_t hip_fail(hipError_t e, const char* what) {
  return fail(LLOPS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Sequence segmentation shared by the workspace size query and the launches.
struct SegPlan {
  int chunk;
  int nseg;
  int64_t seg_len;
};

// target: workgroups per pass to aim for (0 = the default for the dtype).
SegPlan seg_plan(const llops_shape_t* s, bool causal, int64_t target_wg = 0) {
  SegPlan p{};
  const bool bf16 = s->in_dtype == LLOPS_BF16;
  if (bf16) {
    // bf16 MFMA blocks are 32 or 64 tokens (a 128-token block with m = 256
    // does not fit the 160 KiB LDS of a CU); the chunk only orders rounding.
    p.chunk = (causal && s->chunk > 0 && s->chunk <= 32) ? 32 : 64;
  } else {
    p.chunk = s->chunk > 0 ? s->chunk : 64;
  }
  const int64_t BH = s->batch * s->heads;
  const int64_t n = s->n;
  const int64_t target = target_wg > 0 ? target_wg : bf16 ? 512 : 256;  // workgroups to aim for
  int64_t nchunks = (n + p.chunk - 1) / p.chunk;
  if (nchunks < 1) nchunks = 1;
  int64_t want = BH > 0 ? (target + BH - 1) / BH : 1;
  if (want < 1) want = 1;
  int64_t nseg = want < nchunks ? want : nchunks;
  int64_t chunks_per_seg = (nchunks + nseg - 1) / nseg;
  p.seg_len = chunks_per_seg * p.chunk;
  p.nseg = static_cast<int>((nchunks + chunks_per_seg - 1) / chunks_per_seg);
  return p;
}

struct WsLayout {
  size_t phiq, phik, seg, tot, pkq, pkk, gl, gseg, total;
};

// ---- causal backward: workspace plan ---------------------------------------
// Causal attention over given bf16 features (no feature map, no normaliser)
// is the building block of the backward; its shape as an llops_shape_t.
llops_shape_t feat_attn_shape(const llops_shape_t* s, int M, int DV) {
  llops_shape_t t = *s;
  t.m = M;
  t.dv = DV;
  t.normalize = 0;
  t.delta = 0.f;
  t.chunk = 0;
  t.in_dtype = LLOPS_BF16;
  t.out_dtype = LLOPS_F32;
  return t;
}

// The gated backward splits its passes into 4x the default segments: its gate
// gradient is exact at segment starts and a running sum of per-token terms
// in between, whose rounding grows with the segment length.
constexpr int64_t kGatedBwdWG = 2048;

size_t feat_attn_seg_bytes(const llops_shape_t* s, int M, int DV, bool causal,
                           int64_t target_wg = 0) {
  const llops_shape_t t = feat_attn_shape(s, M, DV);
  const SegPlan sp = seg_plan(&t, causal, target_wg);
  return static_cast<size_t>(s->batch * s->heads) * sp.nseg *
         (static_cast<size_t>(M) * DV + M) * sizeof(float);
}

// a = [dnum | dden | 0] and b = [V | 1 | 0] are MA wide and the phi values
// are contracted in pieces of W columns, with (MA, W) one of the shapes the
// 32x32x16 segment kernels take: (256, 128), (128, 64), (64, 64).
int bwd_ma(const llops_shape_t* s) { return s->dv + 1 <= 64 ? 64 : s->dv + 1 <= 128 ? 128 : 256; }
int bwd_w(const llops_shape_t* s) {
  const int w = bwd_ma(s) == 256 ? 128 : 64;
  return s->m < w ? s->m : w;
}

struct BwdWs {
  size_t phq, phk, pkq, pkk, num, den1, ones, a, ra, b, rb, rdnum, rphq, rphk, vp, tmp, dphq, dphk,
      seg, tot, fb, stot, p0, zb16, total;
};

llops::FeatShape feat_shape(const llops_shape_t* s, int64_t n, int out_bf16);

// Scratch for the fragment-order copy of one Theta set (bf16 shapes with an
// unrolled feature-map kernel only).
size_t pack_bytes(const llops_shape_t* s, int64_t n) {
  if (s->in_dtype != LLOPS_BF16) return 0;
  return llops::featmap_pack_bytes(feat_shape(s, n, 1));
}

WsLayout ws_layout(const llops_shape_t* s, int entry) {
  WsLayout w{};
  const bool gated = entry == LLOPS_ENTRY_GATED_CAUSAL;
  if (gated) entry = LLOPS_ENTRY_CAUSAL;
  if (entry == LLOPS_ENTRY_GATED_DECODE) entry = LLOPS_ENTRY_DECODE;
  const size_t esz = s->in_dtype == LLOPS_BF16 ? 2 : 4;
  const size_t BH = static_cast<size_t>(s->batch * s->heads);
  const size_t per = static_cast<size_t>(s->m) * s->dv + s->m;
  size_t off = 0;
  if (entry == LLOPS_ENTRY_FEATMAP) {
    w.pkq = off;
    off = round_up(off + pack_bytes(s, s->n), 256);
  } else if (entry == LLOPS_ENTRY_FEATMAP_BWD) {
    w.seg = off;
    if (s->in_dtype == LLOPS_BF16)
      off = round_up(off + llops::featmap_bwd_ws_bytes(feat_shape(s, s->n, 0)), 256);
  } else if (entry == LLOPS_ENTRY_LINATTN || entry == LLOPS_ENTRY_CAUSAL) {
    const SegPlan sp = seg_plan(s, entry == LLOPS_ENTRY_CAUSAL);
    const size_t phib = BH * static_cast<size_t>(s->n) * s->m * esz;
    w.phiq = off;
    off = round_up(off + phib, 256);
    w.phik = off;
    off = round_up(off + phib, 256);
    w.seg = off;
    off = round_up(off + BH * sp.nseg * per * sizeof(float), 256);
    w.tot = off;
    if (entry == LLOPS_ENTRY_LINATTN) off = round_up(off + BH * per * sizeof(float), 256);
    const size_t pkb = pack_bytes(s, s->n);
    w.pkq = off;
    off = round_up(off + pkb, 256);
    w.pkk = off;
    off = round_up(off + pkb, 256);
    if (gated) {  // chunk-local gate sums [BH][n rounded up to 32], segment gate sums [BH][nseg]
      w.gl = off;
      off = round_up(off + BH * static_cast<size_t>((s->n + 31) / 32 * 32) * sizeof(float), 256);
      w.gseg = off;
      off = round_up(off + BH * sp.nseg * sizeof(float), 256);
    }
  } else if (entry == LLOPS_ENTRY_DECODE) {
    const size_t phib = BH * s->m * sizeof(float);
    w.phiq = off;
    off = round_up(off + phib, 256);
    w.phik = off;
    off = round_up(off + phib, 256);
    const size_t pkb = pack_bytes(s, 1);
    w.pkq = off;
    off = round_up(off + pkb, 256);
    w.pkk = off;
    off = round_up(off + pkb, 256);
  }
  w.total = off;
  return w;
}

// The non-causal backward needs no reversed copies; it keeps the segment
// totals instead.
bool num_den_one_pass(const llops_shape_t* s, bool causal);

bool on32(const llops_shape_t* s, bool causal, int M, int DV);

// The causal backwards' suffix sums (dphi_K and dV: key i >= query j) run as
// anti-causal output passes on the 32x32x16 kernels when their in-place forms
// apply (phi read in place, rows written in place); otherwise as causal
// passes over reversed copies of their operands (and, gated, reversed gates).
// LLOPS_BWD_REVERSED=1 in the environment (read at each call, by the workspace
// query too) selects the reversed form wherever the anti-causal one applies.
bool bwd_anti(const llops_shape_t* s) {
  const char* env = getenv("LLOPS_BWD_REVERSED");
  if (env && env[0] == '1') return false;
  return on32(s, true, bwd_ma(s), bwd_w(s)) && on32(s, true, s->m, s->dv) &&
         s->n * s->m * 2 < (int64_t{1} << 31);
}

BwdWs bwd_ws(const llops_shape_t* s, bool causal) {
  BwdWs w{};
  const size_t R = static_cast<size_t>(s->batch * s->heads) * static_cast<size_t>(s->n);
  const size_t m = s->m, dv = s->dv, MA = bwd_ma(s), W = bwd_w(s);
  const bool rev = causal && !bwd_anti(s);  // reversed copies needed
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  w.phq = take(R * m * 2);
  w.phk = take(R * m * 2);
  w.pkq = take(pack_bytes(s, s->n));
  w.pkk = take(pack_bytes(s, s->n));
  // den1: M 1 per row; on the 32x32x16 shapes the num pass writes it, else a
  // pass over all-ones values 16 wide ([R][16], column 0 read)
  const bool one = num_den_one_pass(s, causal);
  w.num = take(R * dv * 4);
  w.den1 = take(s->normalize ? R * (one ? 1 : 16) * 4 : 0);
  w.ones = take(s->normalize && !one ? R * 16 * 2 : 0);
  w.a = take(R * MA * 2);
  w.ra = take(rev ? R * MA * 2 : 0);
  w.b = take(R * MA * 2);
  w.rb = take(rev ? R * MA * 2 : 0);
  w.rdnum = take(R * dv * 2);
  w.rphq = take(rev ? R * m * 2 : 0);
  w.rphk = take(rev ? R * m * 2 : 0);
  w.vp = take(R * W * 2);
  w.tmp = take(R * (W > dv ? W : dv) * 4);
  w.dphq = take(R * m * 2);
  w.dphk = take(R * m * 2);
  size_t seg = feat_attn_seg_bytes(s, s->m, s->dv, causal);
  const size_t seg2 = feat_attn_seg_bytes(s, static_cast<int>(MA), static_cast<int>(W), causal);
  const size_t seg3 = one ? 0 : feat_attn_seg_bytes(s, s->m, 16, causal);
  if (seg2 > seg) seg = seg2;
  if (seg3 > seg) seg = seg3;
  w.seg = take(seg);
  // per (b, h) totals of the non-causal passes (largest of the shapes above)
  const size_t BH = static_cast<size_t>(s->batch * s->heads);
  size_t per = m * dv + m;
  if (MA * W + MA > per) per = MA * W + MA;
  w.tot = take(causal ? 0 : BH * per * sizeof(float));
  w.fb = take(llops::featmap_bwd_ws_bytes(feat_shape(s, s->n, 0)));
  // causal, from an initial state: totals for dS0 / dz0, the initial state of
  // a dphi_Q slice pass, and z0 broadcast for a separate M 1 pass
  w.stot = take(causal ? BH * (m * dv + m) * sizeof(float) : 0);
  w.p0 = take(causal ? BH * MA * W * sizeof(float) : 0);
  w.zb16 = take(causal && !one ? BH * m * 16 * sizeof(float) : 0);
  w.total = off;
  return w;
}

bool is01(int32_t x) { return x == 0 || x == 1; }

llops_status_t validate(const llops_shape_t* s, int entry) {
  if (!s) return fail(LLOPS_ERR_INVALID_ARG, "shape is null");
  if (entry == LLOPS_ENTRY_GATED_CAUSAL) entry = LLOPS_ENTRY_CAUSAL;
  if (entry == LLOPS_ENTRY_GATED_DECODE) entry = LLOPS_ENTRY_DECODE;
  // the backward takes the feature map's shape rules
  if (entry == LLOPS_ENTRY_FEATMAP_BWD) entry = LLOPS_ENTRY_FEATMAP;
  if (s->batch < 0 || s->heads < 0) return fail(LLOPS_ERR_INVALID_ARG, "batch/heads < 0");
  if (entry != LLOPS_ENTRY_DECODE && s->n < 0) return fail(LLOPS_ERR_INVALID_ARG, "n < 0");
  if (s->d < 1 || s->m < 1 || s->p < 1 || s->t < 1)
    return fail(LLOPS_ERR_INVALID_ARG, "d, m, p, t must be >= 1 (d=%d m=%d p=%d t=%d)", s->d,
                s->m, s->p, s->t);
  if (entry != LLOPS_ENTRY_FEATMAP && s->dv < 1)
    return fail(LLOPS_ERR_INVALID_ARG, "dv must be >= 1");
  if (!is01(s->in_dtype) || !is01(s->out_dtype))
    return fail(LLOPS_ERR_INVALID_ARG, "bad dtype enum (in=%d out=%d)", s->in_dtype, s->out_dtype);
  if (!is01(s->square) || !is01(s->normalize) || !is01(s->theta_per_head))
    return fail(LLOPS_ERR_INVALID_ARG, "square/normalize/theta_per_head must be 0 or 1");
  if (entry != LLOPS_ENTRY_FEATMAP && s->normalize && (!isfinite(s->delta) || s->delta < 0.f))
    return fail(LLOPS_ERR_INVALID_ARG, "delta must be finite and >= 0");
  if (!(s->chunk == 0 || s->chunk == 16 || s->chunk == 32 || s->chunk == 64 || s->chunk == 128))
    return fail(LLOPS_ERR_INVALID_ARG, "chunk must be 0, 16, 32, 64 or 128 (got %d)", s->chunk);
  if (s->p > 8 || s->t > 64 || s->d > 256 || s->m > 1024 ||
      (entry != LLOPS_ENTRY_FEATMAP && s->dv > 256))
    return fail(LLOPS_ERR_UNSUPPORTED, "size limits: p<=8, t<=64, d<=256, dv<=256, m<=1024");
  if (s->heads > 65535) return fail(LLOPS_ERR_UNSUPPORTED, "heads > 65535");
  if ((entry == LLOPS_ENTRY_LINATTN || entry == LLOPS_ENTRY_CAUSAL) && s->batch * s->heads > 65535)
    return fail(LLOPS_ERR_UNSUPPORTED, "batch * heads > 65535");
  // the feature map addresses the rows of one workgroup by 32-bit offsets
  if (entry != LLOPS_ENTRY_DECODE && s->batch > 1 && s->heads * s->n >= (int64_t(1) << 30))
    return fail(LLOPS_ERR_UNSUPPORTED, "batch > 1 with heads * n >= 2^30");
  if (entry != LLOPS_ENTRY_FEATMAP && s->out_dtype != LLOPS_F32)
    return fail(LLOPS_ERR_UNSUPPORTED, "attention outputs are fp32 only");
  if (s->in_dtype == LLOPS_BF16) {
    if (s->d % 16 || s->m % 16 || s->p * s->d > 1024)
      return fail(LLOPS_ERR_UNSUPPORTED, "bf16 needs d %% 16 == 0, m %% 16 == 0, p*d <= 1024");
    if (entry == LLOPS_ENTRY_LINATTN || entry == LLOPS_ENTRY_CAUSAL) {
      if (s->m % 32 || s->m > 256 || s->dv % 16 || s->dv > 128)
        return fail(LLOPS_ERR_UNSUPPORTED,
                    "bf16 attention needs m %% 32 == 0, m <= 256, dv %% 16 == 0, dv <= 128");
    }
    if (entry == LLOPS_ENTRY_DECODE && s->dv % 4)
      return fail(LLOPS_ERR_UNSUPPORTED, "bf16 decode needs dv %% 4 == 0");
  }
  return LLOPS_OK;
}

llops_status_t need(const void* p, const char* name) {
  if (!p) return fail(LLOPS_ERR_INVALID_ARG, "%s is null", name);
  if (!aligned16(p)) return fail(LLOPS_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return LLOPS_OK;
}

llops_status_t need4(const void* p, const char* name) {
  if (!p) return fail(LLOPS_ERR_INVALID_ARG, "%s is null", name);
  if (reinterpret_cast<uintptr_t>(p) & 3u)
    return fail(LLOPS_ERR_INVALID_ARG, "%s is not 4-byte aligned", name);
  return LLOPS_OK;
}

llops_status_t opt(const void* p, const char* name) {
  if (p && !aligned16(p)) return fail(LLOPS_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return LLOPS_OK;
}

#define LLOPS_TRY(expr)                        \
  do {                                         \
    const llops_status_t _st = (expr);         \
    if (_st != LLOPS_OK) return _st;           \
  } while (0)

#define LLOPS_HIP(expr, what)                  \
  do {                                         \
    const hipError_t _e = (expr);              \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

llops::FeatShape feat_shape(const llops_shape_t* s, int64_t n, int out_bf16) {
  llops::FeatShape f{};
  f.B = s->batch;
  f.H = s->heads;
  f.n = n;
  f.d = s->d;
  f.m = s->m;
  f.p = s->p;
  f.t = s->t;
  f.theta_per_head = s->theta_per_head;
  f.square = s->square;
  f.out_bf16 = out_bf16;
  return f;
}

llops::AttnShape attn_shape(const llops_shape_t* s, bool causal, int64_t target_wg = 0) {
  const SegPlan sp = seg_plan(s, causal, target_wg);
  llops::AttnShape a{};
  a.BH = s->batch * s->heads;
  a.n = s->n;
  a.m = s->m;
  a.dv = s->dv;
  a.chunk = sp.chunk;
  a.nseg = sp.nseg;
  a.seg_len = sp.seg_len;
  a.causal = causal ? 1 : 0;
  a.normalize = s->normalize;
  a.delta = s->normalize ? s->delta : 0.f;
  return a;
}

llops_status_t validate_attn_bwd(const llops_shape_t* s, bool causal) {
  LLOPS_TRY(validate(s, causal ? LLOPS_ENTRY_CAUSAL : LLOPS_ENTRY_LINATTN));
  if (s->in_dtype != LLOPS_BF16)
    return fail(LLOPS_ERR_UNSUPPORTED, "attention backward takes bf16 Q, K, V and Theta only");
  if (!llops::featmap_bwd_supported(feat_shape(s, s->n, 0)) ||
      !(s->m == 64 || s->m == 128 || s->m == 256))
    return fail(LLOPS_ERR_UNSUPPORTED,
                "attention backward kernels: p = 2, t in {1, 4}, d in {64, 128}, m in {64, 128, 256} "
                "(got p=%d t=%d d=%d m=%d)", s->p, s->t, s->d, s->m);
  return LLOPS_OK;
}

// The gated causal form: fp32 inputs on the fp32 kernels (any shape), bf16
// inputs on the 32x32x16 segment kernels only.
llops_status_t validate_gated(const llops_shape_t* s) {
  LLOPS_TRY(validate(s, LLOPS_ENTRY_GATED_CAUSAL));
  if (s->in_dtype != LLOPS_BF16) return LLOPS_OK;
  const llops::AttnShape a = attn_shape(s, true);
  if (s->batch * s->heads > 0 && !llops::attn32_supported(a))
    return fail(LLOPS_ERR_UNSUPPORTED,
                "gated causal attention kernels: (m, dv) in {(256, 128), (128, 64), (64, 64)} "
                "(got m=%d dv=%d)", s->m, s->dv);
  return LLOPS_OK;
}

// out_i = sum_{j<=i} (fq_i . fk_j) v_j (causal) or sum over all j (tot holds
// the per-(b, h) totals then) over bf16 features fq, fk [BH][n][M] and values
// v [BH][n][DV]; fp32 out. The forward's segment kernels.
// outb (bf16, rows ldo apart) and rev (rows written in reversed order): the
// 32x32x16 kernels only (on32).
bool on32(const llops_shape_t* s, bool causal, int M, int DV) {
  const llops_shape_t t = feat_attn_shape(s, M, DV);
  return llops::attn32_supported(attn_shape(&t, causal));
}

hipError_t attn_on_features(const llops_shape_t* s, bool causal, int M, int DV,
                            const uint16_t* fq, const uint16_t* fk, const uint16_t* v, float* out,
                            float* seg, float* tot, hipStream_t st,
                            const float* S0init = nullptr, uint16_t* outb = nullptr, int ldo = 0,
                            int rev = 0, int vld = 0, bool anti = false) {
  const llops_shape_t t = feat_attn_shape(s, M, DV);
  llops::AttnShape a = attn_shape(&t, causal);
  const int64_t per = static_cast<int64_t>(M) * DV + M;
  const bool mf32 = llops::attn32_supported(a);
  if ((outb || rev || vld) && !mf32) return hipErrorInvalidValue;
  if (anti) {  // suffix sums: the scan from the last segment, chunks from the last
    if (!causal || !mf32 || rev || S0init) return hipErrorInvalidValue;
    a.anti = 1;
  }
  hipError_t e = vld    ? llops::launch_seg_state32_v(a, fk, v, vld, seg, st)
                 : mf32 ? llops::launch_seg_state32(a, fk, v, seg, st)
                        : llops::launch_seg_state_bf16(a, fk, v, seg, st);
  if (e != hipSuccess) return e;
  const float* state = seg;
  int64_t st_seg = per, st_bh = per * a.nseg;
  if (causal) {  // S0init: [BH][M*DV] initial state (null = zeros)
    e = llops::launch_seg_scan(a, seg, S0init, nullptr, nullptr, nullptr, 1, st);
  } else {
    e = llops::launch_seg_scan(a, seg, nullptr, nullptr, tot, tot + static_cast<int64_t>(M) * DV,
                               0, st);
    state = tot;
    st_seg = 0;
    st_bh = per;
  }
  if (e != hipSuccess) return e;
  if (outb || rev)
    return llops::launch_attn_out32_to(a, fq, fk, v, state, st_seg, st_bh, out, outb, ldo, rev, st,
                                       vld);
  return mf32 ? llops::launch_attn_out32(a, fq, fk, v, state, st_seg, st_bh, out, st)
              : llops::launch_attn_out_bf16(a, fq, fk, v, state, st_seg, st_bh, out, st);
}

// The backward's chain-rule passes on narrow operands (m = 256, dv = 128
// kernels): phi_Q rows are stored as qald bf16 and read as [row | one? | 0]
// (likewise phi_K), without padded copies; values are the phi slice v (rows
// vld apart), rows go to outb (bf16, ldo apart). LLOPS_BWD_PADDED=1 in the
// environment selects the padded copies instead.
bool bwd_padded() {
  const char* env = getenv("LLOPS_BWD_PADDED");
  return env && env[0] == '1';
}

hipError_t attn_on_aug(const llops_shape_t* s, bool causal, bool anti, int M, int DV,
                       const uint16_t* fq, int qald, int qone, const uint16_t* fk, int kald,
                       int kone, const uint16_t* v, int vld, uint16_t* outb, int ldo, float* seg,
                       float* tot, hipStream_t st, const float* S0init = nullptr) {
  const llops_shape_t t = feat_attn_shape(s, M, DV);
  llops::AttnShape a = attn_shape(&t, causal);
  const int64_t per = static_cast<int64_t>(M) * DV + M;
  if (anti) {  // suffix sums: the scan from the last segment, chunks from the last
    if (!causal || S0init) return hipErrorInvalidValue;
    a.anti = 1;
  }
  hipError_t e = llops::launch_seg_state32_aug(a, fk, kald, kone, v, vld, seg, st);
  if (e != hipSuccess) return e;
  const float* state = seg;
  int64_t st_seg = per, st_bh = per * a.nseg;
  if (causal) {  // S0init: [BH][M*DV] initial state (null = zeros)
    e = llops::launch_seg_scan(a, seg, S0init, nullptr, nullptr, nullptr, 1, st);
  } else {
    e = llops::launch_seg_scan(a, seg, nullptr, nullptr, tot, tot + static_cast<int64_t>(M) * DV,
                               0, st);
    state = tot;
    st_seg = 0;
    st_bh = per;
  }
  if (e != hipSuccess) return e;
  return llops::launch_attn_out32_aug(a, fq, qald, qone, fk, kald, kone, v, vld, state, st_seg,
                                      st_bh, outb, ldo, st);
}

// num = M V and den = M 1 in one pass on the 32x32x16 shapes: the output pass
// forms each row's denominator phi_Q,i . z_i for the normalised form anyway,
// so it stores it beside the unnormalised row. (S0init, z0init): the initial
// state (causal; null = zeros).
bool num_den_one_pass(const llops_shape_t* s, bool causal) {
  const llops_shape_t t = feat_attn_shape(s, s->m, s->dv);
  return llops::attn32_supported(attn_shape(&t, causal));
}

hipError_t attn_num_den(const llops_shape_t* s, bool causal, const uint16_t* fq,
                        const uint16_t* fk, const uint16_t* v, float* num, float* den, float* seg,
                        float* tot, hipStream_t st, const float* S0init, const float* z0init) {
  llops_shape_t t = feat_attn_shape(s, s->m, s->dv);
  t.normalize = 1;  // delta stays 0: den is phi_Q . z
  const llops::AttnShape a = attn_shape(&t, causal);
  if (!llops::attn32_supported(a)) return hipErrorInvalidValue;
  const int64_t MD = static_cast<int64_t>(s->m) * s->dv, per = MD + s->m;
  hipError_t e = llops::launch_seg_state32(a, fk, v, seg, st);
  if (e != hipSuccess) return e;
  const float* state = seg;
  int64_t st_seg = per, st_bh = per * a.nseg;
  if (causal) {
    e = llops::launch_seg_scan(a, seg, S0init, z0init, nullptr, nullptr, 1, st);
  } else {
    e = llops::launch_seg_scan(a, seg, nullptr, nullptr, tot, tot + MD, 0, st);
    state = tot;
    st_seg = 0;
    st_bh = per;
  }
  if (e != hipSuccess) return e;
  return llops::launch_attn_out32_den(a, fq, fk, v, state, st_seg, st_bh, num, den, st);
}

// ---- gated causal backward ---------------------------------------------------

struct GBwdWs {
  BwdWs b;  // the ungated backward's buffers (its seg and den1/ones are not used)
  size_t glf, grev, glr, gseg, gden, dc, seg, seg2, dgb, p0, total;
};

GBwdWs gated_bwd_ws(const llops_shape_t* s) {
  GBwdWs w{};
  w.b = bwd_ws(s, true);
  const bool rev = !bwd_anti(s);  // reversed gates for the reversed passes
  size_t off = w.b.total;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  const size_t BH = static_cast<size_t>(s->batch * s->heads);
  const size_t R = BH * static_cast<size_t>(s->n);
  const size_t nld = static_cast<size_t>((s->n + 31) / 32 * 32);
  const int MA = bwd_ma(s), W = bwd_w(s);
  w.glf = take(BH * nld * 4);   // chunk-local sums of the forward gates
  w.grev = take(rev ? R * 4 : 0);        // gates of the reversed sequence
  w.glr = take(rev ? BH * nld * 4 : 0);  // and their chunk-local sums
  const llops_shape_t t = feat_attn_shape(s, s->m, s->dv);
  w.gseg = take(BH * static_cast<size_t>(seg_plan(&t, true, kGatedBwdWG).nseg) * 4);
  w.gden = take(s->normalize ? R * 4 : 0);  // M 1 per row, from the num pass
  w.dc = take(R * 4);           // d/dc_i = phi_Q,i . dphi_Q,i - phi_K,i . dphi_K,i
  size_t seg = feat_attn_seg_bytes(s, s->m, s->dv, true, kGatedBwdWG);
  const size_t seg2 = feat_attn_seg_bytes(s, MA, W, true, kGatedBwdWG);
  if (seg2 > seg) seg = seg2;
  w.seg = take(seg);
  w.seg2 = take(feat_attn_seg_bytes(s, MA, W, true, kGatedBwdWG));  // suffix states, dphi_Q slices
  w.dgb = take(BH * static_cast<size_t>(seg_plan(&t, true, kGatedBwdWG).nseg) * 4);  // dg at starts
  w.p0 = take(BH * static_cast<size_t>(MA) * W * 4);  // initial state of a dphi_Q slice pass
  w.total = off;
  return w;
}

llops_status_t validate_gated_bwd(const llops_shape_t* s) {
  LLOPS_TRY(validate_attn_bwd(s, true));
  if (!((s->m == 256 && s->dv == 128) || (s->m == 128 && s->dv == 64) ||
        (s->m == 64 && s->dv == 64)))
    return fail(LLOPS_ERR_UNSUPPORTED,
                "gated backward kernels: (m, dv) in {(256, 128), (128, 64), (64, 64)} "
                "(got m=%d dv=%d)", s->m, s->dv);
  return LLOPS_OK;
}

// out_i = sum_{j<=i} exp(c_i - c_j) (fq_i . fk_j) v_j over bf16 features from a
// zero state, gl the chunk-local sums of the pass's gates; the gated segment
// kernels.
hipError_t gated_attn_on_features(const llops_shape_t* s, int M, int DV, const uint16_t* fq,
                                  const uint16_t* fk, const uint16_t* v, const float* gl,
                                  float* out, float* seg, float* gseg, hipStream_t st,
                                  const float* S0init = nullptr, int vld = 0, int rev = 0) {
  const llops_shape_t t = feat_attn_shape(s, M, DV);
  const llops::AttnShape a = attn_shape(&t, true, kGatedBwdWG);
  if (!llops::attn32_supported(a)) return hipErrorInvalidValue;
  hipError_t e = vld ? llops::launch_seg_state32_gated_v(a, fk, v, vld, gl, gseg, seg, false, st)
                     : llops::launch_seg_state32_gated(a, fk, v, gl, gseg, seg, st);
  if (e == hipSuccess)
    e = llops::launch_seg_scan_gated(a, seg, gseg, S0init, nullptr, nullptr, nullptr, st);
  if (e == hipSuccess)
    e = (vld || rev) ? llops::launch_attn_out32_gated_to(a, fq, fk, v, gl, seg, out, rev, vld, st)
                     : llops::launch_attn_out32_gated(a, fq, fk, v, gl, seg, out, st);
  return e;
}

// gated_attn_on_features on narrow operands (attn_on_aug): phi_Q rows stored
// as qald bf16 (a one at column qald if qone), phi_K likewise; fp32 rows to out.
hipError_t gated_attn_on_aug(const llops_shape_t* s, int M, int DV, const uint16_t* fq, int qald,
                             int qone, const uint16_t* fk, int kald, int kone, const uint16_t* v,
                             int vld, const float* gl, float* out, float* seg, float* gseg,
                             hipStream_t st, const float* S0init) {
  const llops_shape_t t = feat_attn_shape(s, M, DV);
  const llops::AttnShape a = attn_shape(&t, true, kGatedBwdWG);
  hipError_t e =
      llops::launch_seg_state32_gated_aug(a, fk, kald, kone, v, vld, gl, gseg, seg, false, st);
  if (e == hipSuccess)
    e = llops::launch_seg_scan_gated(a, seg, gseg, S0init, nullptr, nullptr, nullptr, st);
  if (e == hipSuccess)
    e = llops::launch_attn_out32_gated_aug(a, fq, qald, qone, fk, kald, kone, v, vld, gl, seg, out,
                                           st);
  return e;
}

// Gated num = M V and den = M 1 per row in one pass (see attn_num_den).
hipError_t gated_attn_num_den(const llops_shape_t* s, const uint16_t* fq, const uint16_t* fk,
                              const uint16_t* v, const float* gl, float* num, float* den,
                              float* seg, float* gseg, hipStream_t st, const float* S0init,
                              const float* z0init) {
  llops_shape_t t = feat_attn_shape(s, s->m, s->dv);
  t.normalize = 1;  // delta stays 0: den is phi_Q . z
  const llops::AttnShape a = attn_shape(&t, true, kGatedBwdWG);
  if (!llops::attn32_supported(a)) return hipErrorInvalidValue;
  hipError_t e = llops::launch_seg_state32_gated(a, fk, v, gl, gseg, seg, st);
  if (e == hipSuccess)
    e = llops::launch_seg_scan_gated(a, seg, gseg, S0init, z0init, nullptr, nullptr, st);
  if (e == hipSuccess) e = llops::launch_attn_out32_gated_den(a, fq, fk, v, gl, seg, num, den, st);
  return e;
}

// Totals over all rows of fk^T v (and fk^T 1) per (b, h) into Stot [BH][M*DV]
// and ztot (null, or Stot + M*DV for one contiguous [BH][M*DV + M] block).
hipError_t state_total(const llops_shape_t* s, int M, int DV, const uint16_t* fk,
                       const uint16_t* v, float* seg, float* Stot, float* ztot, hipStream_t st) {
  const llops_shape_t t = feat_attn_shape(s, M, DV);
  const llops::AttnShape a = attn_shape(&t, true);
  hipError_t e = llops::attn32_supported(a) ? llops::launch_seg_state32(a, fk, v, seg, st)
                                            : llops::launch_seg_state_bf16(a, fk, v, seg, st);
  if (e == hipSuccess) e = llops::launch_seg_scan(a, seg, nullptr, nullptr, Stot, ztot, 0, st);
  return e;
}

// With LLOPS_FUSED_Q=1 in the environment the causal bf16 forward projects
// phi_Q inside its output pass (phi_Q never reaches HBM), where a fused kernel
// exists for the shape and Theta_Q has a fragment-order copy (more than 1024
// rows per head). Both paths compute the same values bit for bit; the
// two-kernel path (feature maps of Q and K, then the segment passes) is the
// default because it measures faster on MI355X (the fused pass re-streams
// Theta_Q from L2 every 64 rows instead of every 256).
bool fused_q(const llops_shape_t* s, const llops::AttnShape& a) {
  const char* env = getenv("LLOPS_FUSED_Q");
  if (!env || env[0] != '1') return false;
  return pack_bytes(s, s->n) > 0 && llops::attn32_fq_supported(a, s->d, s->p, s->t);
}

// Shared body of the non-causal and causal forward passes.
llops_status_t attention(const llops_shape_t* s, bool causal, const void* Q, const void* K,
                         const void* V, const void* tq, const void* tk, const float* S0,
                         const float* z0, void* out, float* S_final, float* z_final, void* ws,
                         size_t ws_bytes, hipStream_t st) {
  const int entry = causal ? LLOPS_ENTRY_CAUSAL : LLOPS_ENTRY_LINATTN;
  LLOPS_TRY(validate(s, entry));
  const int64_t BH = s->batch * s->heads;
  if (BH == 0) return LLOPS_OK;
  if (s->n == 0) {  // empty sequences: Q/K/V/out may be null; the state passes through
    LLOPS_TRY(opt(S0, "S0"));
    LLOPS_TRY(opt(z0, "z0"));
    LLOPS_TRY(opt(S_final, "S_final"));
    LLOPS_TRY(opt(z_final, "z_final"));
    if (causal && (S_final || z_final))
      LLOPS_HIP(llops::launch_state_init(BH, s->m, s->dv, S0, z0, S_final, z_final, st),
                "state_init");
    return LLOPS_OK;
  }
  LLOPS_TRY(need(Q, "Q"));
  LLOPS_TRY(need(K, "K"));
  LLOPS_TRY(need(V, "V"));
  LLOPS_TRY(need(tq, "theta_q"));
  LLOPS_TRY(need(tk, "theta_k"));
  LLOPS_TRY(need(out, "out"));
  LLOPS_TRY(opt(S0, "S0"));
  LLOPS_TRY(opt(z0, "z0"));
  LLOPS_TRY(opt(S_final, "S_final"));
  LLOPS_TRY(opt(z_final, "z_final"));
  const WsLayout L = ws_layout(s, entry);
  if (ws_bytes < L.total)
    return fail(LLOPS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  if (L.total && !ws) return fail(LLOPS_ERR_INVALID_ARG, "ws is null");
  if (ws) LLOPS_TRY(opt(ws, "ws"));
  char* w = static_cast<char*>(ws);
  const bool bf16 = s->in_dtype == LLOPS_BF16;
  const llops::AttnShape a = attn_shape(s, causal);
  const int64_t per = static_cast<int64_t>(s->m) * s->dv + s->m;
  float* seg = reinterpret_cast<float*>(w + L.seg);
  llops::FeatJob jobs[2] = {{Q, tq, w + L.phiq, w + L.pkq}, {K, tk, w + L.phik, w + L.pkk}};
  const llops::FeatShape fs = feat_shape(s, s->n, bf16 ? 1 : 0);
  if (bf16 && causal && fused_q(s, a)) {
    // phi_Q is projected inside the output pass: only phi_K goes through HBM
    LLOPS_HIP(llops::launch_featmap_bf16(fs, &jobs[1], 1, st), "featmap");
    LLOPS_HIP(llops::launch_pack_theta(fs, tq, w + L.pkq, st), "pack_theta");
    const uint16_t* pk = reinterpret_cast<const uint16_t*>(w + L.phik);
    const uint16_t* vv = static_cast<const uint16_t*>(V);
    LLOPS_HIP(llops::launch_seg_state32(a, pk, vv, seg, st), "seg_state");
    LLOPS_HIP(llops::launch_seg_scan(a, seg, S0, z0, S_final, z_final, 1, st), "seg_scan");
    const int64_t pk_hstride =
        s->theta_per_head ? static_cast<int64_t>(s->p) * s->t * s->d * s->m : 0;
    LLOPS_HIP(llops::launch_attn_out32_fq(a, s->d, s->p, s->t, static_cast<const uint16_t*>(Q),
                                          reinterpret_cast<const uint16_t*>(w + L.pkq),
                                          pk_hstride, s->heads, s->square, pk, vv, seg, per,
                                          per * a.nseg, static_cast<float*>(out), st),
              "attn_out_fq");
  } else if (bf16) {
    LLOPS_HIP(llops::launch_featmap_bf16(fs, jobs, 2, st), "featmap");
    const uint16_t* pq = reinterpret_cast<const uint16_t*>(w + L.phiq);
    const uint16_t* pk = reinterpret_cast<const uint16_t*>(w + L.phik);
    const uint16_t* vv = static_cast<const uint16_t*>(V);
    const bool mf32 = llops::attn32_supported(a);  // 32x32x16 kernels for this (m, dv)
    if (mf32)
      LLOPS_HIP(llops::launch_seg_state32(a, pk, vv, seg, st), "seg_state");
    else
      LLOPS_HIP(llops::launch_seg_state_bf16(a, pk, vv, seg, st), "seg_state");
    const float* state = seg;
    int64_t st_seg = per, st_bh = per * a.nseg;
    if (causal) {
      LLOPS_HIP(llops::launch_seg_scan(a, seg, S0, z0, S_final, z_final, 1, st), "seg_scan");
    } else {
      float* tot = reinterpret_cast<float*>(w + L.tot);
      LLOPS_HIP(llops::launch_seg_scan(a, seg, nullptr, nullptr, tot,
                                       tot + static_cast<int64_t>(s->m) * s->dv, 0, st),
                "seg_scan");
      state = tot;
      st_seg = 0;
      st_bh = per;
    }
    float* o = static_cast<float*>(out);
    if (mf32)
      LLOPS_HIP(llops::launch_attn_out32(a, pq, pk, vv, state, st_seg, st_bh, o, st), "attn_out");
    else
      LLOPS_HIP(llops::launch_attn_out_bf16(a, pq, pk, vv, state, st_seg, st_bh, o, st),
                "attn_out");
  } else if (!causal && llops::linattn_small_f32_ok(BH, s->n, s->d, s->dv, s->m, s->p, s->t)) {
    // small fp32 sequences: the whole non-causal pass in one launch
    const int64_t th_hstride =
        s->theta_per_head ? static_cast<int64_t>(s->p) * s->t * s->d * s->m : 0;
    LLOPS_HIP(llops::launch_linattn_small_f32(
                  s->batch, s->heads, s->n, s->d, s->dv, s->m, s->p, s->t,
                  static_cast<const float*>(Q), static_cast<const float*>(K),
                  static_cast<const float*>(V), static_cast<const float*>(tq),
                  static_cast<const float*>(tk), th_hstride, s->square, s->normalize, s->delta,
                  static_cast<float*>(out), st),
              "linattn_small_f32");
  } else {
    LLOPS_HIP(llops::launch_featmap_f32(fs, jobs, 2, st), "featmap");
    const float* pq = reinterpret_cast<const float*>(w + L.phiq);
    const float* pk = reinterpret_cast<const float*>(w + L.phik);
    const float* vv = static_cast<const float*>(V);
    LLOPS_HIP(llops::launch_seg_state_f32(a, pk, vv, seg, st), "seg_state");
    if (causal) {
      LLOPS_HIP(llops::launch_seg_scan(a, seg, S0, z0, S_final, z_final, 1, st), "seg_scan");
      LLOPS_HIP(llops::launch_attn_out_f32(a, pq, pk, vv, seg, per, per * a.nseg,
                                           static_cast<float*>(out), st),
                "attn_out");
    } else {
      float* tot = reinterpret_cast<float*>(w + L.tot);
      LLOPS_HIP(llops::launch_seg_scan(a, seg, nullptr, nullptr, tot,
                                       tot + static_cast<int64_t>(s->m) * s->dv, 0, st),
                "seg_scan");
      LLOPS_HIP(llops::launch_attn_out_f32(a, pq, pk, vv, tot, 0, per, static_cast<float*>(out),
                                           st),
                "attn_out");
    }
  }
  return LLOPS_OK;
}

}  // namespace

namespace llops {
namespace {
struct ProfState {
  hipEvent_t* events = nullptr;
  const char** names = nullptr;
  int32_t cap = 0;
  int32_t n = 0;
  bool armed = false;
};
thread_local ProfState g_prof;
}  // namespace

void prof_before(const char* name, hipStream_t st) {
  if (!g_prof.armed || g_prof.n >= g_prof.cap) return;
  if (g_prof.names) g_prof.names[g_prof.n] = name;
  (void)hipEventRecord(g_prof.events[2 * g_prof.n], st);
}

void prof_after(hipStream_t st) {
  if (!g_prof.armed || g_prof.n >= g_prof.cap) return;
  (void)hipEventRecord(g_prof.events[2 * g_prof.n + 1], st);
  ++g_prof.n;
}
}  // namespace llops

extern "C" {

llops_status_t llops_profile_arm(hipEvent_t* events, const char** names, int32_t capacity) {
  if (!events || capacity < 0) return fail(LLOPS_ERR_INVALID_ARG, "profile: bad events/capacity");
  llops::g_prof.events = events;
  llops::g_prof.names = names;
  llops::g_prof.cap = capacity;
  llops::g_prof.n = 0;
  llops::g_prof.armed = true;
  return LLOPS_OK;
}

int32_t llops_profile_disarm(void) {
  const int32_t n = llops::g_prof.n;
  llops::g_prof = llops::ProfState{};
  return n;
}

size_t llops_workspace_bytes(const llops_shape_t* shape, int32_t entry) {
  if (!shape || entry < LLOPS_ENTRY_FEATMAP || entry > LLOPS_ENTRY_GATED_CAUSAL_BWD) return 0;
  if (entry == LLOPS_ENTRY_GATED_CAUSAL_BWD)
    return validate_gated_bwd(shape) == LLOPS_OK ? gated_bwd_ws(shape).total : 0;
  if (entry == LLOPS_ENTRY_GATED_CAUSAL && validate_gated(shape) != LLOPS_OK) return 0;
  if (entry == LLOPS_ENTRY_CAUSAL_BWD || entry == LLOPS_ENTRY_LINATTN_BWD) {
    const bool causal = entry == LLOPS_ENTRY_CAUSAL_BWD;
    if (validate_attn_bwd(shape, causal) != LLOPS_OK) return 0;
    return bwd_ws(shape, causal).total;
  }
  if (validate(shape, entry) != LLOPS_OK) return 0;
  return ws_layout(shape, entry).total;
}

llops_status_t llops_featmap(const llops_shape_t* s, const void* X, const void* theta, void* phi,
                             void* ws, size_t ws_bytes, hipStream_t st) {
  LLOPS_TRY(validate(s, LLOPS_ENTRY_FEATMAP));
  if (s->batch * s->heads == 0 || s->n == 0) return LLOPS_OK;  // empty: pointers may be null
  LLOPS_TRY(need(X, "X"));
  LLOPS_TRY(need(theta, "theta"));
  LLOPS_TRY(need(phi, "phi"));
  if (s->in_dtype == LLOPS_F32 && s->out_dtype != LLOPS_F32)
    return fail(LLOPS_ERR_UNSUPPORTED, "fp32 inputs produce fp32 phi only");
  const WsLayout L = ws_layout(s, LLOPS_ENTRY_FEATMAP);
  if (ws_bytes < L.total)
    return fail(LLOPS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  if (L.total && !ws) return fail(LLOPS_ERR_INVALID_ARG, "ws is null");
  if (ws) LLOPS_TRY(opt(ws, "ws"));
  llops::FeatJob job{X, theta, phi, L.total ? static_cast<char*>(ws) + L.pkq : nullptr};
  const llops::FeatShape fs = feat_shape(s, s->n, s->out_dtype == LLOPS_BF16 ? 1 : 0);
  if (s->in_dtype == LLOPS_BF16)
    LLOPS_HIP(llops::launch_featmap_bf16(fs, &job, 1, st), "featmap");
  else
    LLOPS_HIP(llops::launch_featmap_f32(fs, &job, 1, st), "featmap");
  return LLOPS_OK;
}

llops_status_t llops_featmap_bwd(const llops_shape_t* s, const void* X, const void* theta,
                                 const void* dphi, float* dX, float* dtheta, void* ws,
                                 size_t ws_bytes, hipStream_t st) {
  LLOPS_TRY(validate(s, LLOPS_ENTRY_FEATMAP_BWD));
  if (s->in_dtype != LLOPS_BF16)
    return fail(LLOPS_ERR_UNSUPPORTED, "featmap backward takes bf16 X and Theta only");
  const llops::FeatShape fs = feat_shape(s, s->n, 0);
  if (!llops::featmap_bwd_supported(fs))
    return fail(LLOPS_ERR_UNSUPPORTED,
                "featmap backward kernels: p = 2, t in {1, 4}, d in {64, 128}, m %% 32 == 0 "
                "(got p=%d t=%d d=%d m=%d)", s->p, s->t, s->d, s->m);
  if (s->heads == 0) return LLOPS_OK;  // nothing to write
  const bool rows = s->batch > 0 && s->n > 0;
  LLOPS_TRY(need(theta, "theta"));
  LLOPS_TRY(need(dtheta, "dtheta"));
  if (rows) {
    LLOPS_TRY(need(X, "X"));
    LLOPS_TRY(need(dphi, "dphi"));
    LLOPS_TRY(need(dX, "dX"));
  }
  const WsLayout L = ws_layout(s, LLOPS_ENTRY_FEATMAP_BWD);
  if (ws_bytes < L.total)
    return fail(LLOPS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  if (L.total && !ws) return fail(LLOPS_ERR_INVALID_ARG, "ws is null");
  if (ws) LLOPS_TRY(opt(ws, "ws"));
  LLOPS_HIP(llops::launch_featmap_bwd(fs, X, theta, dphi, s->out_dtype == LLOPS_BF16 ? 1 : 0, dX,
                                      dtheta, L.total ? static_cast<char*>(ws) + L.seg : nullptr,
                                      st),
            "featmap_bwd");
  return LLOPS_OK;
}

llops_status_t llops_linattn_fwd(const llops_shape_t* s, const void* Q, const void* K,
                                 const void* V, const void* theta_q, const void* theta_k,
                                 void* out, void* ws, size_t ws_bytes, hipStream_t st) {
  return attention(s, false, Q, K, V, theta_q, theta_k, nullptr, nullptr, out, nullptr, nullptr,
                   ws, ws_bytes, st);
}

llops_status_t llops_linattn_causal_fwd(const llops_shape_t* s, const void* Q, const void* K,
                                        const void* V, const void* theta_q, const void* theta_k,
                                        const float* S0, const float* z0, void* out,
                                        float* S_final, float* z_final, void* ws,
                                        size_t ws_bytes, hipStream_t st) {
  return attention(s, true, Q, K, V, theta_q, theta_k, S0, z0, out, S_final, z_final, ws,
                   ws_bytes, st);
}

llops_status_t llops_linattn_gated_causal_fwd(const llops_shape_t* s, const void* Q, const void* K,
                                              const void* V, const void* theta_q,
                                              const void* theta_k, const float* log_gate,
                                              const float* S0, const float* z0, void* out,
                                              float* S_final, float* z_final, void* ws,
                                              size_t ws_bytes, hipStream_t st) {
  LLOPS_TRY(validate_gated(s));
  const int64_t BH = s->batch * s->heads;
  if (BH == 0) return LLOPS_OK;
  LLOPS_TRY(opt(S0, "S0"));
  LLOPS_TRY(opt(z0, "z0"));
  LLOPS_TRY(opt(S_final, "S_final"));
  LLOPS_TRY(opt(z_final, "z_final"));
  if (s->n == 0) {  // no tokens, no decay: the state passes through
    if (S_final || z_final)
      LLOPS_HIP(llops::launch_state_init(BH, s->m, s->dv, S0, z0, S_final, z_final, st),
                "state_init");
    return LLOPS_OK;
  }
  LLOPS_TRY(need(Q, "Q"));
  LLOPS_TRY(need(K, "K"));
  LLOPS_TRY(need(V, "V"));
  LLOPS_TRY(need(theta_q, "theta_q"));
  LLOPS_TRY(need(theta_k, "theta_k"));
  LLOPS_TRY(need4(log_gate, "log_gate"));
  LLOPS_TRY(need(out, "out"));
  const WsLayout L = ws_layout(s, LLOPS_ENTRY_GATED_CAUSAL);
  if (ws_bytes < L.total)
    return fail(LLOPS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  if (!ws) return fail(LLOPS_ERR_INVALID_ARG, "ws is null");
  LLOPS_TRY(opt(ws, "ws"));
  char* w = static_cast<char*>(ws);
  const llops::AttnShape a = attn_shape(s, true);
  float* seg = reinterpret_cast<float*>(w + L.seg);
  float* gl = reinterpret_cast<float*>(w + L.gl);
  float* gseg = reinterpret_cast<float*>(w + L.gseg);
  llops::FeatJob jobs[2] = {{Q, theta_q, w + L.phiq, w + L.pkq}, {K, theta_k, w + L.phik, w + L.pkk}};
  if (s->in_dtype != LLOPS_BF16) {
    LLOPS_HIP(llops::launch_featmap_f32(feat_shape(s, s->n, 0), jobs, 2, st), "featmap");
    const float* pq = reinterpret_cast<const float*>(w + L.phiq);
    const float* pk = reinterpret_cast<const float*>(w + L.phik);
    const float* vv = static_cast<const float*>(V);
    LLOPS_HIP(llops::launch_seg_state_f32_gated(a, pk, vv, log_gate, gseg, seg, st),
              "seg_state_f32_gated");
    LLOPS_HIP(llops::launch_seg_scan_gated(a, seg, gseg, S0, z0, S_final, z_final, st), "seg_scan");
    LLOPS_HIP(llops::launch_attn_out_f32_gated(a, pq, pk, vv, log_gate, seg,
                                               static_cast<float*>(out), st),
              "attn_out_f32_gated");
    return LLOPS_OK;
  }
  LLOPS_HIP(llops::launch_featmap_bf16(feat_shape(s, s->n, 1), jobs, 2, st), "featmap");
  const uint16_t* pq = reinterpret_cast<const uint16_t*>(w + L.phiq);
  const uint16_t* pk = reinterpret_cast<const uint16_t*>(w + L.phik);
  const uint16_t* vv = static_cast<const uint16_t*>(V);
  LLOPS_HIP(llops::launch_gate_cumsum32(BH, s->n, log_gate, gl, st), "gate_cumsum");
  LLOPS_HIP(llops::launch_seg_state32_gated(a, pk, vv, gl, gseg, seg, st), "seg_state_gated");
  LLOPS_HIP(llops::launch_seg_scan_gated(a, seg, gseg, S0, z0, S_final, z_final, st), "seg_scan");
  LLOPS_HIP(llops::launch_attn_out32_gated(a, pq, pk, vv, gl, seg, static_cast<float*>(out), st),
            "attn_out_gated");
  return LLOPS_OK;
}

// Shared body of the causal and non-causal attention backward.
// S0, z0 (causal only, nullable): the forward continued from an initial
// state; dS0, dz0 (nullable): its gradients.
static llops_status_t attn_backward(const llops_shape_t* s, bool causal, const void* Q, const void* K,
                             const void* V, const void* theta_q, const void* theta_k,
                             const float* dO, float* dQ, float* dK, float* dV, float* dtheta_q,
                             float* dtheta_k, void* ws, size_t ws_bytes, hipStream_t st,
                             const float* S0 = nullptr, const float* z0 = nullptr,
                             float* dS0 = nullptr, float* dz0 = nullptr) {
  LLOPS_TRY(validate_attn_bwd(s, causal));
  const int64_t BH = s->batch * s->heads;
  if (s->heads == 0) return LLOPS_OK;
  LLOPS_TRY(need(theta_q, "theta_q"));
  LLOPS_TRY(need(theta_k, "theta_k"));
  LLOPS_TRY(need(dtheta_q, "dtheta_q"));
  LLOPS_TRY(need(dtheta_k, "dtheta_k"));
  const int64_t R = BH * s->n;
  if (R > 0) {
    LLOPS_TRY(need(Q, "Q"));
    LLOPS_TRY(need(K, "K"));
    LLOPS_TRY(need(V, "V"));
    LLOPS_TRY(need(dO, "dO"));
    LLOPS_TRY(need(dQ, "dQ"));
    LLOPS_TRY(need(dK, "dK"));
    LLOPS_TRY(need(dV, "dV"));
  }
  LLOPS_TRY(opt(S0, "S0"));
  LLOPS_TRY(opt(z0, "z0"));
  LLOPS_TRY(opt(dS0, "dS0"));
  LLOPS_TRY(opt(dz0, "dz0"));
  const BwdWs L = bwd_ws(s, causal);
  if (ws_bytes < L.total)
    return fail(LLOPS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  if (L.total && !ws) return fail(LLOPS_ERR_INVALID_ARG, "ws is null");
  if (ws) LLOPS_TRY(opt(ws, "ws"));
  char* w = static_cast<char*>(ws);
  auto u16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(w + off); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  const llops::FeatShape fs0 = feat_shape(s, s->n, 0);
  float* fb = L.fb ? f32(L.fb) : nullptr;
  if (R == 0) {  // no rows: the Theta (and initial-state) gradients are zero
    LLOPS_HIP(llops::launch_featmap_bwd(fs0, Q, theta_q, dO, 0, dQ, dtheta_q, fb, st), "featmap_bwd");
    LLOPS_HIP(llops::launch_featmap_bwd(fs0, K, theta_k, dO, 0, dK, dtheta_k, fb, st), "featmap_bwd");
    if (dS0 || dz0)
      LLOPS_HIP(llops::launch_state_init(BH, s->m, s->dv, nullptr, nullptr, dS0, dz0, st),
                "state_init");
    return LLOPS_OK;
  }
  const int m = s->m, dv = s->dv, MA = bwd_ma(s), W = bwd_w(s);
  const int64_t n = s->n;
  uint16_t *phq = u16(L.phq), *phk = u16(L.phk);
  float* seg = f32(L.seg);
  float* tot = causal ? nullptr : f32(L.tot);
  // feature maps of Q and K (bf16, as the forward stores them)
  llops::FeatJob jobs[2] = {{Q, theta_q, phq, w + L.pkq}, {K, theta_k, phk, w + L.pkk}};
  LLOPS_HIP(llops::launch_featmap_bf16(feat_shape(s, n, 1), jobs, 2, st), "featmap");
  // num = M V and, with the normaliser, M 1: one pass on the 32x32x16
  // shapes, else a second pass over all-ones values. Unnormalised, dnum = dO
  // and dden = 0, so neither is formed.
  float* num = s->normalize ? f32(L.num) : nullptr;
  float* den1 = nullptr;
  int den_ld = 16;
  if (s->normalize && num_den_one_pass(s, causal)) {
    den1 = f32(L.den1);
    den_ld = 1;
    LLOPS_HIP(attn_num_den(s, causal, phq, phk, static_cast<const uint16_t*>(V), num, den1, seg,
                           tot, st, S0, z0),
              "attn num den");
  } else if (s->normalize) {
    LLOPS_HIP(attn_on_features(s, causal, m, dv, phq, phk, static_cast<const uint16_t*>(V), num,
                               seg, tot, st, S0),
              "attn num");
  }
  if (s->normalize && den_ld == 16) {
    den1 = f32(L.den1);
    LLOPS_HIP(llops::launch_fill_ones16(u16(L.ones), R, st), "ones");
    const float* zinit = nullptr;  // z0 in every column of the all-ones pass
    if (z0) {
      LLOPS_HIP(llops::launch_state_bcast(z0, BH, m, 16, f32(L.zb16), st), "state");
      zinit = f32(L.zb16);
    }
    LLOPS_HIP(attn_on_features(s, causal, m, 16, phq, phk, u16(L.ones), den1, seg, tot, st, zinit),
              "attn den");
  }
  // a = [dnum | dden | 0], b = [V | 1 | 0]; with reversed copies (causal,
  // off the anti-causal path) also ra, rb and dnum reversed, else dnum in order
  const bool anti = causal && bwd_anti(s);
  const bool rev = causal && !anti;
  uint16_t *a = u16(L.a), *b = u16(L.b), *dn = u16(L.rdnum);
  uint16_t *ra = rev ? u16(L.ra) : nullptr, *rb = rev ? u16(L.rb) : nullptr;
  const bool inplace = on32(s, causal, MA, W);
  const bool sliced = inplace && n * m * 2 < (int64_t{1} << 31);
  const bool init = causal && (S0 || z0);
  // the chain-rule passes read [dnum | dden | 0] from a narrow copy (held
  // where a would be) and [V | 1 | 0] from V itself instead of the padded
  // copies, where their kernels apply
  const llops_shape_t ta = feat_attn_shape(s, MA, W);
  const bool aug = !rev && sliced && !bwd_padded() && dv % 8 == 0 && dv + 8 <= MA &&
                   llops::aug32_supported(attn_shape(&ta, causal));
  if (aug)
    LLOPS_HIP(llops::launch_make_ab_aug(num, den1, dO, dv, R, s->normalize,
                                        s->normalize ? s->delta : 0.f, a, dn, den_ld, st),
              "make_ab");
  else
    LLOPS_HIP(llops::launch_make_ab(num, den1, dO, static_cast<const uint16_t*>(V), dv, MA, n, R,
                                    s->normalize, s->normalize ? s->delta : 0.f, a, ra, b, rb, dn,
                                    rev ? 1 : 0, den_ld, st),
              "make_ab");
  uint16_t* vp = u16(L.vp);
  float* tmp = f32(L.tmp);
  uint16_t *dphq = u16(L.dphq), *dphk = u16(L.dphk);  // bf16, as the forward stores phi
  uint16_t *rphq = rev ? u16(L.rphq) : nullptr, *rphk = rev ? u16(L.rphk) : nullptr;
  if (rev) {
    LLOPS_HIP(llops::launch_rows_copy_bf16(phq, m, 0, rphq, m, 0, m, n, R, 1, st), "rows");
    LLOPS_HIP(llops::launch_rows_copy_bf16(phk, m, 0, rphk, m, 0, m, n, R, 1, st), "rows");
  }
  // initial-state gradients: dS0 = sum_i phi_Q,i dnum_i^T (rows of both in
  // one order, reversed or not), dz0 = sum_i dden_i phi_Q,i (dden is column dv of a)
  if (causal && dS0)
    LLOPS_HIP(state_total(s, m, dv, rev ? rphq : phq, dn, seg, dS0, nullptr, st), "dS0");
  if (causal && dz0) {
    float* stot = f32(L.stot);
    // the dden column (with zeros after it) as a 16-wide value block; only
    // column 0 of the total below is kept. The narrow a holds 8 columns from
    // dv on: they go into both halves of the block, so every column is defined
    if (aug) {
      LLOPS_HIP(llops::launch_rows_copy_bf16(a, dv + 8, dv, vp, 16, 0, 8, n, R, 0, st), "rows");
      LLOPS_HIP(llops::launch_rows_copy_bf16(a, dv + 8, dv, vp, 16, 8, 8, n, R, 0, st), "rows");
    } else {
      LLOPS_HIP(llops::launch_rows_copy_bf16(a, MA, dv, vp, 16, 0, 16, n, R, 0, st), "rows");
    }
    LLOPS_HIP(state_total(s, m, 16, phq, vp, seg, stot, stot + static_cast<int64_t>(m) * 16, st),
              "dz0");
    LLOPS_HIP(llops::launch_col_extract(stot, BH, m, static_cast<int64_t>(m) * 16 + m, 16, dz0, st),
              "dz0");
  }
  // dphi_Q_i = sum_{j(<=i)} (a_i . b_j) phi_K_j (+ dnum_i . S0 + dden_i z0 from an
  // initial state), W columns of phi_K at a time
  // On the 32x32x16 kernels the passes write dphi (bf16, a column slice) and
  // dV in place (in the original row order when they run over the reversed
  // sequence); otherwise through tmp and a row copy. They also read their phi
  // slice in place (rows m apart; on the reversed path the reversed sequence's
  // from the reversed copy of phi_Q) instead of from a sliced copy.
  const uint16_t* vv = static_cast<const uint16_t*>(V);
  for (int p0 = 0; aug && p0 < m; p0 += W) {
    // dphi_Q_i = sum_{j(<=i)} (a_i . b_j) phi_K_j, a = [dnum | dden], b = [V | 1]
    // (+ dnum_i . S0 + dden_i z0 from an initial state: its rows past dv are
    // zero, so the skipped feature tiles stay zero)
    if (init)
      LLOPS_HIP(llops::launch_build_p0(S0, z0, BH, m, dv, MA, W, p0, f32(L.p0), st), "state");
    LLOPS_HIP(attn_on_aug(s, causal, false, MA, W, a, dv + 8, 0, vv, dv, 1, phk + p0, m, dphq + p0,
                          m, seg, tot, st, init ? f32(L.p0) : nullptr),
              "attn dphi_q");
    // dphi_K_j = sum_{i(>=j)} (a_i . b_j) phi_Q_i: suffix sums (anti-causal)
    LLOPS_HIP(attn_on_aug(s, causal, anti, MA, W, vv, dv, 1, a, dv + 8, 0, phq + p0, m, dphk + p0,
                          m, seg, tot, st),
              "attn dphi_k");
  }
  for (int p0 = 0; !aug && p0 < m; p0 += W) {
    if (!sliced)
      LLOPS_HIP(llops::launch_rows_copy_bf16(phk, m, p0, vp, W, 0, W, n, R, 0, st), "rows");
    if (init)
      LLOPS_HIP(llops::launch_build_p0(S0, z0, BH, m, dv, MA, W, p0, f32(L.p0), st), "state");
    LLOPS_HIP(attn_on_features(s, causal, MA, W, a, b, sliced ? phk + p0 : vp, tmp, seg, tot, st,
                               init ? f32(L.p0) : nullptr, inplace ? dphq + p0 : nullptr, m, 0,
                               sliced ? m : 0),
              "attn dphi_q");
    if (!inplace)
      LLOPS_HIP(llops::launch_rows_copy_f32_bf16(tmp, W, 0, dphq, m, p0, W, n, R, 0, st), "rows");
  }
  // dphi_K_j = sum_{i(>=j)} (a_i . b_j) phi_Q_i: anti-causal, or causal over
  // the reversed sequence
  const int rv = rev ? 1 : 0;
  for (int p0 = 0; !aug && anti && p0 < m; p0 += W)
    LLOPS_HIP(attn_on_features(s, true, MA, W, b, a, phq + p0, tmp, seg, tot, st, nullptr,
                               dphk + p0, m, 0, m, true),
              "attn dphi_k");
  for (int p0 = 0; !aug && !anti && p0 < m; p0 += W) {
    if (!sliced)
      LLOPS_HIP(llops::launch_rows_copy_bf16(phq, m, p0, vp, W, 0, W, n, R, rv, st), "rows");
    const uint16_t* qv = sliced ? (causal ? rphq : phq) + p0 : vp;
    LLOPS_HIP(attn_on_features(s, causal, MA, W, causal ? rb : b, causal ? ra : a, qv, tmp, seg,
                               tot, st, nullptr, inplace ? dphk + p0 : nullptr, m,
                               inplace ? rv : 0, sliced ? m : 0),
              "attn dphi_k");
    if (!inplace)
      LLOPS_HIP(llops::launch_rows_copy_f32_bf16(tmp, W, 0, dphk, m, p0, W, n, R, rv, st), "rows");
  }
  // dV_j = sum_{i(>=j)} (phi_Q_i . phi_K_j) dnum_i: anti-causal, or causal over
  // the reversed sequence
  if (anti) {
    LLOPS_HIP(attn_on_features(s, true, m, dv, phk, phq, dn, dV, seg, nullptr, st, nullptr,
                               nullptr, 0, 0, 0, true),
              "attn dv");
  } else if (causal && on32(s, true, m, dv)) {
    LLOPS_HIP(attn_on_features(s, true, m, dv, rphk, rphq, dn, dV, seg, nullptr, st, nullptr,
                               nullptr, 0, 1),
              "attn dv");
  } else if (causal) {
    LLOPS_HIP(attn_on_features(s, true, m, dv, rphk, rphq, dn, tmp, seg, nullptr, st), "attn dv");
    LLOPS_HIP(llops::launch_rows_copy_f32(tmp, dv, 0, dV, dv, 0, dv, n, R, 1, st), "rows");
  } else {
    LLOPS_HIP(attn_on_features(s, false, m, dv, phk, phq, dn, dV, seg, tot, st), "attn dv");
  }
  // through the feature maps
  LLOPS_HIP(llops::launch_featmap_bwd(fs0, Q, theta_q, dphq, 1, dQ, dtheta_q, fb, st),
            "featmap_bwd q");
  LLOPS_HIP(llops::launch_featmap_bwd(fs0, K, theta_k, dphk, 1, dK, dtheta_k, fb, st),
            "featmap_bwd k");
  return LLOPS_OK;
}

llops_status_t llops_linattn_causal_bwd(const llops_shape_t* s, const void* Q, const void* K,
                                        const void* V, const void* theta_q, const void* theta_k,
                                        const float* dO, float* dQ, float* dK, float* dV,
                                        float* dtheta_q, float* dtheta_k, void* ws,
                                        size_t ws_bytes, hipStream_t st) {
  return attn_backward(s, true, Q, K, V, theta_q, theta_k, dO, dQ, dK, dV, dtheta_q, dtheta_k, ws,
                       ws_bytes, st);
}

llops_status_t llops_linattn_causal_bwd_state(const llops_shape_t* s, const void* Q, const void* K,
                                              const void* V, const void* theta_q,
                                              const void* theta_k, const float* S0,
                                              const float* z0, const float* dO, float* dQ,
                                              float* dK, float* dV, float* dtheta_q,
                                              float* dtheta_k, float* dS0, float* dz0, void* ws,
                                              size_t ws_bytes, hipStream_t st) {
  return attn_backward(s, true, Q, K, V, theta_q, theta_k, dO, dQ, dK, dV, dtheta_q, dtheta_k, ws,
                       ws_bytes, st, S0, z0, dS0, dz0);
}

llops_status_t llops_linattn_bwd(const llops_shape_t* s, const void* Q, const void* K,
                                 const void* V, const void* theta_q, const void* theta_k,
                                 const float* dO, float* dQ, float* dK, float* dV,
                                 float* dtheta_q, float* dtheta_k, void* ws, size_t ws_bytes,
                                 hipStream_t st) {
  return attn_backward(s, false, Q, K, V, theta_q, theta_k, dO, dQ, dK, dV, dtheta_q, dtheta_k, ws,
                       ws_bytes, st);
}

static llops_status_t gated_bwd_body(const llops_shape_t* s, const void* Q, const void* K,
                                     const void* V, const void* theta_q, const void* theta_k,
                                     const float* log_gate, const float* S0, const float* z0,
                                     const float* dO, float* dQ, float* dK, float* dV,
                                     float* dtheta_q, float* dtheta_k, float* dlog_gate,
                                     float* dS0, float* dz0, void* ws, size_t ws_bytes,
                                     hipStream_t st) {
  LLOPS_TRY(validate_gated_bwd(s));
  const int64_t BH = s->batch * s->heads;
  if (s->heads == 0) return LLOPS_OK;
  LLOPS_TRY(need(theta_q, "theta_q"));
  LLOPS_TRY(need(theta_k, "theta_k"));
  LLOPS_TRY(need(dtheta_q, "dtheta_q"));
  LLOPS_TRY(need(dtheta_k, "dtheta_k"));
  const int64_t R = BH * s->n;
  if (R > 0) {
    LLOPS_TRY(need(Q, "Q"));
    LLOPS_TRY(need(K, "K"));
    LLOPS_TRY(need(V, "V"));
    LLOPS_TRY(need4(log_gate, "log_gate"));
    LLOPS_TRY(need(dO, "dO"));
    LLOPS_TRY(need(dQ, "dQ"));
    LLOPS_TRY(need(dK, "dK"));
    LLOPS_TRY(need(dV, "dV"));
    LLOPS_TRY(need4(dlog_gate, "dlog_gate"));
  }
  LLOPS_TRY(opt(S0, "S0"));
  LLOPS_TRY(opt(z0, "z0"));
  LLOPS_TRY(opt(dS0, "dS0"));
  LLOPS_TRY(opt(dz0, "dz0"));
  const GBwdWs L = gated_bwd_ws(s);
  if (ws_bytes < L.total)
    return fail(LLOPS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  if (!ws) return fail(LLOPS_ERR_INVALID_ARG, "ws is null");
  LLOPS_TRY(opt(ws, "ws"));
  char* w = static_cast<char*>(ws);
  auto u16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(w + off); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  const llops::FeatShape fs0 = feat_shape(s, s->n, 0);
  float* fb = L.b.fb ? f32(L.b.fb) : nullptr;
  if (R == 0) {  // no rows: the Theta (and initial-state) gradients are zero
    LLOPS_HIP(llops::launch_featmap_bwd(fs0, Q, theta_q, dO, 0, dQ, dtheta_q, fb, st), "featmap_bwd");
    LLOPS_HIP(llops::launch_featmap_bwd(fs0, K, theta_k, dO, 0, dK, dtheta_k, fb, st), "featmap_bwd");
    if (dS0 || dz0)
      LLOPS_HIP(llops::launch_state_init(BH, s->m, s->dv, nullptr, nullptr, dS0, dz0, st),
                "state_init");
    return LLOPS_OK;
  }
  const int m = s->m, dv = s->dv, MA = bwd_ma(s), W = bwd_w(s);
  const int64_t n = s->n;
  uint16_t *phq = u16(L.b.phq), *phk = u16(L.b.phk);
  float *seg = f32(L.seg), *gseg = f32(L.gseg);
  llops::FeatJob jobs[2] = {{Q, theta_q, phq, w + L.b.pkq}, {K, theta_k, phk, w + L.b.pkk}};
  LLOPS_HIP(llops::launch_featmap_bf16(feat_shape(s, n, 1), jobs, 2, st), "featmap");
  // chunk-local gate sums, forward and (off the anti-causal path) for the
  // reversed sequence
  const bool anti = bwd_anti(s);
  float *glf = f32(L.glf), *grev = anti ? nullptr : f32(L.grev), *glr = anti ? nullptr : f32(L.glr);
  LLOPS_HIP(llops::launch_gate_cumsum32(BH, n, log_gate, glf, st), "gate_cumsum");
  if (!anti) {
    LLOPS_HIP(llops::launch_gate_reverse_shift(log_gate, n, R, grev, st), "gate_reverse");
    LLOPS_HIP(llops::launch_gate_cumsum32(BH, n, grev, glr, st), "gate_cumsum");
  }
  // num = M V and, normalised, M 1 per row from the same pass
  // unnormalised, dnum = dO and dden = 0: num is not formed
  float* num = s->normalize ? f32(L.b.num) : nullptr;
  const uint16_t* vv = static_cast<const uint16_t*>(V);
  float* den = nullptr;
  if (s->normalize) {
    den = f32(L.gden);
    LLOPS_HIP(gated_attn_num_den(s, phq, phk, vv, glf, num, den, seg, gseg, st, S0, z0),
              "attn num den");
  }
  uint16_t *a = u16(L.b.a), *b = u16(L.b.b), *dn = u16(L.b.rdnum);
  uint16_t *ra = anti ? nullptr : u16(L.b.ra), *rb = anti ? nullptr : u16(L.b.rb);
  // narrow chain-rule operands (as in the ungated backward) on the anti-causal
  // path of the m = 256, dv = 128 kernels, with phi read in place
  const llops_shape_t tMW0 = feat_attn_shape(s, MA, W);
  const bool aug = anti && n * m * 2 < (int64_t{1} << 31) && !bwd_padded() && dv % 8 == 0 &&
                   dv + 8 <= MA &&
                   llops::aug32_supported(attn_shape(&tMW0, true, kGatedBwdWG));
  if (aug)
    LLOPS_HIP(llops::launch_make_ab_aug(num, den, dO, dv, R, s->normalize,
                                        s->normalize ? s->delta : 0.f, a, dn, 1, st),
              "make_ab");
  else
    LLOPS_HIP(llops::launch_make_ab(num, den, dO, vv, dv, MA, n, R, s->normalize,
                                    s->normalize ? s->delta : 0.f, a, ra, b, rb, dn, anti ? 0 : 1,
                                    1, st),
              "make_ab");
  uint16_t* vp = u16(L.b.vp);
  float* tmp = f32(L.b.tmp);
  float* dc = f32(L.dc);
  uint16_t *dphq = u16(L.b.dphq), *dphk = u16(L.b.dphk);
  // dphi_Q_i = sum_{j<=i} exp(c_i - c_j) (a_i . b_j) phi_K_j; dc_i += phi_Q,i . dphi_Q,i.
  // The gate gradient at each segment start t0 is exact from states:
  // dg_t0 = <U_t0, P_t0-1> with P the pass's prefix state sum_{j<t0} (decayed to t0-1)
  // b_j phi_K,j^T and U_t0 = sum_{i>=t0} exp(c_i - c_{t0-1}) a_i phi_Q,i^T, summed
  // over the W-column slices; between segment starts the suffix sums of dc fill in.
  const llops_shape_t tMW = feat_attn_shape(s, MA, W);
  const llops::AttnShape aMW = attn_shape(&tMW, true, kGatedBwdWG);
  const int64_t perMW = static_cast<int64_t>(MA) * W + MA;
  float *seg2 = f32(L.seg2), *dgb = f32(L.dgb);
  const bool init = S0 || z0;
  // The passes read their phi slice in place (rows m apart; on the reversed
  // path the reversed sequence's from the reversed copy of phi_Q) unless phi
  // is too long for a 32-bit view, and dV is written in the original row order.
  const bool sliced = n * m * 2 < (int64_t{1} << 31);
  uint16_t *rphq = anti ? nullptr : u16(L.b.rphq), *rphk = anti ? nullptr : u16(L.b.rphk);
  if (!anti) {
    LLOPS_HIP(llops::launch_rows_copy_bf16(phq, m, 0, rphq, m, 0, m, n, R, 1, st), "rows");
    LLOPS_HIP(llops::launch_rows_copy_bf16(phk, m, 0, rphk, m, 0, m, n, R, 1, st), "rows");
  }
  for (int p0 = 0; p0 < m; p0 += W) {
    if (!sliced)
      LLOPS_HIP(llops::launch_rows_copy_bf16(phk, m, p0, vp, W, 0, W, n, R, 0, st), "rows");
    if (init)
      LLOPS_HIP(llops::launch_build_p0(S0, z0, BH, m, dv, MA, W, p0, f32(L.p0), st), "state");
    if (aug)
      LLOPS_HIP(gated_attn_on_aug(s, MA, W, a, dv + 8, 0, vv, dv, 1, phk + p0, m, glf, tmp, seg,
                                  gseg, st, init ? f32(L.p0) : nullptr),
                "attn dphi_q");
    else
      LLOPS_HIP(gated_attn_on_features(s, MA, W, a, b, sliced ? phk + p0 : vp, glf, tmp, seg, gseg,
                                       st, init ? f32(L.p0) : nullptr, sliced ? m : 0),
                "attn dphi_q");
    // dc_i += phi_Q,i . dphi_Q,i, and the slice of dphi_Q stored as bf16
    LLOPS_HIP(llops::launch_rowdot_acc(tmp, W, phq, m, p0, W, n, R, 0, 1.f, p0 == 0 ? 1 : 0, dc,
                                       st, dphq),
              "rowdot");
    if (aug) {
      LLOPS_HIP(llops::launch_seg_state32_gated_aug(aMW, a, dv + 8, 0, phq + p0, m, glf, gseg, seg2,
                                                    true, st),
                "anchored");
    } else if (sliced) {
      LLOPS_HIP(llops::launch_seg_state32_gated_v(aMW, a, phq + p0, m, glf, gseg, seg2, true, st),
                "anchored");
    } else {
      LLOPS_HIP(llops::launch_rows_copy_bf16(phq, m, p0, vp, W, 0, W, n, R, 0, st), "rows");
      LLOPS_HIP(llops::launch_seg_state32_anchored(aMW, a, vp, glf, gseg, seg2, st), "anchored");
    }
    LLOPS_HIP(llops::launch_seg_rscan_gated(BH, aMW.nseg, perMW, static_cast<int64_t>(MA) * W,
                                            seg2, gseg, st),
              "rscan");
    LLOPS_HIP(llops::launch_seg_dot(BH, aMW.nseg, perMW, static_cast<int64_t>(MA) * W, seg, seg2,
                                    p0 == 0 ? 1 : 0, dgb, st),
              "segdot");
    // segment 0's suffix state is sum_i exp(c_i) a_i phi_Q,i^T: [dS0^T; dz0^T] for this slice
    LLOPS_HIP(llops::launch_state_grad_slice(seg2, aMW.nseg, perMW, BH, m, dv, W, p0, dS0, dz0, st),
              "state grad");
    if (anti) {
      // dphi_K_j = sum_{i>=j} exp(c_i - c_j) (a_i . b_j) phi_Q_i for this slice: the
      // anti-causal pass starts each segment from the start-anchored suffix state
      // of the next one, which seg2 now holds; dc_j -= phi_K,j . dphi_K,j
      llops::AttnShape ga = aMW;
      ga.anti = 1;
      if (aug)
        LLOPS_HIP(llops::launch_attn_out32_gated_aug(ga, vv, dv, 1, a, dv + 8, 0, phq + p0, m, glf,
                                                     seg2, tmp, st),
                  "attn dphi_k");
      else
        LLOPS_HIP(llops::launch_attn_out32_gated_to(ga, b, a, phq + p0, glf, seg2, tmp, 0, m, st),
                  "attn dphi_k");
      LLOPS_HIP(llops::launch_rowdot_acc(tmp, W, phk, m, p0, W, n, R, 0, -1.f, 0, dc, st, dphk),
                "rowdot");
    }
  }
  // off the anti-causal path: dphi_K_j = sum_{i>=j} exp(c_i - c_j) (a_i . b_j)
  // phi_Q_i over the reversed sequence with its shifted gates; dc_j -= phi_K,j . dphi_K,j
  for (int p0 = 0; !anti && p0 < m; p0 += W) {
    if (!sliced)
      LLOPS_HIP(llops::launch_rows_copy_bf16(phq, m, p0, vp, W, 0, W, n, R, 1, st), "rows");
    LLOPS_HIP(gated_attn_on_features(s, MA, W, rb, ra, sliced ? rphq + p0 : vp, glr, tmp, seg,
                                     gseg, st, nullptr, sliced ? m : 0),
              "attn dphi_k");
    LLOPS_HIP(llops::launch_rowdot_acc(tmp, W, phk, m, p0, W, n, R, 1, -1.f, 0, dc, st, dphk),
              "rowdot");
  }
  // dV_j = sum_{i>=j} M_ij dnum_i: anti-causal from start-anchored suffix
  // states (state pass, reverse scan), or over the reversed sequence with
  // rows written back in the original order
  if (anti) {
    const llops_shape_t tmd = feat_attn_shape(s, m, dv);
    llops::AttnShape amd = attn_shape(&tmd, true, kGatedBwdWG);
    const int64_t permd = static_cast<int64_t>(m) * dv + m;
    LLOPS_HIP(llops::launch_seg_state32_anchored(amd, phq, dn, glf, gseg, seg, st), "anchored");
    LLOPS_HIP(llops::launch_seg_rscan_gated(BH, amd.nseg, permd, static_cast<int64_t>(m) * dv, seg,
                                            gseg, st),
              "rscan");
    amd.anti = 1;
    LLOPS_HIP(llops::launch_attn_out32_gated_to(amd, phk, phq, dn, glf, seg, dV, 0, 0, st),
              "attn dv");
  } else {
    LLOPS_HIP(gated_attn_on_features(s, m, dv, rphk, rphq, dn, glr, dV, seg, gseg, st, nullptr, 0,
                                     1),
              "attn dv");
  }
  // dlog_gate_l = sum_{i>=l} dc_i, anchored at the exact segment-start values
  LLOPS_HIP(llops::launch_seg_bridge_dg(dc, BH, n, aMW.seg_len, aMW.nseg, dgb, dlog_gate, st),
            "bridge");
  LLOPS_HIP(llops::launch_featmap_bwd(fs0, Q, theta_q, dphq, 1, dQ, dtheta_q, fb, st),
            "featmap_bwd q");
  LLOPS_HIP(llops::launch_featmap_bwd(fs0, K, theta_k, dphk, 1, dK, dtheta_k, fb, st),
            "featmap_bwd k");
  return LLOPS_OK;
}

llops_status_t llops_linattn_gated_causal_bwd(const llops_shape_t* s, const void* Q, const void* K,
                                              const void* V, const void* theta_q,
                                              const void* theta_k, const float* log_gate,
                                              const float* dO, float* dQ, float* dK, float* dV,
                                              float* dtheta_q, float* dtheta_k, float* dlog_gate,
                                              void* ws, size_t ws_bytes, hipStream_t st) {
  return gated_bwd_body(s, Q, K, V, theta_q, theta_k, log_gate, nullptr, nullptr, dO, dQ, dK, dV,
                        dtheta_q, dtheta_k, dlog_gate, nullptr, nullptr, ws, ws_bytes, st);
}

llops_status_t llops_linattn_gated_causal_bwd_state(
    const llops_shape_t* s, const void* Q, const void* K, const void* V, const void* theta_q,
    const void* theta_k, const float* log_gate, const float* S0, const float* z0, const float* dO,
    float* dQ, float* dK, float* dV, float* dtheta_q, float* dtheta_k, float* dlog_gate,
    float* dS0, float* dz0, void* ws, size_t ws_bytes, hipStream_t st) {
  return gated_bwd_body(s, Q, K, V, theta_q, theta_k, log_gate, S0, z0, dO, dQ, dK, dV, dtheta_q,
                        dtheta_k, dlog_gate, dS0, dz0, ws, ws_bytes, st);
}

static llops_status_t decode_impl(const llops_shape_t* s, const void* q, const void* k,
                                  const void* v, const void* theta_q, const void* theta_k,
                                  const float* log_gate, float* S, float* z, void* out, void* ws,
                                  size_t ws_bytes, hipStream_t st) {
  LLOPS_TRY(validate(s, LLOPS_ENTRY_DECODE));
  const int64_t BH = s->batch * s->heads;
  if (BH == 0) return LLOPS_OK;  // empty: pointers may be null
  LLOPS_TRY(need(q, "q"));
  LLOPS_TRY(need(k, "k"));
  LLOPS_TRY(need(v, "v"));
  LLOPS_TRY(need(theta_q, "theta_q"));
  LLOPS_TRY(need(theta_k, "theta_k"));
  LLOPS_TRY(need(S, "S"));
  LLOPS_TRY(need(z, "z"));
  LLOPS_TRY(need(out, "out"));
  if (log_gate) LLOPS_TRY(need4(log_gate, "log_gate"));
  const WsLayout L = ws_layout(s, LLOPS_ENTRY_DECODE);
  if (ws_bytes < L.total)
    return fail(LLOPS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  if (L.total && !ws) return fail(LLOPS_ERR_INVALID_ARG, "ws is null");
  if (ws) LLOPS_TRY(opt(ws, "ws"));
  char* w = static_cast<char*>(ws);
  float* fq = reinterpret_cast<float*>(w + L.phiq);
  float* fk = reinterpret_cast<float*>(w + L.phik);
  const llops::FeatShape fs = feat_shape(s, 1, 0);
  const bool packed = pack_bytes(s, 1) > 0;
  llops::FeatJob jobs[2] = {{q, theta_q, fq, packed ? w + L.pkq : nullptr},
                            {k, theta_k, fk, packed ? w + L.pkk : nullptr}};
  const bool bf16 = s->in_dtype == LLOPS_BF16;
  if (bf16)
    LLOPS_HIP(llops::launch_featmap_bf16(fs, jobs, 2, st), "featmap");
  else
    LLOPS_HIP(llops::launch_featmap_f32(fs, jobs, 2, st), "featmap");
  LLOPS_HIP(llops::launch_decode_state(BH, s->m, s->dv, fq, fk, v, bf16 ? 1 : 0, S, z,
                                       static_cast<float*>(out), s->normalize,
                                       s->normalize ? s->delta : 0.f, log_gate, st),
            "decode_state");
  return LLOPS_OK;
}

llops_status_t llops_decode_step(const llops_shape_t* s, const void* q, const void* k,
                                 const void* v, const void* theta_q, const void* theta_k, float* S,
                                 float* z, void* out, void* ws, size_t ws_bytes, hipStream_t st) {
  return decode_impl(s, q, k, v, theta_q, theta_k, nullptr, S, z, out, ws, ws_bytes, st);
}

llops_status_t llops_gated_decode_step(const llops_shape_t* s, const void* q, const void* k,
                                       const void* v, const void* theta_q, const void* theta_k,
                                       const float* log_gate, float* S, float* z, void* out,
                                       void* ws, size_t ws_bytes, hipStream_t st) {
  if (s && s->batch * s->heads > 0) LLOPS_TRY(need4(log_gate, "log_gate"));
  return decode_impl(s, q, k, v, theta_q, theta_k, log_gate, S, z, out, ws, ws_bytes, st);
}

}  // extern "C"

// ---- decode without a caller workspace --------------------------------------
// The scratch of llops_decode_step_noalloc (phi_q and phi_k, plus repacked
// Theta copies for batches above 1024 rows per head) lives in this static
// device array. Each GPU the library runs on holds its own copy for the life
// of the process; host code never uses the array's name as an address, only
// the per-device pointer that hipGetSymbolAddress returns for it.
constexpr size_t kNoAllocScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch's address on the device `stream` runs on, looked up once per
// device with that device current (then restored).
llops_status_t noalloc_scratch(hipStream_t st, void** out) {
  int cur = 0;
  LLOPS_HIP(hipGetDevice(&cur), "hipGetDevice");
  int dev = cur;
  if (st) LLOPS_HIP(hipStreamGetDevice(st, &dev), "hipStreamGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LLOPS_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table covers", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur) LLOPS_HIP(hipSetDevice(dev), "hipSetDevice");
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) LLOPS_HIP(hipSetDevice(cur), "hipSetDevice");
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(LLOPS_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LLOPS_OK;
}

}  // namespace

extern "C" {

llops_status_t llops_decode_step_noalloc(const llops_shape_t* s, const void* q, const void* k,
                                         const void* v, const void* theta_q, const void* theta_k,
                                         float* S, float* z, void* out, hipStream_t st) {
  LLOPS_TRY(validate(s, LLOPS_ENTRY_DECODE));
  const size_t need = ws_layout(s, LLOPS_ENTRY_DECODE).total;
  if (need > kNoAllocScratchBytes)
    return fail(LLOPS_ERR_UNSUPPORTED,
                "decode without a workspace: this shape needs %zu bytes of scratch, the static "
                "buffer holds %zu", need, kNoAllocScratchBytes);
  if (s->batch * s->heads == 0) return LLOPS_OK;
  void* ws = nullptr;
  LLOPS_TRY(noalloc_scratch(st, &ws));
  return decode_impl(s, q, k, v, theta_q, theta_k, nullptr, S, z, out, ws, kNoAllocScratchBytes,
                     st);
}

const char* llops_status_str(llops_status_t status) {
  switch (status) {
    case LLOPS_OK: return "LLOPS_OK";
    case LLOPS_ERR_INVALID_ARG: return "LLOPS_ERR_INVALID_ARG";
    case LLOPS_ERR_UNSUPPORTED: return "LLOPS_ERR_UNSUPPORTED";
    case LLOPS_ERR_WORKSPACE: return "LLOPS_ERR_WORKSPACE";
    case LLOPS_ERR_HIP: return "LLOPS_ERR_HIP";
    default: return "LLOPS_ERR_UNKNOWN";
  }
}

const char* llops_last_error(void) { return g_err; }

}  // extern "C"
