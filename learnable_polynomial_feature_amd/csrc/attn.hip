// Linear-attention contraction over precomputed LLoPS features.
//
//   non-causal: out = phi_Q (phi_K^T V) [/ (phi_Q (phi_K^T 1) + delta)]
//     (LLoPS notes, overall framework; low-rank-attention blog, Performer
//      section: associativity and the numerator/denominator form)
//   causal:     out_i = phi_Q,i S_i [/ (phi_Q,i z_i + delta)], S_i, z_i summed over j <= i
//     (LLoPS paper Sec. 1: streaming form with constant-size state; blog:
//      causal masking by incremental cumulative sums)
//
// Work decomposition (one GPU): every (batch, head) sequence is cut into
// `nseg` segments so that batch*heads*nseg workgroups fill the chip.
//   P1 seg_state: per segment, dS = phi_K^T V and dz = phi_K^T 1 (MFMA; dz via
//      a constant all-ones B fragment).
//   scan:         exclusive prefix of (dS, dz) over segments, seeded with
//                 (S0, z0); the total is the final state.
//   P2 attn_out:  per segment, walk blocks of C tokens: the masked block
//      A^T = phi_K phi_Q^T (MFMA) goes to LDS in bf16; the normaliser row sums
//      read the same rounded A; out = A V + phi_Q S on MFMA with S held in
//      fp32 accumulator registers (each wave owns dv/4 columns of S and feeds
//      them straight back as bf16 B fragments, k-permuted to match the
//      accumulator layout); then S += phi_K^T V, z += colsum(phi_K).
#include "device.h"
#include "kernels.h"

namespace llops {
namespace {

struct AttnArgs {
  int64_t BH, n;
  int m, dv, chunk, nseg;
  int64_t seg_len;
  int normalize;
  float delta;
};

AttnArgs to_args(const AttnShape& s) {
  AttnArgs a{};
  a.BH = s.BH;
  a.n = s.n;
  a.m = s.m;
  a.dv = s.dv;
  a.chunk = s.chunk;
  a.nseg = s.nseg;
  a.seg_len = s.seg_len;
  a.normalize = s.normalize;
  a.delta = s.delta;
  return a;
}

// Load an 8x8 bf16 block (rows r0..r0+7 of a row-major [rows][ld] matrix,
// columns c0..c0+7), zero-filling rows >= rmax.
__device__ __forceinline__ void load_block8(const uint16_t* base, int64_t ld, int64_t r0,
                                            int64_t rmax, int c0, u32x4 out[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r0 + i;
    out[i] = (r < rmax) ? ld16(base + r * ld + c0) : u32x4{0u, 0u, 0u, 0u};
  }
}

// ============================================================================
// P1: per-segment state partials, bf16 features
// ============================================================================
template <int MTW, int NT>
__global__ __launch_bounds__(256) void seg_state_bf16(AttnArgs a, const uint16_t* __restrict__ phik,
                                                      const uint16_t* __restrict__ v,
                                                      float* __restrict__ seg) {
  constexpr int TB = 64;        // tokens per stage (two 32-wide k-steps)
  constexpr int LROW = TB + 8;  // padded row of the transposed stage
  extern __shared__ __align__(16) uint16_t smem[];
  const int m = a.m, dv = NT * 16;
  uint16_t* KT = smem;             // [m][LROW]   phi_K^T
  uint16_t* VT = smem + m * LROW;  // [dv][LROW]  V^T
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: MFMAs under a condition on it must branch, not
  // be masked through EXEC (an MFMA runs for the whole wave regardless)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t bh = blockIdx.y;
  const int gseg = blockIdx.x;
  const int64_t t0 = gseg * a.seg_len;
  const int64_t t1 = min(a.n, t0 + a.seg_len);
  const uint16_t* K = phik + bh * a.n * m;
  const uint16_t* Vb = v + bh * a.n * dv;
  const int MT = m / 16;

  f32x4 acc[MTW][NT + 1];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int c = 0; c <= NT; ++c) acc[i][c] = zero4();
  const bf16x8 ones = as_bf16x8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  const int nkb = (TB / 8) * (m / 8), nvb = (TB / 8) * (dv / 8);
  for (int64_t tb = t0; tb < t1; tb += TB) {
    __syncthreads();
    for (int sb = tid; sb < nkb + nvb; sb += 256) {
      u32x4 blk[8], tr[8];
      if (sb < nkb) {
        const int jb = sb / (m / 8), f8 = sb - jb * (m / 8);
        load_block8(K, m, tb + jb * 8, t1, f8 * 8, blk);
        transpose8x8(blk, tr);
#pragma unroll
        for (int e = 0; e < 8; ++e) st16(KT + (f8 * 8 + e) * LROW + jb * 8, tr[e]);
      } else {
        const int s2 = sb - nkb;
        const int jb = s2 / (dv / 8), c8 = s2 - jb * (dv / 8);
        load_block8(Vb, dv, tb + jb * 8, t1, c8 * 8, blk);
        transpose8x8(blk, tr);
#pragma unroll
        for (int e = 0; e < 8; ++e) st16(VT + (c8 * 8 + e) * LROW + jb * 8, tr[e]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int rt = w + 4 * i;
      if (rt >= MT) continue;
#pragma unroll
      for (int ks = 0; ks < TB / 32; ++ks) {
        const bf16x8 af = as_bf16x8(ld16(KT + (rt * 16 + c16) * LROW + ks * 32 + g * 8));
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          const bf16x8 bf = as_bf16x8(ld16(VT + (ct * 16 + c16) * LROW + ks * 32 + g * 8));
          acc[i][ct] = mfma16x16x32(af, bf, acc[i][ct]);
        }
        acc[i][NT] = mfma16x16x32(af, ones, acc[i][NT]);
      }
    }
  }
  float* out = seg + (bh * a.nseg + gseg) * (static_cast<int64_t>(m) * dv + m);
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    const int rt = w + 4 * i;
    if (rt >= MT) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int f = rt * 16 + g * 4 + e;
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) out[f * dv + ct * 16 + c16] = acc[i][ct][e];
      if (c16 == 0) out[m * dv + f] = acc[i][NT][e];
    }
  }
}

// ============================================================================
// Segment scan (any dtype: state is fp32)
// ============================================================================
__global__ __launch_bounds__(256) void seg_scan_kernel(int nseg, int m, int dv,
                                                       float* __restrict__ seg,
                                                       const float* S0, const float* z0,
                                                       float* Sout, int64_t Sout_bh,
                                                       float* zout, int64_t zout_bh,
                                                       int exclusive,
                                                       const float* __restrict__ gseg,
                                                       int reverse) {
  const int64_t per = static_cast<int64_t>(m) * dv + m;
  const int64_t mdv = static_cast<int64_t>(m) * dv;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (e >= per) return;
  float acc = 0.f;
  if (e < mdv) {
    if (S0) acc = S0[bh * mdv + e];
  } else {
    if (z0) acc = z0[bh * m + (e - mdv)];
  }
  // reverse: from the last segment back to the first (suffix sums)
  const int64_t step = reverse ? -per : per;
  float* p = seg + bh * nseg * per + e + (reverse ? (nseg - 1) * per : 0);
  if (gseg) {  // gated: the prefix decays through each segment before its own sum is added
    const float* gs = gseg + bh * nseg;
    for (int gi = 0; gi < nseg; ++gi, p += step) {
      const float x = *p;
      if (exclusive) *p = acc;
      acc = fmaf(__expf(gs[gi]), acc, x);
    }
  } else {
    for (int gi = 0; gi < nseg; ++gi, p += step) {
      const float x = *p;
      if (exclusive) *p = acc;
      acc += x;
    }
  }
  if (e < mdv) {
    if (Sout) Sout[bh * Sout_bh + e] = acc;
  } else {
    if (zout) zout[bh * zout_bh + (e - mdv)] = acc;
  }
}

// ============================================================================
// P2: output pass, bf16 features
// ============================================================================
template <int C, int MTM, int NTW, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_out_bf16(AttnArgs a, const uint16_t* __restrict__ phiq,
                                                     const uint16_t* __restrict__ phik,
                                                     const uint16_t* __restrict__ v,
                                                     const float* __restrict__ state,
                                                     int64_t st_seg, int64_t st_bh,
                                                     float* __restrict__ out) {
  constexpr int CROW = C + 8;
  constexpr int CT = C / 16;
  extern __shared__ __align__(16) uint16_t smem[];
  const int m = a.m, dv = a.dv;
  const int MROW = m + 8;
  const int MT = m / 16, NT = dv / 16;
  uint16_t* Qs = smem;                  // [C][MROW]
  uint16_t* Ks = Qs + C * MROW;         // [C][MROW]
  uint16_t* KT = Ks + C * MROW;         // [m][CROW]
  uint16_t* VT = KT + m * CROW;         // [dv][CROW]
  uint16_t* As = VT + dv * CROW;        // [C][CROW]  A[i][j] (query i, key j)
  float* zs = reinterpret_cast<float*>(As + C * CROW);  // [m]
  float* dens = zs + m;                                 // [C]  1 / (den + delta)

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: MFMAs under a condition on it must branch, not
  // be masked through EXEC (an MFMA runs for the whole wave regardless)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t bh = blockIdx.y;
  const int gseg = blockIdx.x;
  const int64_t t0 = gseg * a.seg_len;
  const int64_t t1 = min(a.n, t0 + a.seg_len);
  const uint16_t* Qg = phiq + bh * a.n * m;
  const uint16_t* Kg = phik + bh * a.n * m;
  const uint16_t* Vg = v + bh * a.n * dv;
  float* Og = out + bh * a.n * dv;
  const float* Sin = state + bh * st_bh + gseg * st_seg;

  // S columns owned by this wave: ct = w + 4*i
  f32x4 S[MTM][NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int ct = w + 4 * i;
#pragma unroll
    for (int rt = 0; rt < MTM; ++rt) {
      f32x4 x = zero4();
      if (rt < MT && ct < NT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = Sin[(rt * 16 + g * 4 + e) * dv + ct * 16 + c16];
      }
      S[rt][i] = x;
    }
  }
  for (int f = tid; f < m; f += 256) zs[f] = Sin[m * dv + f];

  const int nqb = (C / 8) * (m / 8), nvb = (C / 8) * (dv / 8);
  for (int64_t c0 = t0; c0 < t1; c0 += C) {
    // ---- stage phi_Q, phi_K (natural and transposed) and V^T
    // non-causal blocks only need phi_Q (S and z are the totals)
    const int nstage = CAUSAL ? 2 * nqb + nvb : nqb;
    for (int sb = tid; sb < nstage; sb += 256) {
      u32x4 blk[8], tr[8];
      if (sb < nqb) {
        const int jb = sb / (m / 8), f8 = sb - jb * (m / 8);
        load_block8(Qg, m, c0 + jb * 8, t1, f8 * 8, blk);
#pragma unroll
        for (int e = 0; e < 8; ++e) st16(Qs + (jb * 8 + e) * MROW + f8 * 8, blk[e]);
      } else if (sb < 2 * nqb) {
        const int s2 = sb - nqb;
        const int jb = s2 / (m / 8), f8 = s2 - jb * (m / 8);
        load_block8(Kg, m, c0 + jb * 8, t1, f8 * 8, blk);
#pragma unroll
        for (int e = 0; e < 8; ++e) st16(Ks + (jb * 8 + e) * MROW + f8 * 8, blk[e]);
        transpose8x8(blk, tr);
#pragma unroll
        for (int e = 0; e < 8; ++e) st16(KT + (f8 * 8 + e) * CROW + jb * 8, tr[e]);
      } else {
        const int s2 = sb - 2 * nqb;
        const int jb = s2 / (dv / 8), c8 = s2 - jb * (dv / 8);
        load_block8(Vg, dv, c0 + jb * 8, t1, c8 * 8, blk);
        transpose8x8(blk, tr);
#pragma unroll
        for (int e = 0; e < 8; ++e) st16(VT + (c8 * 8 + e) * CROW + jb * 8, tr[e]);
      }
    }
    __syncthreads();

    if (CAUSAL) {
      // ---- masked A^T tiles (key rows j, query columns i), j <= i kept
      for (int k = w; k < CT * CT; k += 4) {
        const int jt = k / CT, it = k - jt * CT;
        f32x4 acc = zero4();
        if (jt <= it) {
          const uint16_t* arow = Ks + (jt * 16 + c16) * MROW + g * 8;
          const uint16_t* brow = Qs + (it * 16 + c16) * MROW + g * 8;
          for (int kq = 0; kq < m / 32; ++kq)
            acc = mfma16x16x32(as_bf16x8(ld16(arow + kq * 32)), as_bf16x8(ld16(brow + kq * 32)), acc);
          if (jt == it) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (g * 4 + e > c16) acc[e] = 0.f;
          }
        }
        const uint32_t lo = pack_bf16x2(acc[0], acc[1]), hi = pack_bf16x2(acc[2], acc[3]);
        *reinterpret_cast<u32x2*>(As + (it * 16 + c16) * CROW + jt * 16 + g * 4) = u32x2{lo, hi};
      }
      __syncthreads();
    }

    // ---- normaliser: dens[i] = 1 / (sum_j A[i][j] + phi_Q[i] . z + delta)
    if (a.normalize) {
      constexpr int TPR = 256 / C;  // threads per row (4 or 8)
      const int i = tid / TPR, q = tid - i * TPR;
      float s = 0.f;
      if (CAUSAL)
        for (int j = q; j < C; j += TPR) s += bf16_to_f32(As[i * CROW + j]);
      for (int f = q; f < m; f += TPR) s += bf16_to_f32(Qs[i * MROW + f]) * zs[f];
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) s += __shfl_xor(s, o);
      if (q == 0) dens[i] = 1.f / (s + a.delta);
      __syncthreads();
    }

    // ---- out = A V + phi_Q S  (rows of this block, this wave's columns)
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int ct = w + 4 * i;
      if (ct >= NT) continue;
      for (int it = 0; it < CT; ++it) {
        f32x4 acc = zero4();
        if (CAUSAL) {
#pragma unroll
          for (int ks = 0; ks < C / 32; ++ks) {
            if (ks * 32 > it * 16 + 15) continue;  // keys beyond this query block are masked
            const bf16x8 af = as_bf16x8(ld16(As + (it * 16 + c16) * CROW + ks * 32 + g * 8));
            const bf16x8 bf = as_bf16x8(ld16(VT + (ct * 16 + c16) * CROW + ks * 32 + g * 8));
            acc = mfma16x16x32(af, bf, acc);
          }
        }
        const uint16_t* qrow = Qs + (it * 16 + c16) * MROW + g * 4;
#pragma unroll
        for (int kq = 0; kq < MTM / 2; ++kq) {
          if (2 * kq >= MT) continue;
          const u32x2 q0 = *reinterpret_cast<const u32x2*>(qrow + kq * 32);
          const u32x2 q1 = *reinterpret_cast<const u32x2*>(qrow + kq * 32 + 16);
          const bf16x8 af = as_bf16x8(u32x4{q0[0], q0[1], q1[0], q1[1]});
          const f32x4 s0 = S[2 * kq][i], s1 = S[2 * kq + 1][i];
          const bf16x8 bf = as_bf16x8(u32x4{pack_bf16x2(s0[0], s0[1]), pack_bf16x2(s0[2], s0[3]),
                                            pack_bf16x2(s1[0], s1[1]), pack_bf16x2(s1[2], s1[3])});
          acc = mfma16x16x32(af, bf, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = it * 16 + g * 4 + e;
          const int64_t tok = c0 + r;
          if (tok < t1) {
            const float val = a.normalize ? acc[e] * dens[r] : acc[e];
            Og[tok * dv + ct * 16 + c16] = val;
          }
        }
      }
    }

    if (CAUSAL) {
      // ---- S += phi_K^T V for this wave's columns
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        const int ct = w + 4 * i;
        if (ct >= NT) continue;
#pragma unroll
        for (int ks = 0; ks < C / 32; ++ks) {
          const bf16x8 bf = as_bf16x8(ld16(VT + (ct * 16 + c16) * CROW + ks * 32 + g * 8));
#pragma unroll
          for (int rt = 0; rt < MTM; ++rt) {
            if (rt >= MT) continue;
            const bf16x8 af = as_bf16x8(ld16(KT + (rt * 16 + c16) * CROW + ks * 32 + g * 8));
            S[rt][i] = mfma16x16x32(af, bf, S[rt][i]);
          }
        }
      }
      // ---- z += column sums of phi_K (after the normaliser read z)
      for (int f = tid; f < m; f += 256) {
        float s = 0.f;
        for (int j = 0; j < C; ++j) s += bf16_to_f32(Ks[j * MROW + f]);
        zs[f] += s;
      }
    }
    __syncthreads();
  }
}

// ============================================================================
// fp32 SIMT versions (fp32 inputs: exact-arithmetic reference-grade path)
// ============================================================================
__global__ __launch_bounds__(256) void seg_state_f32(AttnArgs a, const float* __restrict__ phik,
                                                     const float* __restrict__ v,
                                                     float* __restrict__ seg) {
  const int m = a.m, dv = a.dv;
  const int64_t bh = blockIdx.y;
  const int gseg = blockIdx.x;
  const int64_t t0 = gseg * a.seg_len;
  const int64_t t1 = min(a.n, t0 + a.seg_len);
  const float* K = phik + bh * a.n * m;
  const float* V = v + bh * a.n * dv;
  const int64_t per = static_cast<int64_t>(m) * dv + m;
  float* out = seg + (bh * a.nseg + gseg) * per;
  for (int64_t e = threadIdx.x; e < per; e += 256) {
    float s = 0.f;
    if (e < static_cast<int64_t>(m) * dv) {
      const int f = static_cast<int>(e / dv), c = static_cast<int>(e - static_cast<int64_t>(f) * dv);
      for (int64_t j = t0; j < t1; ++j) s = fmaf(K[j * m + f], V[j * dv + c], s);
    } else {
      const int f = static_cast<int>(e - static_cast<int64_t>(m) * dv);
      for (int64_t j = t0; j < t1; ++j) s += K[j * m + f];
    }
    out[e] = s;
  }
}

// Small non-causal fp32 problems in one launch: one workgroup of 512 threads
// per (b, h) sequence computes phi_K tile by tile, accumulates the state
// [S | z], then phi_Q tile by tile and the read-out (paper Sec. 1: S =
// phi_K^T V, z = phi_K^T 1, out = phi_Q S / (phi_Q z + delta)). Four launches
// (feature map, segment states, scan, output) cost more than the whole
// problem at these sizes. (d, m, p, t) are compile-time so every loop
// unrolls and LDS reads pipeline. Work goes in 4-wide groups (float4 through
// LDS): (row, 4 features) for phi, (feature, column group, row quarter) for
// the state, (row, column group) for the output; the value tile carries an
// extra [1 0 0 0] column group, so z and phi_Q z come out as one more group.
// The state is summed per tile (its row quarters first), then into the
// running sum: short chains keep the fp32 rounding near that of the
// segment passes.
constexpr int kSmallTR = 256;  // rows per tile
constexpr int kSmallNT = 512;  // threads per workgroup

struct SmallArgs {
  const float* Q;
  const float* K;
  const float* V;
  const float* tq;  // [H'][p][t][d][m]
  const float* tk;
  float* out;
  int64_t H, n;
  int dv;
  int64_t th_hstride;  // elements between heads' Theta (0 = shared)
  int square, normalize;
  float delta;
};

__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st_f4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void fma4(float a, const float4& b, float4& c) {
  c.x = fmaf(a, b.x, c.x);
  c.y = fmaf(a, b.y, c.y);
  c.z = fmaf(a, b.z, c.z);
  c.w = fmaf(a, b.w, c.w);
}

template <int D, int M, int P, int T>
struct SmallGeom {
  static constexpr int PTDM = P * T * D * M;
  // LDS floats for value width dv: Theta_K, Theta_Q, [S | z] (M x W), X and
  // the value tile, phi, per-quarter state partials, denominators
  static constexpr int64_t floats(int dv) {
    return 2LL * PTDM + M * (dv + 4) + kSmallTR * (D + (dv + 4) + M + 1) + 4LL * M * (dv + 4);
  }
};

template <int D, int M, int P, int T>
__global__ __launch_bounds__(kSmallNT) void linattn_small_f32(SmallArgs a) {
  using G = SmallGeom<D, M, P, T>;
  constexpr int PTDM = G::PTDM, D4 = D / 4, M4 = M / 4, TR = kSmallTR, NT = kSmallNT;
  static_assert(D % 4 == 0 && M % 4 == 0, "4-wide groups");
  extern __shared__ __align__(16) float sm[];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t h = bh % a.H;
  const int dv = a.dv, W = dv + 4, W4 = W / 4, V4 = dv / 4;
  float* thk = sm;
  float* thq = thk + PTDM;
  float* Sa = thq + PTDM;             // M x W
  float* X = Sa + M * W;              // TR x D
  float* Va = X + TR * D;             // TR x W
  float* ph = Va + TR * W;            // TR x M
  float* den = ph + TR * M;           // TR
  float* part = den + TR;             // 4 x M x W
  const float* gk = a.tk + h * a.th_hstride;
  const float* gq = a.tq + h * a.th_hstride;
  for (int i = tid; i < PTDM / 4; i += NT) {
    st_f4(thk + 4 * i, ld_f4(gk + 4 * i));
    st_f4(thq + 4 * i, ld_f4(gq + 4 * i));
  }
  const int64_t n = a.n;
  const float* Kb = a.K + bh * n * D;
  const float* Qb = a.Q + bh * n * D;
  const float* Vb = a.V + bh * n * dv;
  float* Ob = a.out + bh * n * dv;
  const int nt = static_cast<int>((n + TR - 1) / TR);
  auto rows_of = [&](int tile) {
    return static_cast<int>(min(static_cast<int64_t>(TR), n - static_cast<int64_t>(tile) * TR));
  };
  // A tile's rows travel through registers one tile ahead: this thread's
  // pieces tid + NT q of X (TR*D4 <= 2 NT) and of the value tile (K tiles;
  // TR*W4 <= 3 NT).
  static_assert(TR * D4 <= 2 * NT, "two X pieces per thread");
  float4 xp[2], vp[3];
#pragma unroll
  for (int q = 0; q < 2; ++q) xp[q] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int q = 0; q < 3; ++q) vp[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fetch = [&](const float* src, int tile, bool values) {
    const int64_t r0 = static_cast<int64_t>(tile) * TR;
    const int rows = rows_of(tile);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = tid + NT * q;
      if (i < TR * D4) {
        const int row = i / D4, k4 = i - row * D4;
        xp[q] = row < rows ? ld_f4(src + (r0 + row) * D + 4 * k4) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    if (values) {
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const int i = tid + NT * q;
        if (i < TR * W4) {
          const int row = i / W4, c4 = i - row * W4;
          vp[q] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (row < rows)
            vp[q] = c4 < V4 ? ld_f4(Vb + (r0 + row) * dv + 4 * c4) : make_float4(1.f, 0.f, 0.f, 0.f);
        }
      }
    }
  };
  auto place = [&](bool values) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (tid + NT * q < TR * D4) st_f4(X + 4 * (tid + NT * q), xp[q]);
    if (values) {
#pragma unroll
      for (int q = 0; q < 3; ++q)
        if (tid + NT * q < TR * W4) st_f4(Va + 4 * (tid + NT * q), vp[q]);
    }
  };
  // phi of the tile's rows with Theta th: thread = (4 rows, features
  // 4q .. 4q+3), so each Theta read from LDS serves four rows
  constexpr int PR = 2;  // rows per thread
  static_assert(TR % PR == 0, "whole row groups");
  auto phi_tile = [&](const float* th, int rows) {
    for (int gi = tid; gi < (TR / PR) * M4; gi += NT) {
      const int rb = gi / M4, f = (gi - rb * M4) * 4, row0 = rb * PR;
      float xr[PR][D];  // this thread's rows, held for all (j, r)
#pragma unroll
      for (int i = 0; i < PR; ++i)
#pragma unroll
        for (int k4 = 0; k4 < D4; ++k4) {
          const float4 x = ld_f4(X + (row0 + i) * D + 4 * k4);
          xr[i][4 * k4] = x.x;
          xr[i][4 * k4 + 1] = x.y;
          xr[i][4 * k4 + 2] = x.z;
          xr[i][4 * k4 + 3] = x.w;
        }
      float4 acc[PR];
#pragma unroll
      for (int i = 0; i < PR; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 1
      for (int r = 0; r < T; ++r) {
        float4 prod[PR];
#pragma unroll
        for (int j = 0; j < P; ++j) {
          const float* tb = th + (j * T + r) * D * M + f;
          float4 y[PR];
#pragma unroll
          for (int i = 0; i < PR; ++i) y[i] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int k = 0; k < D; ++k) {
            const float4 w = ld_f4(tb + k * M);
#pragma unroll
            for (int i = 0; i < PR; ++i) fma4(xr[i][k], w, y[i]);
          }
#pragma unroll
          for (int i = 0; i < PR; ++i) {
            if (j == 0) {
              prod[i] = y[i];
            } else {
              prod[i].x *= y[i].x;
              prod[i].y *= y[i].y;
              prod[i].z *= y[i].z;
              prod[i].w *= y[i].w;
            }
          }
        }
#pragma unroll
        for (int i = 0; i < PR; ++i) {
          acc[i].x += prod[i].x;
          acc[i].y += prod[i].y;
          acc[i].z += prod[i].z;
          acc[i].w += prod[i].w;
        }
      }
#pragma unroll
      for (int i = 0; i < PR; ++i) {
        float4 v = acc[i];
        if (a.square) {
          v.x *= v.x;
          v.y *= v.y;
          v.z *= v.z;
          v.w *= v.w;
        }
        if (row0 + i >= rows) v = make_float4(0.f, 0.f, 0.f, 0.f);
        st_f4(ph + (row0 + i) * M + f, v);
      }
    }
  };
  __syncthreads();
  // state: thread = (group (feature, column group), row quarter); the
  // quarters' sums are added in a fixed order into the running sum
  const int SG = M * W4;
  static_assert(TR % 4 == 0, "row quarters");
  float4 sacc = make_float4(0.f, 0.f, 0.f, 0.f);  // threads tid < SG own group tid
  fetch(Kb, 0, true);
  for (int tile = 0; tile < nt; ++tile) {
    const int rows = rows_of(tile);
    place(true);
    __syncthreads();
    // the next tile (or the first query tile) is in flight while this one runs
    if (tile + 1 < nt)
      fetch(Kb, tile + 1, true);
    else
      fetch(Qb, 0, false);
    phi_tile(thk, rows);
    __syncthreads();
    for (int u = tid; u < 4 * SG; u += NT) {
      const int qr = u / SG, g = u - qr * SG, f = g / W4, c4 = g - f * W4;
      float4 ps = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
      for (int row = qr * (TR / 4); row < (qr + 1) * (TR / 4); ++row)
        fma4(ph[row * M + f], ld_f4(Va + row * W + 4 * c4), ps);
      st_f4(part + 4 * u, ps);
    }
    __syncthreads();
    if (tid < SG) {
      float4 t = ld_f4(part + 4 * tid);
#pragma unroll
      for (int qr = 1; qr < 4; ++qr) {
        const float4 v = ld_f4(part + 4 * (qr * SG + tid));
        t.x += v.x;
        t.y += v.y;
        t.z += v.z;
        t.w += v.w;
      }
      sacc.x += t.x;
      sacc.y += t.y;
      sacc.z += t.z;
      sacc.w += t.w;
    }
  }
  if (tid < SG) st_f4(Sa + (tid / W4) * W + 4 * (tid % W4), sacc);
  __syncthreads();
  // read-out: thread = (row, column group); the last column group is phi_Q z
  for (int tile = 0; tile < nt; ++tile) {
    const int64_t r0 = static_cast<int64_t>(tile) * TR;
    const int rows = rows_of(tile);
    place(false);
    __syncthreads();
    if (tile + 1 < nt) fetch(Qb, tile + 1, false);
    phi_tile(thq, rows);
    __syncthreads();
    float4 o[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      o[q] = make_float4(0.f, 0.f, 0.f, 0.f);
      const int g = tid + NT * q;
      if (g < TR * W4) {
        const int row = g / W4, c4 = g - row * W4;
#pragma unroll 8
        for (int f = 0; f < M; ++f) fma4(ph[row * M + f], ld_f4(Sa + f * W + 4 * c4), o[q]);
        if (c4 == V4) den[row] = o[q].x + a.delta;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int g = tid + NT * q;
      if (g < TR * W4) {
        const int row = g / W4, c4 = g - row * W4;
        if (row < rows && c4 < V4) {
          float4 v = o[q];
          if (a.normalize) {
            const float dd = den[row];
            v.x /= dd;
            v.y /= dd;
            v.z /= dd;
            v.w /= dd;
          }
          st_f4(Ob + (r0 + row) * dv + 4 * c4, v);
        }
      }
    }
    __syncthreads();
  }
}

template <bool CAUSAL>
__global__ __launch_bounds__(256) void attn_out_f32(AttnArgs a, const float* __restrict__ phiq,
                                                    const float* __restrict__ phik,
                                                    const float* __restrict__ v,
                                                    float* __restrict__ state, int64_t st_seg,
                                                    int64_t st_bh, float* __restrict__ out) {
  extern __shared__ float fsm[];
  const int C = a.chunk;
  float* A = fsm;          // [C][C]
  float* den = A + C * C;  // [C]
  const int m = a.m, dv = a.dv;
  const int64_t bh = blockIdx.y;
  const int gseg = blockIdx.x;
  const int64_t t0 = gseg * a.seg_len;
  const int64_t t1 = min(a.n, t0 + a.seg_len);
  const float* Q = phiq + bh * a.n * m;
  const float* K = phik + bh * a.n * m;
  const float* V = v + bh * a.n * dv;
  float* O = out + bh * a.n * dv;
  float* S = state + bh * st_bh + gseg * st_seg;  // [m][dv] then z [m]
  float* z = S + static_cast<int64_t>(m) * dv;
  const int tid = threadIdx.x;
  for (int64_t c0 = t0; c0 < t1; c0 += C) {
    const int nc = static_cast<int>(min<int64_t>(C, t1 - c0));
    if (CAUSAL) {
      for (int e = tid; e < C * C; e += 256) {
        const int i = e / C, j = e - i * C;
        float s = 0.f;
        if (j <= i && i < nc)
          for (int f = 0; f < m; ++f) s = fmaf(Q[(c0 + i) * m + f], K[(c0 + j) * m + f], s);
        A[e] = s;
      }
      __syncthreads();
    }
    if (a.normalize) {
      for (int i = tid; i < nc; i += 256) {
        float s = 0.f;
        if (CAUSAL)
          for (int j = 0; j <= i; ++j) s += A[i * C + j];
        for (int f = 0; f < m; ++f) s = fmaf(Q[(c0 + i) * m + f], z[f], s);
        den[i] = s + a.delta;
      }
      __syncthreads();
    }
    for (int e = tid; e < nc * dv; e += 256) {
      const int i = e / dv, c = e - i * dv;
      float s = 0.f;
      if (CAUSAL)
        for (int j = 0; j <= i; ++j) s = fmaf(A[i * C + j], V[(c0 + j) * dv + c], s);
      for (int f = 0; f < m; ++f) s = fmaf(Q[(c0 + i) * m + f], S[f * dv + c], s);
      O[(c0 + i) * dv + c] = a.normalize ? s / den[i] : s;
    }
    if (CAUSAL) {
      __syncthreads();
      const int64_t per = static_cast<int64_t>(m) * dv + m;
      for (int64_t e = tid; e < per; e += 256) {
        if (e < static_cast<int64_t>(m) * dv) {
          const int f = static_cast<int>(e / dv), c = static_cast<int>(e - static_cast<int64_t>(f) * dv);
          float s = S[e];
          for (int j = 0; j < nc; ++j) s = fmaf(K[(c0 + j) * m + f], V[(c0 + j) * dv + c], s);
          S[e] = s;
        } else {
          const int f = static_cast<int>(e - static_cast<int64_t>(m) * dv);
          float s = z[f];
          for (int j = 0; j < nc; ++j) s += K[(c0 + j) * m + f];
          z[f] = s;
        }
      }
    }
    __syncthreads();
  }
}

// Gated fp32 passes: the state decays by exp(g_j) before token j is added
// (a per-token scalar forgetting gate: the LLoPS notes, limitations and
// outlook). Pass 1 runs the recurrence S = exp(g_j) S + phi_K,j v_j^T over
// its segment and writes the segment's sum of g; the output pass walks
// chunks with chunk-local inclusive gate sums L (every exponent <= 0 for
// g <= 0): A_ij = exp(L_i - L_j) phi_Q,i . phi_K,j (j <= i), the carried
// state weighted by exp(L_i), and S = exp(T) S + sum_j exp(T - L_j) phi_K,j v_j^T.
__global__ __launch_bounds__(256) void seg_state_f32_gated(AttnArgs a, const float* __restrict__ phik,
                                                           const float* __restrict__ v,
                                                           const float* __restrict__ lg,
                                                           float* __restrict__ gseg,
                                                           float* __restrict__ seg) {
  const int m = a.m, dv = a.dv;
  const int64_t bh = blockIdx.y;
  const int gs = blockIdx.x;
  const int64_t t0 = gs * a.seg_len;
  const int64_t t1 = min(a.n, t0 + a.seg_len);
  const float* K = phik + bh * a.n * m;
  const float* V = v + bh * a.n * dv;
  const float* G = lg + bh * a.n;
  const int64_t per = static_cast<int64_t>(m) * dv + m;
  float* out = seg + (bh * a.nseg + gs) * per;
  for (int64_t e = threadIdx.x; e < per; e += 256) {
    float s = 0.f;
    if (e < static_cast<int64_t>(m) * dv) {
      const int f = static_cast<int>(e / dv), c = static_cast<int>(e - static_cast<int64_t>(f) * dv);
      for (int64_t j = t0; j < t1; ++j) s = fmaf(K[j * m + f], V[j * dv + c], expf(G[j]) * s);
    } else {
      const int f = static_cast<int>(e - static_cast<int64_t>(m) * dv);
      for (int64_t j = t0; j < t1; ++j) s = fmaf(expf(G[j]), s, K[j * m + f]);
    }
    out[e] = s;
  }
  if (threadIdx.x == 0) {
    float tot = 0.f;
    for (int64_t j = t0; j < t1; ++j) tot += G[j];
    gseg[bh * a.nseg + gs] = tot;
  }
}

__global__ __launch_bounds__(256) void attn_out_f32_gated(AttnArgs a, const float* __restrict__ phiq,
                                                          const float* __restrict__ phik,
                                                          const float* __restrict__ v,
                                                          const float* __restrict__ lg,
                                                          float* __restrict__ state,
                                                          float* __restrict__ out) {
  extern __shared__ float fsm[];
  const int C = a.chunk;
  float* A = fsm;          // [C][C]
  float* den = A + C * C;  // [C]
  float* L = den + C;      // [C] chunk-local inclusive gate sums
  const int m = a.m, dv = a.dv;
  const int64_t bh = blockIdx.y;
  const int gs = blockIdx.x;
  const int64_t t0 = gs * a.seg_len;
  const int64_t t1 = min(a.n, t0 + a.seg_len);
  const float* Q = phiq + bh * a.n * m;
  const float* K = phik + bh * a.n * m;
  const float* V = v + bh * a.n * dv;
  const float* G = lg + bh * a.n;
  float* O = out + bh * a.n * dv;
  const int64_t per = static_cast<int64_t>(m) * dv + m;
  float* S = state + (bh * a.nseg + gs) * per;  // [m][dv] then z [m]
  float* z = S + static_cast<int64_t>(m) * dv;
  const int tid = threadIdx.x;
  for (int64_t c0 = t0; c0 < t1; c0 += C) {
    const int nc = static_cast<int>(min<int64_t>(C, t1 - c0));
    if (tid == 0) {
      float acc = 0.f;
      for (int i = 0; i < nc; ++i) {
        acc += G[c0 + i];
        L[i] = acc;
      }
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += 256) {
      const int i = e / C, j = e - i * C;
      float s = 0.f;
      if (j <= i && i < nc) {
        for (int f = 0; f < m; ++f) s = fmaf(Q[(c0 + i) * m + f], K[(c0 + j) * m + f], s);
        s *= expf(L[i] - L[j]);
      }
      A[e] = s;
    }
    __syncthreads();
    if (a.normalize) {
      for (int i = tid; i < nc; i += 256) {
        float s = 0.f, qz = 0.f;
        for (int j = 0; j <= i; ++j) s += A[i * C + j];
        for (int f = 0; f < m; ++f) qz = fmaf(Q[(c0 + i) * m + f], z[f], qz);
        den[i] = fmaf(expf(L[i]), qz, s) + a.delta;
      }
      __syncthreads();
    }
    for (int e = tid; e < nc * dv; e += 256) {
      const int i = e / dv, c = e - i * dv;
      float s = 0.f, qs = 0.f;
      for (int j = 0; j <= i; ++j) s = fmaf(A[i * C + j], V[(c0 + j) * dv + c], s);
      for (int f = 0; f < m; ++f) qs = fmaf(Q[(c0 + i) * m + f], S[f * dv + c], qs);
      s = fmaf(expf(L[i]), qs, s);
      O[(c0 + i) * dv + c] = a.normalize ? s / den[i] : s;
    }
    __syncthreads();
    const float T = L[nc - 1];
    const float decay = expf(T);
    for (int64_t e = tid; e < per; e += 256) {
      if (e < static_cast<int64_t>(m) * dv) {
        const int f = static_cast<int>(e / dv), c = static_cast<int>(e - static_cast<int64_t>(f) * dv);
        float s = decay * S[e];
        for (int j = 0; j < nc; ++j)
          s = fmaf(expf(T - L[j]) * K[(c0 + j) * m + f], V[(c0 + j) * dv + c], s);
        S[e] = s;
      } else {
        const int f = static_cast<int>(e - static_cast<int64_t>(m) * dv);
        float s = decay * z[f];
        for (int j = 0; j < nc; ++j) s = fmaf(expf(T - L[j]), K[(c0 + j) * m + f], s);
        z[f] = s;
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void state_init_kernel(int64_t total_S, int64_t total_z,
                                                         const float* S0, const float* z0,
                                                         float* S, float* z) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e < total_S && S) S[e] = S0 ? S0[e] : 0.f;
  if (e < total_z && z) z[e] = z0 ? z0[e] : 0.f;
}

template <int C, int MTM, int NTW, bool CAUSAL>
hipError_t launch_out_t(const AttnArgs& a, dim3 grid, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const float* state, int64_t ss, int64_t sb,
                        float* out, hipStream_t st) {
  const size_t lds = (2ull * C * (a.m + 8) + static_cast<size_t>(a.m) * (C + 8) +
                      static_cast<size_t>(a.dv) * (C + 8) + static_cast<size_t>(C) * (C + 8)) *
                         sizeof(uint16_t) +
                     (a.m + C) * sizeof(float);
  const hipError_t e = allow_lds(attn_out_bf16<C, MTM, NTW, CAUSAL>, lds);
  if (e != hipSuccess) return e;
  LLOPS_LAUNCH("attn_out_bf16", st, (attn_out_bf16<C, MTM, NTW, CAUSAL>), grid, dim3(256), lds, st, a, q, k, v,
                     state, ss, sb, out);
  return hipGetLastError();
}

template <int C, bool CAUSAL>
hipError_t launch_out_c(const AttnArgs& a, dim3 grid, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const float* state, int64_t ss, int64_t sb,
                        float* out, hipStream_t st) {
  const bool wide = a.dv > 64;
  if (a.m <= 64)
    return wide ? launch_out_t<C, 4, 2, CAUSAL>(a, grid, q, k, v, state, ss, sb, out, st)
                : launch_out_t<C, 4, 1, CAUSAL>(a, grid, q, k, v, state, ss, sb, out, st);
  if (a.m <= 128)
    return wide ? launch_out_t<C, 8, 2, CAUSAL>(a, grid, q, k, v, state, ss, sb, out, st)
                : launch_out_t<C, 8, 1, CAUSAL>(a, grid, q, k, v, state, ss, sb, out, st);
  return wide ? launch_out_t<C, 16, 2, CAUSAL>(a, grid, q, k, v, state, ss, sb, out, st)
              : launch_out_t<C, 16, 1, CAUSAL>(a, grid, q, k, v, state, ss, sb, out, st);
}

template <int MTW, int NT>
hipError_t launch_state_t(const AttnArgs& a, dim3 grid, const uint16_t* k, const uint16_t* v,
                          float* seg, hipStream_t st) {
  const size_t lds = static_cast<size_t>(a.m + a.dv) * (64 + 8) * sizeof(uint16_t);
  LLOPS_LAUNCH("seg_state_bf16", st, (seg_state_bf16<MTW, NT>), grid, dim3(256), lds, st, a, k, v, seg);
  return hipGetLastError();
}

template <int MTW>
hipError_t launch_state_m(const AttnArgs& a, dim3 grid, const uint16_t* k, const uint16_t* v,
                          float* seg, hipStream_t st) {
  switch (a.dv / 16) {
    case 1: return launch_state_t<MTW, 1>(a, grid, k, v, seg, st);
    case 2: return launch_state_t<MTW, 2>(a, grid, k, v, seg, st);
    case 3: return launch_state_t<MTW, 3>(a, grid, k, v, seg, st);
    case 4: return launch_state_t<MTW, 4>(a, grid, k, v, seg, st);
    case 5: return launch_state_t<MTW, 5>(a, grid, k, v, seg, st);
    case 6: return launch_state_t<MTW, 6>(a, grid, k, v, seg, st);
    case 7: return launch_state_t<MTW, 7>(a, grid, k, v, seg, st);
    case 8: return launch_state_t<MTW, 8>(a, grid, k, v, seg, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_seg_state_bf16(const AttnShape& s, const uint16_t* phik, const uint16_t* v,
                                 float* seg, hipStream_t st) {
  const AttnArgs a = to_args(s);
  dim3 grid(static_cast<unsigned>(s.nseg), static_cast<unsigned>(s.BH));
  if (s.m <= 64) return launch_state_m<1>(a, grid, phik, v, seg, st);
  if (s.m <= 128) return launch_state_m<2>(a, grid, phik, v, seg, st);
  return launch_state_m<4>(a, grid, phik, v, seg, st);
}

hipError_t launch_seg_state_f32(const AttnShape& s, const float* phik, const float* v,
                                float* seg, hipStream_t st) {
  const AttnArgs a = to_args(s);
  dim3 grid(static_cast<unsigned>(s.nseg), static_cast<unsigned>(s.BH));
  LLOPS_LAUNCH("seg_state_f32", st, seg_state_f32, grid, dim3(256), 0, st, a, phik, v, seg);
  return hipGetLastError();
}

hipError_t launch_seg_scan(const AttnShape& s, float* seg, const float* S0, const float* z0,
                           float* Sout, float* zout, int exclusive, hipStream_t st) {
  // Sout is [BH][m*dv] and zout [BH][m] unless they alias one contiguous
  // [BH][m*dv + m] buffer (zout == Sout + m*dv), which the non-causal path uses.
  const int64_t mdv = static_cast<int64_t>(s.m) * s.dv;
  const int64_t per = mdv + s.m;
  int64_t Sb = mdv, zb = s.m;
  if (Sout && zout == Sout + mdv) {
    Sb = per;
    zb = per;
  }
  dim3 grid(static_cast<unsigned>((per + 255) / 256), static_cast<unsigned>(s.BH));
  LLOPS_LAUNCH("seg_scan", st, seg_scan_kernel, grid, dim3(256), 0, st, s.nseg, s.m, s.dv, seg, S0, z0,
                     Sout, Sb, zout, zb, exclusive, static_cast<const float*>(nullptr),
                     s.anti ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_seg_scan_gated(const AttnShape& s, float* seg, const float* gseg,
                                 const float* S0, const float* z0, float* Sout, float* zout,
                                 hipStream_t st) {
  if (s.anti) return hipErrorInvalidValue;  // gated suffix scans run on reversed sequences
  const int64_t mdv = static_cast<int64_t>(s.m) * s.dv;
  const int64_t per = mdv + s.m;
  dim3 grid(static_cast<unsigned>((per + 255) / 256), static_cast<unsigned>(s.BH));
  LLOPS_LAUNCH("seg_scan", st, seg_scan_kernel, grid, dim3(256), 0, st, s.nseg, s.m, s.dv, seg, S0,
               z0, Sout, mdv, zout, static_cast<int64_t>(s.m), 1, gseg, 0);
  return hipGetLastError();
}

hipError_t launch_attn_out_bf16(const AttnShape& s, const uint16_t* phiq, const uint16_t* phik,
                                const uint16_t* v, const float* state, int64_t st_seg,
                                int64_t st_bh, float* out, hipStream_t st) {
  if (s.anti) return hipErrorInvalidValue;  // the anti-causal form runs on attn_out32 only
  const AttnArgs a = to_args(s);
  dim3 grid(static_cast<unsigned>(s.nseg), static_cast<unsigned>(s.BH));
  if (s.causal) {
    if (s.chunk == 32)
      return launch_out_c<32, true>(a, grid, phiq, phik, v, state, st_seg, st_bh, out, st);
    return launch_out_c<64, true>(a, grid, phiq, phik, v, state, st_seg, st_bh, out, st);
  }
  return launch_out_c<64, false>(a, grid, phiq, phik, v, state, st_seg, st_bh, out, st);
}

hipError_t launch_attn_out_f32(const AttnShape& s, const float* phiq, const float* phik,
                               const float* v, float* state, int64_t st_seg, int64_t st_bh,
                               float* out, hipStream_t st) {
  if (s.anti) return hipErrorInvalidValue;
  const AttnArgs a = to_args(s);
  dim3 grid(static_cast<unsigned>(s.nseg), static_cast<unsigned>(s.BH));
  const size_t lds = (static_cast<size_t>(s.chunk) * s.chunk + s.chunk) * sizeof(float);
  hipError_t e = allow_lds(attn_out_f32<true>, lds);
  if (e == hipSuccess) e = allow_lds(attn_out_f32<false>, lds);
  if (e != hipSuccess) return e;
  if (s.causal)
    LLOPS_LAUNCH("attn_out_f32", st, attn_out_f32<true>, grid, dim3(256), lds, st, a, phiq, phik, v, state,
                       st_seg, st_bh, out);
  else
    LLOPS_LAUNCH("attn_out_f32", st, attn_out_f32<false>, grid, dim3(256), lds, st, a, phiq, phik, v, state,
                       st_seg, st_bh, out);
  return hipGetLastError();
}

// (d, m, p, t) of the small-sequence kernel's instantiations
int small_key(int d, int m, int p, int t) {
  const int key = d * 1000000 + m * 1000 + p * 10 + t;
  switch (key) {
    case 16032022: return key;  // d = 16, m = 32, p = 2, t = 2
    default: return 0;
  }
}

bool linattn_small_f32_ok(int64_t BH, int64_t n, int d, int dv, int m, int p, int t) {
  if (BH <= 0 || BH > 0x7fffffffLL || n <= 0 || n > 1024 || dv % 4 || dv <= 0) return false;
  if (!small_key(d, m, p, t)) return false;
  const int W4 = dv / 4 + 1;
  if (m * W4 > kSmallNT || kSmallTR * W4 > 3 * kSmallNT) return false;
  return SmallGeom<16, 32, 2, 2>::floats(dv) * 4 <= 160 * 1024;
}

hipError_t launch_linattn_small_f32(int64_t B, int64_t H, int64_t n, int d, int dv, int m, int p,
                                    int t, const float* Q, const float* K, const float* V,
                                    const float* tq, const float* tk, int64_t th_hstride,
                                    int square, int normalize, float delta, float* out,
                                    hipStream_t st) {
  if (!linattn_small_f32_ok(B * H, n, d, dv, m, p, t)) return hipErrorInvalidValue;
  SmallArgs a{Q, K, V, tq, tk, out, H, n, dv, th_hstride, square, normalize, delta};
  switch (small_key(d, m, p, t)) {
    case 16032022: {
      const size_t lds = static_cast<size_t>(SmallGeom<16, 32, 2, 2>::floats(dv) * 4);
      const hipError_t e = allow_lds(linattn_small_f32<16, 32, 2, 2>, lds);
      if (e != hipSuccess) return e;
      LLOPS_LAUNCH("linattn_small_f32", st, (linattn_small_f32<16, 32, 2, 2>),
                   dim3(static_cast<unsigned>(B * H)), dim3(kSmallNT),
                   lds, st, a);
      break;
    }
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_seg_state_f32_gated(const AttnShape& s, const float* phik, const float* v,
                                      const float* log_gate, float* gseg, float* seg,
                                      hipStream_t st) {
  const AttnArgs a = to_args(s);
  dim3 grid(static_cast<unsigned>(s.nseg), static_cast<unsigned>(s.BH));
  LLOPS_LAUNCH("seg_state_f32_gated", st, seg_state_f32_gated, grid, dim3(256), 0, st, a, phik, v,
               log_gate, gseg, seg);
  return hipGetLastError();
}

hipError_t launch_attn_out_f32_gated(const AttnShape& s, const float* phiq, const float* phik,
                                     const float* v, const float* log_gate, float* state,
                                     float* out, hipStream_t st) {
  if (s.anti) return hipErrorInvalidValue;
  if (!s.causal) return hipErrorInvalidValue;
  const AttnArgs a = to_args(s);
  dim3 grid(static_cast<unsigned>(s.nseg), static_cast<unsigned>(s.BH));
  const size_t lds = (static_cast<size_t>(s.chunk) * s.chunk + 2 * s.chunk) * sizeof(float);
  const hipError_t e = allow_lds(attn_out_f32_gated, lds);
  if (e != hipSuccess) return e;
  LLOPS_LAUNCH("attn_out_f32_gated", st, attn_out_f32_gated, grid, dim3(256), lds, st, a, phiq,
               phik, v, log_gate, state, out);
  return hipGetLastError();
}

hipError_t launch_state_init(int64_t BH, int m, int dv, const float* S0, const float* z0,
                             float* S, float* z, hipStream_t st) {
  const int64_t tS = BH * m * dv, tz = BH * m;
  const int64_t tot = tS > tz ? tS : tz;
  if (tot == 0) return hipSuccess;
  LLOPS_LAUNCH("state_init", st, state_init_kernel, dim3(static_cast<unsigned>((tot + 255) / 256)),
                     dim3(256), 0, st, tS, tz, S0, z0, S, z);
  return hipGetLastError();
}

}  // namespace llops
