// Segment passes of LLoPS linear attention on 32x32x16 bf16 MFMA.
//
//   causal:     out_i = phi_Q,i S_i [/ (phi_Q,i z_i + delta)], S_i = sum_{j<=i} phi_K,j v_j^T
//     (LLoPS paper Sec. 1: streaming form with a constant-size state; low-rank
//      attention blog: causal masking by incremental cumulative sums)
//   non-causal: out = phi_Q S [/ (phi_Q z + delta)] with S, z over all tokens
//     (LLoPS notes, overall framework; blog, Performer section; SLAY notes,
//      key design 3 for the +delta)
//
// The state pass has one wave per 32 value columns (dv / 32 waves), the
// output pass two (one per feature half). Each wave owns its columns of the
// fp32 state S (accumulator tiles) and a share of the normaliser state z,
// kept as accumulator tiles of S against an all-ones value block so that z
// and phi_Q . z come out of the same MFMAs. A segment is
// walked in chunks of 32 tokens whose phi_Q / phi_K / V rows are staged in
// LDS in their natural row-major layout (double buffered; the next chunk is
// prefetched into registers while the current one computes). Operands that
// contract over tokens are read with ds_read_b64_tr_b16 (transposing LDS
// reads), so no transposed copy is ever stored.
//
// Gated variant (causal only): a per-token scalar decay a_i = exp(g_i)
// scales the whole state before token i is added, S_i = a_i S_{i-1} +
// phi_K,i v_i^T (the forgetting gates the LLoPS notes name as future work,
// limitations and outlook, with Mamba2's semiseparable form as the example).
// With L the inclusive sum of g inside each 32-token chunk (gate_cumsum32
// below) and T its value at the chunk's last token, a chunk contributes
//   intra: A_qk = exp(L_q - L_k) phi_Q,q . phi_K,k  (k <= q),
//   inter: exp(L_q) phi_Q,q S_prev,
//   carry: S = exp(T) S_prev + phi_K^T diag(exp(T - L_k)) V,
// and every exponent is <= 0 when g <= 0, so no factor overflows. The
// per-chunk L values ride in LDS behind the chunk's rows.
//
// Anti-causal form (the backwards' suffix sums, key j >= query i): the output
// pass walks a segment's chunks from the last to the first with the mirrored
// intra-chunk mask, and each segment starts from the sum over the segments
// after it; gated, query rows take exp(T - L_i), keys exp(L_j), the state
// still decays by exp(T), and again no exponent is positive.
//
// Fragment conventions for v_mfma_f32_32x32x16_bf16 (lane l, c = l % 32,
// hh = l / 32): an accumulator element 4i+e holds row 8i + 4hh + e of column
// c. Taken as an operand, rows 0..15 of a tile (elements 0..7) put k-values
// {4hh..4hh+3, 8+4hh..8+4hh+3} in lane half hh; every other operand of the
// same product is read with that same k order ("P16" below).
#include "device.h"
#include "kernels.h"

namespace llops {
namespace {

constexpr int kC = 32;  // tokens per chunk

struct Seg32Args {
  int64_t n;
  int64_t seg_len;   // tokens per segment (multiple of kC)
  int nseg;
  int normalize;
  float delta;
  const float* gl;   // gated: chunk-local inclusive sums of log gates [BH][n]
  float* gseg;       // gated pass 1: per-segment sum of log gates [BH][nseg]
  // AUG passes (the backward's chain-rule operands): phi_Q (phi_K) rows are
  // qald (kald) bf16 per row, then zeros, with a bf16 one at column qald
  // (kald) when qone (kone) is set; see AugRows
  int qald, kald;
  int qone, kone;
};

// A narrow feature row read as M bf16: the ald values of a stored row (row
// stride ald, a multiple of 8), then zeros, with a bf16 one at column ald if
// `one`. This is the backward's [dnum | dden | 0] (stored [dnum | dden],
// padded to a multiple of 8) and [v | 1 | 0] (v itself) without their
// padded copies. Piece q (16 bytes) of a row is stored piece q (q < ald/8),
// else zeros: the others are requested past the view, where the hardware
// range check reads zeros, so the one load a piece takes is unconditional.
struct AugRows {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t row;   // stored row bytes
  int ald8;       // stored pieces per row
  uint32_t one;   // bf16 one (0x3F80) or 0, ORed into element 0 of piece ald8
};
__device__ __forceinline__ AugRows aug_rows(const uint16_t* rows0, int ald, int one, int64_t row0,
                                            uint32_t rows) {
  return AugRows{make_rsrc(rows0 + row0 * ald, rows * static_cast<uint32_t>(ald) * 2u),
                 static_cast<uint32_t>(ald) * 2u, ald / 8, one ? 0x3F80u : 0u};
}
// Narrow rows fill at most kAugTiles 32-feature tiles (ald + one <= 160);
// the tiles after them hold zeros in every operand and state, so the AUG
// passes skip their products (adding exact zeros changes no sum).
constexpr int kAugTiles = 5;
// piece q of row `row` of chunk c (kC rows a chunk)
__device__ __forceinline__ u32x4 aug_ld(const AugRows& v, int row, int q, int c) {
  constexpr uint32_t kPast = 0x80000000u;  // past any view (views stay below 2^31 bytes)
  const uint32_t off = q < v.ald8 ? static_cast<uint32_t>(row) * v.row + q * 16u : kPast;
  u32x4 r = buf_ld16_nt(v.rs, off, static_cast<uint32_t>(c) * (kC * v.row));
  r[0] |= q == v.ald8 ? v.one : 0u;
  return r;
}

constexpr int kGL = 2 * kC;  // LDS slots (uint16) of one chunk's 32 fp32 gate sums

// Row stride of the gate sums L [BH][n rounded up to 32]: every chunk's 32
// values start on a 128-byte boundary.
__host__ __device__ __forceinline__ int64_t gl_ld(int64_t n) { return (n + kC - 1) / kC * kC; }

// Smallest LDS row stride (bf16 elements) of at least `cols` whose byte
// offset mod 256 (the 64 banks) is 2 * res or its mirror 256 - 2 * res (a
// read touches the mirrored set of banks, so conflicts are the same). Which
// residue a read pattern wants was measured per pattern: 16-byte row reads
// 16 or 48 bytes; transposing reads 64 bytes; a block read both ways 48
// bytes (1x and 2x).
constexpr int lds_stride_at(int cols, int res) { return cols + ((res - cols) % 128 + 128) % 128; }
constexpr int lds_stride(int cols, int res) {
  return lds_stride_at(cols, res) < lds_stride_at(cols, 128 - res) ? lds_stride_at(cols, res)
                                                                   : lds_stride_at(cols, 128 - res);
}

// Scale the 8 bf16 values of an operand fragment by s[0..7] (fp32 products,
// rounded back to bf16 to nearest even).
__device__ __forceinline__ bf16x8 scale_frag(bf16x8 x, const float* s) {
  const u32x4 u = __builtin_bit_cast(u32x4, x);
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = pack_bf16x2(__uint_as_float(u[q] << 16) * s[2 * q],
                       __uint_as_float(u[q] & 0xFFFF0000u) * s[2 * q + 1]);
  return as_bf16x8(r);
}

// ---- finish of an output-pass chunk ----------------------------------------
// A finishing wave keeps 16 of the chunk's 32 rows: element e (0..7) of lane
// half hh is chunk row 8 * ((kept + e) / 4) + 4 * hh + e % 4, kept = 0 or 8.
__device__ __forceinline__ int kept_row(int kept, int e, int hh) {
  return 8 * ((kept + e) >> 2) + 4 * hh + (e & 3);
}
// The row whose denominator a lane forms: lane i of every 16-lane row takes
// the row of element i % 8 of its half, so that a broadcast from lane e of
// each 16-lane row (DPP row_newbcast, no LDS traffic) hands every lane the
// denominator of its element e.
__device__ __forceinline__ int den_row(int kept, int lane) {
  return kept_row(kept, lane & 7, lane >> 5);
}
template <int E>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + E, 0xF, 0xF, false));
}
// val[e] *= the inverse denominator of element e's row (inv: den_row's)
__device__ __forceinline__ void scale_rows(float (&val)[8], float inv) {
  val[0] *= row_bcast<0>(inv);
  val[1] *= row_bcast<1>(inv);
  val[2] *= row_bcast<2>(inv);
  val[3] *= row_bcast<3>(inv);
  val[4] *= row_bcast<4>(inv);
  val[5] *= row_bcast<5>(inv);
  val[6] *= row_bcast<6>(inv);
  val[7] *= row_bcast<7>(inv);
}
// t[k] *= the value lane k of this lane's 16-lane row holds (k = 0..15)
__device__ __forceinline__ void scale_rows16(f32x16& t, float f) {
  t[0] *= row_bcast<0>(f);
  t[1] *= row_bcast<1>(f);
  t[2] *= row_bcast<2>(f);
  t[3] *= row_bcast<3>(f);
  t[4] *= row_bcast<4>(f);
  t[5] *= row_bcast<5>(f);
  t[6] *= row_bcast<6>(f);
  t[7] *= row_bcast<7>(f);
  t[8] *= row_bcast<8>(f);
  t[9] *= row_bcast<9>(f);
  t[10] *= row_bcast<10>(f);
  t[11] *= row_bcast<11>(f);
  t[12] *= row_bcast<12>(f);
  t[13] *= row_bcast<13>(f);
  t[14] *= row_bcast<14>(f);
  t[15] *= row_bcast<15>(f);
}
// Denominator of a chunk row: delta, then the row sum of the rounded masked
// weights (rs), then the z-tile owners' partials (lo, hi: the row's 8 wave
// slots; wave w = half * NWD + value tile) in wave order, first feature half
// then second, NZ z tiles per half.
template <int NWD, int NZ>
__device__ __forceinline__ float den_sum(float delta, float rs, u32x4 lo, u32x4 hi) {
  const float pv[8] = {__uint_as_float(lo[0]), __uint_as_float(lo[1]), __uint_as_float(lo[2]),
                       __uint_as_float(lo[3]), __uint_as_float(hi[0]), __uint_as_float(hi[1]),
                       __uint_as_float(hi[2]), __uint_as_float(hi[3])};
  float dq = delta + rs;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int d = 0; d < NZ; ++d) dq += pv[hf * NWD + d];
  return dq;
}

// Gate sums of the 16 tokens 8i + 4hh + e (i, e < 4) this lane's fragments
// cover (accumulator rows, P16 operand k-values), element 4i + e.
__device__ __forceinline__ void gate_rows(const float* gls, int hh, float (&L)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(gls + 8 * i + 4 * hh);
#pragma unroll
    for (int e = 0; e < 4; ++e) L[4 * i + e] = x[e];
  }
}

// f(token) for the 16 tokens of this lane's elements (element k: token
// 8(k/4) + 4hh + k%4): each lane evaluates f once, at element (lane % 16)'s
// token, and a DPP row broadcast from lane k hands out element k's value.
template <class F>
__device__ __forceinline__ void per_row16(int lane, int hh, F f, float (&out)[16]) {
  const int i16 = lane & 15;
  const float v = f(8 * (i16 >> 2) + 4 * hh + (i16 & 3));
  out[0] = row_bcast<0>(v);
  out[1] = row_bcast<1>(v);
  out[2] = row_bcast<2>(v);
  out[3] = row_bcast<3>(v);
  out[4] = row_bcast<4>(v);
  out[5] = row_bcast<5>(v);
  out[6] = row_bcast<6>(v);
  out[7] = row_bcast<7>(v);
  out[8] = row_bcast<8>(v);
  out[9] = row_bcast<9>(v);
  out[10] = row_bcast<10>(v);
  out[11] = row_bcast<11>(v);
  out[12] = row_bcast<12>(v);
  out[13] = row_bcast<13>(v);
  out[14] = row_bcast<14>(v);
  out[15] = row_bcast<15>(v);
}

// Carry weights w_k = exp(T - L_k) of this lane's 16 tokens, element 4i + e
// (0 past the chunk's valid rows); elements 8ks..8ks+7 line up with the P16
// k-values of the ks-th V fragment of the chunk. One exp per lane.
__device__ __forceinline__ void gate_carry(const float* gls, int lane, int hh, float T, int valid,
                                           float (&wv)[16]) {
  per_row16(lane, hh, [&](int tok) { return tok < valid ? __expf(T - gls[tok]) : 0.f; }, wv);
}

template <int M, int DV>
struct Seg32Geom {
  static constexpr int NW = DV / 32;       // waves per workgroup
  static constexpr int NT = NW * 64;       // threads
  static constexpr int FT = M / 32;        // feature tiles
  static constexpr int ZT = FT / NW > 0 ? FT / NW : 1;  // z tiles per wave
  static constexpr int MP = M + 32;        // LDS row strides (elements): rows 64 bytes
  static constexpr int VP = DV + 32;       //   apart mod 256, conflict-free tr reads
  static constexpr int BUF = kC * MP * 2 + kC * VP;  // one chunk: phi_Q, phi_K, V
  static constexpr int QCH = kC * M / 8, VCH = kC * DV / 8;  // 16-byte pieces per chunk
  static constexpr int LPT_Q = QCH / NT, LPT_V = VCH / NT;
  static_assert(QCH % NT == 0 && VCH % NT == 0, "chunk splits evenly over the threads");
  static_assert(FT % NW == 0 || NW % FT == 0, "z tiles split over the waves");
};

// ============================================================================
// Pass 1: per-segment (dS, dz) = (phi_K^T V, phi_K^T 1)
// ============================================================================
// ANCHOR (gated only): the segment's sum anchored at its start instead of
// carried to its end, sum_k exp(c_k - c_{t0-1}) phi_K,k v_k^T: weights
// exp(D + L_k) with D the sum of the segment's earlier chunks, no decay of
// the accumulator (every exponent still <= 0 for g <= 0).
// VSTR: the value rows are vld elements apart (a column slice of a wider
// row; v points at the slice's first column).
// AUG: phi_K rows are narrow (AugRows: a.kald, a.kone).
template <int M, int DV, bool GATED, bool ANCHOR = false, bool VSTR = false, bool AUG = false>
__global__ __launch_bounds__(DV * 2) __attribute__((amdgpu_waves_per_eu(2)))
void seg_state32(Seg32Args a, const uint16_t* __restrict__ phik,
                                                     const uint16_t* __restrict__ v,
                                                     float* __restrict__ seg, int vld) {
  using G = Seg32Geom<M, DV>;
  constexpr int FT = G::FT, MP = G::MP, VP = G::VP, NT = G::NT;
  constexpr int BUF = kC * MP + kC * VP + (GATED ? kGL : 0);  // phi_K, V [, gate sums]
  constexpr int LK = G::LPT_Q, LV = G::LPT_V;
  extern __shared__ __align__(16) uint16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: MFMAs under a condition on it must branch, not
  // be masked through EXEC (an MFMA runs for the whole wave regardless)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.y;
  const int gseg = blockIdx.x;
  const int64_t t0 = gseg * a.seg_len;
  const int64_t t1 = min(a.n, t0 + a.seg_len);
  const uint16_t* Kg = phik + bh * a.n * M;
  const int VL = VSTR ? vld : DV;
  const uint16_t* Vg = v + bh * a.n * VL;
  const int nch = static_cast<int>((t1 - t0 + kC - 1) / kC);

  // Raw buffer views of this segment's rows: reads past the segment end
  // return zeros (hardware range check), so every load is unconditional, the
  // number in flight is static and a wait for one chunk never drains the next.
  const uint32_t seg_rows = static_cast<uint32_t>(t1 - t0);
  const __amdgpu_buffer_rsrc_t rsk = make_rsrc(AUG ? phik : Kg + t0 * M, AUG ? 0u : seg_rows * M * 2u);
  AugRows ka{};
  if constexpr (AUG) ka = aug_rows(phik, a.kald, a.kone, bh * a.n + t0, seg_rows);
  static_assert(!AUG || G::NT % (M / 8) == 0, "a thread's pieces share one column");
  // strided: the view ends at the slice's last element
  const __amdgpu_buffer_rsrc_t rsv = make_rsrc(
      Vg + t0 * VL, VSTR ? (seg_rows ? ((seg_rows - 1u) * VL + DV) * 2u : 0u) : seg_rows * DV * 2u);
  // gated: the chunk's 32 gate sums (128 bytes) come with the chunk, one per
  // lane of the first half of wave 0
  const __amdgpu_buffer_rsrc_t rsg =
      make_rsrc(GATED ? a.gl + bh * gl_ld(a.n) + t0 : nullptr,
                GATED ? static_cast<uint32_t>(gl_ld(seg_rows)) * 4u : 0u);
  uint32_t rg = 0u;
  auto load = [&](int c, u32x4 (&rk)[LK], u32x4 (&rv)[LV]) {
    // piece idx of a chunk is 16 contiguous bytes at byte 16 * idx; the rows
    // are streamed once, so the loads are non-temporal (0.316 -> 0.291 ms at
    // 1 x 32 x 65536)
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      if constexpr (AUG)
        rk[i] = aug_ld(ka, (tid + i * NT) / (M / 8), tid % (M / 8), c);
      else
        rk[i] = buf_ld16_nt(rsk, (tid + i * NT) * 16u, static_cast<uint32_t>(c) * (kC * M * 2u));
    }
#pragma unroll
    for (int i = 0; i < LV; ++i)
      rv[i] = buf_ld16_nt(rsv,
                       VSTR ? static_cast<uint32_t>((tid + i * NT) / (DV / 8)) * (VL * 2u) +
                                  static_cast<uint32_t>((tid + i * NT) % (DV / 8)) * 16u
                            : (tid + i * NT) * 16u,
                       static_cast<uint32_t>(c) * (kC * VL * 2u));
    if (GATED && w == 0) rg = buf_ld4(rsg, (lane & 31) * 4u + static_cast<uint32_t>(c) * (kC * 4u));
  };
  auto store = [&](uint16_t* buf, const u32x4 (&rk)[LK], const u32x4 (&rv)[LV]) {
    if (GATED && w == 0 && lane < kC) reinterpret_cast<uint32_t*>(buf + kC * MP + kC * VP)[lane] = rg;
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int idx = tid + i * NT, row = idx / (M / 8), col = idx % (M / 8);
      st16(buf + row * MP + col * 8, rk[i]);
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int idx = tid + i * NT, row = idx / (DV / 8), col = idx % (DV / 8);
      st16(buf + kC * MP + row * VP + col * 8, rv[i]);
    }
  };

  f32x16 S[FT], Z[G::ZT];
#pragma unroll
  for (int f = 0; f < FT; ++f) S[f] = zero16();
#pragma unroll
  for (int z = 0; z < G::ZT; ++z) Z[z] = zero16();
  const bf16x8 ones = as_bf16x8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  const int hh = lane >> 5;
  float gsum = 0.f;  // gated: sum of this segment's log gates

  // one chunk: request chunk c+1 into the registers (clamped past the
  // end), run chunk c from LDS, move chunk c+1 into the other slot, barrier
  u32x4 rk[LK], rv[LV];
  auto step = [&](int c) {
    load(c + 1 < nch ? c + 1 : nch - 1, rk, rv);
    const uint16_t* Ks = smem + (c & 1) * BUF;
    const uint16_t* Vs = Ks + kC * MP;
    // phi_K fragment reads run KD products ahead (pinned: the scheduler
    // would sink each next to its MFMA and expose the LDS latency)
    constexpr int NK = (kC / 16) * FT, KD = NK < 2 ? NK : 2;
    bf16x8 vb[kC / 16], kf[KD], zb[kC / 16];
#pragma unroll
    for (int ks = 0; ks < kC / 16; ++ks) {
      vb[ks] = frag_tr(Vs, VP, ks * 16, w * 32, lane);
      zb[ks] = ones;
    }
    if constexpr (GATED) {
      // S <- exp(T) S + phi_K^T diag(exp(T - L)) V over this chunk
      const float* gls = reinterpret_cast<const float*>(Vs + kC * VP);
      const int64_t left = t1 - (t0 + static_cast<int64_t>(c) * kC);
      const int valid = left < kC ? static_cast<int>(left) : kC;
      const float T = gls[valid - 1];
      float wv[16];
      if constexpr (ANCHOR) {
        per_row16(lane, hh, [&](int tok) { return tok < valid ? __expf(gsum + gls[tok]) : 0.f; },
                  wv);
      } else {
        gate_carry(gls, lane, hh, T, valid, wv);
      }
#pragma unroll
      for (int ks = 0; ks < kC / 16; ++ks) {
        vb[ks] = scale_frag(vb[ks], wv + 8 * ks);
        zb[ks] = as_bf16x8(u32x4{pack_bf16x2(wv[8 * ks + 0], wv[8 * ks + 1]),
                                 pack_bf16x2(wv[8 * ks + 2], wv[8 * ks + 3]),
                                 pack_bf16x2(wv[8 * ks + 4], wv[8 * ks + 5]),
                                 pack_bf16x2(wv[8 * ks + 6], wv[8 * ks + 7])});
      }
      if constexpr (!ANCHOR) {
        const float decay = __expf(T);
#pragma unroll
        for (int f = 0; f < FT; ++f) S[f] *= decay;
#pragma unroll
        for (int z = 0; z < G::ZT; ++z) Z[z] *= decay;
      }
      gsum += T;
    }
    // AUG: the live feature tiles only (kAugTiles)
    constexpr int FL = AUG ? kAugTiles : FT, NL = (kC / 16) * FL;
#pragma unroll
    for (int i = 0; i < KD; ++i) kf[i] = frag_tr(Ks, MP, (i / FL) * 16, (i % FL) * 32, lane);
#pragma unroll
    for (int idx = 0; idx < NL; ++idx) {
      const int ks = idx / FL, f = idx % FL;
      const bf16x8 ka = kf[idx % KD];
      if (idx + KD < NL) kf[idx % KD] = frag_tr(Ks, MP, ((idx + KD) / FL) * 16, ((idx + KD) % FL) * 32, lane);
      S[f] = mfma32x32x16(ka, vb[ks], S[f]);
      if ((f % G::NW) == (w % G::NW) && f / G::NW < G::ZT)
        Z[f / G::NW] = mfma32x32x16(ka, zb[ks], Z[f / G::NW]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c + 1 < nch) store(smem + ((c + 1) & 1) * BUF, rk, rv);
    __syncthreads();
  };

  load(0, rk, rv);
  store(smem, rk, rv);
  __syncthreads();
  for (int c = 0; c < nch; ++c) step(c);
  if (GATED && tid == 0) a.gseg[bh * a.nseg + gseg] = gsum;
  float* out = seg + (bh * a.nseg + gseg) * (static_cast<int64_t>(M) * DV + M);
  const int c32 = lane & 31;
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        out[(f * 32 + 8 * i + 4 * hh + e) * DV + w * 32 + c32] = S[f][4 * i + e];
  if (c32 == 0) {
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      if ((f % G::NW) != (w % G::NW) || f / G::NW >= G::ZT) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          out[static_cast<int64_t>(M) * DV + f * 32 + 8 * i + 4 * hh + e] = Z[f / G::NW][4 * i + e];
    }
  }
}

// ============================================================================
// Pass 2: outputs of one segment, starting from its prefix state
// ============================================================================
// 2 * dv/32 waves: wave w owns value-column tile w % (dv/32) and feature half
// w / (dv/32) of the state (m/64 tiles of 32 features), so every wave keeps
// m/64 fp32 accumulator tiles of S. The two halves of a column tile each
// hold a partial phi_Q S; they swap the partial rows the other one finishes
// through LDS, and each wave normalises and stores 16 of the chunk's 32 rows.
// Wave dvt < m/64 of each half also keeps one z tile (z against all-ones
// values, inside its feature half). Chunks are prefetched two ahead into two
// alternating register sets; the exchange areas alternate by chunk parity, so
// one barrier per chunk orders everything.
template <int M, int DV, bool GATED>
struct Out32Geom {
  static constexpr int NWD = DV / 32;     // value-column tiles
  static constexpr int NW = 2 * NWD;      // waves
  static constexpr int NT = NW * 64;
  static constexpr int FT = M / 32;
  static constexpr int FH = FT / 2;       // feature tiles per half
  // row strides (elements): phi_Q is read in row order only (16-byte reads
  // 1x, 8-byte 2x at 16 bytes mod 256); phi_K both in row order (A^T) and
  // transposed (the state update): 1x and 2x at 48 bytes; V only transposed:
  // 1x at 64 bytes
  static constexpr int QPAD = M + 8, MP = lds_stride(M, 24), VP = lds_stride(DV, 32);
  static constexpr int BUF = kC * QPAD + kC * MP + kC * VP + (GATED ? kGL : 0);  // + gate sums
  static constexpr int QP = kC * M / 8;   // 16-byte pieces of one phi chunk
  static constexpr int VPc = kC * DV / 8;
  // LDS after the two chunk buffers, per parity: xo [NW][8][64] fp32,
  // part [kC][8] fp32 (z partial of wave w at [q][w]), rsum [kC] fp32
  static constexpr int XO = NW * 8 * 64, PART = kC * 8, EXW = XO + PART + kC;
  static_assert(NW <= 8, "z partial slots");
  static constexpr size_t lds_bytes() { return 2ull * BUF * 2 + 2ull * EXW * 4; }
  static_assert(lds_bytes() <= 160 * 1024, "LDS per workgroup");
  static_assert(FT % 2 == 0, "feature tiles split in two halves");
  static_assert(QP % NT == 0 && VPc % NT == 0, "chunk pieces split evenly over the threads");
};

// DENOUT: the row's denominator (without delta) goes to den_out [BH][n] and the
// output row stays unnormalised (a.normalize set, so both are formed as in
// the normalised pass); the backward takes num and den from one pass.
// ANTI (with CAUSAL): the anti-causal form, row i over keys j >= i. The
// segment's chunks run from the last to the first, the state entering a
// segment is the sum over the segments after it, and the intra-chunk mask
// keeps keys at or after the query. Every chunk keeps its natural row order,
// so the backward's suffix sums need no reversed copies of their operands.
// With GATED, key j reaches query i <= j with weight exp(c_j - c_i) (c the
// cumulative log gates): within a chunk exp(L_j - L_i); against the carried
// state the query row is scaled by exp(T - L_i), keys are carried with
// exp(L_j) and the state decays by exp(T) per chunk (L the chunk-local
// inclusive sums, T the chunk's last); every exponent is <= 0. The states
// are then the start-anchored inclusive suffix sums of the segments (slot g:
// the sum from segment g's start on), so segment g starts from slot g + 1
// and the last segment from zero.
// OM, the output rows' destination: 0 out [BH][n][DV]; bit 0 set, row t of
// the pass goes to row n - 1 - t (a pass over the reversed sequence writes
// in the original order); bit 1 set, bf16 (RNE) into outb, rows ldo elements
// apart (a column slice of a wider row).
// AUG: phi_Q and phi_K rows are narrow (AugRows: a.qald, a.qone, a.kald,
// a.kone).
template <int M, int DV, bool CAUSAL, bool GATED, bool DENOUT = false, int OM = 0,
          bool VSTR = false, bool ANTI = false, bool AUG = false>
__global__ __launch_bounds__(DV * 4) __attribute__((amdgpu_waves_per_eu(2)))
void attn_out32(Seg32Args a, const uint16_t* __restrict__ phiq, const uint16_t* __restrict__ phik,
                const uint16_t* __restrict__ v, const float* __restrict__ state, int64_t st_seg,
                int64_t st_bh, float* __restrict__ out, float* __restrict__ den_out,
                uint16_t* __restrict__ outb, int ldo, int vld) {
  using G = Out32Geom<M, DV, GATED>;
  constexpr int FH = G::FH, QPAD = G::QPAD, MP = G::MP, VP = G::VP, NT = G::NT, NWD = G::NWD;
  constexpr int QP = G::QP;
  static_assert(CAUSAL || !GATED, "the gated form is causal");
  static_assert(!ANTI || (CAUSAL && !DENOUT && (OM & 1) == 0),
                "the anti-causal form: no denominator output, rows in place");
  constexpr int NP = CAUSAL ? 2 * QP + G::VPc : QP;  // pieces staged per chunk
  constexpr int LPT = NP / NT;
  extern __shared__ __align__(16) uint16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: see attn pass 1
  const int dvt = w % NWD, half = w / NWD;
  const int f0 = half * FH;                    // first feature tile of this wave
  const bool has_z = dvt < FH;
  const int zj = dvt;                          // z tile = feature tile f0 + zj
  // AUG: this half's live feature tiles (the first kAugTiles of all). The
  // masked chunk product stays with half 0 (on half 1, whose tiles are
  // mostly dead, it measured no faster, and it changes the order in which
  // the two halves' partial rows are summed)
  static_assert(!AUG || (kAugTiles > FH && kAugTiles <= 2 * FH), "live tiles reach the second half");
  const int nlive = AUG ? (half == 0 ? FH : kAugTiles - FH) : FH;
  const int c32 = lane & 31, hh = lane >> 5;
  const int64_t bh = blockIdx.y;
  const int gseg = blockIdx.x;
  const int64_t t0 = gseg * a.seg_len;
  const int64_t t1 = min(a.n, t0 + a.seg_len);
  const uint16_t* Qg = phiq + bh * a.n * M;
  const uint16_t* Kg = phik + bh * a.n * M;
  const int VL = VSTR ? vld : DV;  // value row stride (VSTR: a column slice)
  const uint16_t* Vg = v + bh * a.n * VL;
  float* Og = out + bh * a.n * DV;
  // gated anti-causal: slot g + 1 (start-anchored suffix sums), none for the last
  constexpr bool SHIFT = ANTI && GATED;
  const bool zero_in = SHIFT && gseg + 1 >= a.nseg;
  const float* Sin = state + bh * st_bh + (gseg + (SHIFT ? 1 : 0)) * st_seg;
  const int nch = static_cast<int>((t1 - t0 + kC - 1) / kC);
  float* exbase = reinterpret_cast<float*>(smem + 2 * G::BUF);
  // chunk processed k-th (clamped to the segment; 0 for an empty one): the
  // k-th in order, or the k-th from the end (ANTI)
  auto chunk_at = [&](int k) {
    const int kk = k < nch - 1 ? k : nch - 1;
    const int ch = ANTI ? nch - 1 - kk : kk;
    return ch > 0 ? ch : 0;
  };

  f32x16 S[FH], Z;
#pragma unroll
  for (int j = 0; j < FH; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[j][4 * i + e] = zero_in ? 0.f : Sin[((f0 + j) * 32 + 8 * i + 4 * hh + e) * DV + dvt * 32 + c32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Z[4 * i + e] = has_z && !zero_in
                         ? Sin[static_cast<int64_t>(M) * DV + (f0 + zj) * 32 + 8 * i + 4 * hh + e]
                         : 0.f;
  const bf16x8 ones = as_bf16x8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  // Raw buffer views of this segment's rows: reads past the segment end
  // return zeros (hardware range check), so every load is unconditional and
  // the waits for one chunk never drain the loads of the next.
  const uint32_t seg_rows = static_cast<uint32_t>(t1 - t0);
  const __amdgpu_buffer_rsrc_t rsq = make_rsrc(AUG ? phiq : Qg + t0 * M, AUG ? 0u : seg_rows * M * 2u);
  const __amdgpu_buffer_rsrc_t rsk = make_rsrc(AUG ? phik : Kg + t0 * M, AUG ? 0u : seg_rows * M * 2u);
  AugRows qa{}, ka{};
  if constexpr (AUG) {
    qa = aug_rows(phiq, a.qald, a.qone, bh * a.n + t0, seg_rows);
    ka = aug_rows(phik, a.kald, a.kone, bh * a.n + t0, seg_rows);
  }
  static_assert(!AUG || NT % (M / 8) == 0, "a thread's pieces share one column");
  const __amdgpu_buffer_rsrc_t rsv = make_rsrc(
      Vg + t0 * VL, VSTR ? (seg_rows ? ((seg_rows - 1u) * VL + DV) * 2u : 0u) : seg_rows * DV * 2u);
  // piece p of a chunk: phi_Q rows, then phi_K rows, then V rows, 16
  // contiguous bytes each; a thread's pieces t + i*NT never straddle two
  // tensors, so the selection folds away. Streamed once: non-temporal loads.
  // gated: the chunk's 32 gate sums (128 bytes), one per lane of the first
  // half of wave 0, stored behind the chunk's V rows
  const __amdgpu_buffer_rsrc_t rsg =
      make_rsrc(GATED ? a.gl + bh * gl_ld(a.n) + t0 : nullptr,
                GATED ? static_cast<uint32_t>(gl_ld(seg_rows)) * 4u : 0u);
  auto load = [&](int c, u32x4 (&r)[LPT], uint32_t& rg) {
    if (GATED && w == 0) rg = buf_ld4(rsg, (lane & 31) * 4u + static_cast<uint32_t>(c) * (kC * 4u));
    int t = tid;  // opaque: per-piece offsets are rebuilt, not kept live
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int p = t + i * NT;
      if (AUG && i * NT < QP)
        r[i] = aug_ld(qa, p / (M / 8), p % (M / 8), c);
      else if (AUG && i * NT < 2 * QP)
        r[i] = aug_ld(ka, (p - QP) / (M / 8), (p - QP) % (M / 8), c);
      else if (i * NT < QP)
        r[i] = buf_ld16_nt(rsq, p * 16u, static_cast<uint32_t>(c) * (kC * M * 2u));
      else if (i * NT < 2 * QP)
        r[i] = buf_ld16_nt(rsk, (p - QP) * 16u, static_cast<uint32_t>(c) * (kC * M * 2u));
      else
        r[i] = buf_ld16_nt(rsv,
                        VSTR ? static_cast<uint32_t>((p - 2 * QP) / (DV / 8)) * (VL * 2u) +
                                   static_cast<uint32_t>((p - 2 * QP) % (DV / 8)) * 16u
                             : (p - 2 * QP) * 16u,
                        static_cast<uint32_t>(c) * (kC * VL * 2u));
    }
  };
  auto store = [&](uint16_t* buf, const u32x4 (&r)[LPT], const uint32_t& rg) {
    if (GATED && w == 0 && lane < kC)
      reinterpret_cast<uint32_t*>(buf + kC * QPAD + kC * MP + kC * VP)[lane] = rg;
    int t = tid;
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int p = t + i * NT;
      uint16_t* dst;
      if (i * NT < QP) {
        dst = buf + (p / (M / 8)) * QPAD + (p % (M / 8)) * 8;
      } else if (i * NT < 2 * QP) {
        const int pp = p - QP;
        dst = buf + kC * QPAD + (pp / (M / 8)) * MP + (pp % (M / 8)) * 8;
      } else {
        const int pp = p - 2 * QP;
        dst = buf + kC * QPAD + kC * MP + (pp / (DV / 8)) * VP + (pp % (DV / 8)) * 8;
      }
      st16(dst, r[i]);
    }
  };

  // one chunk: prefetch chunk c+2 into `ld` (whose chunk c is already in
  // LDS; unconditional, clamped, so wait counts stay static), compute chunk
  // c, move chunk c+1 from `wr` into the other LDS slot, publish partials,
  // barrier, finish this wave's rows
  auto step = [&](int c, u32x4 (&ld)[LPT], uint32_t& ldg, const u32x4 (&wr)[LPT], const uint32_t& wrg) {
    load(chunk_at(c + 2), ld, ldg);
    // Lane-dependent bases pass through an empty asm so the compiler cannot
    // hoist every derived LDS address and mask compare out of the chunk loop
    // (kept live across iterations they exhaust the 256-register budget).
    int lbase = (c & 1) * G::BUF;
    asm volatile("" : "+v"(lbase));
    int lim = c32 - 4 * hh;  // key 8i+4hh+e reaches query c32 iff 8i+e <= lim (ANTI: >=)
    asm volatile("" : "+v"(lim));
    const uint16_t* Qs = smem + lbase;
    const uint16_t* Ks = Qs + kC * QPAD;
    const uint16_t* Vs = Ks + kC * MP;
    int exoff = (c & 1) * G::EXW;
    asm volatile("" : "+v"(exoff));
    float* ex = exbase + exoff;
    float* xo = ex;
    float* part = ex + G::XO;
    float* rsum = part + G::PART;
    const int64_t c0 = t0 + static_cast<int64_t>(chunk_at(c)) * kC;
    // gated: the chunk's gate sums L sit behind its V rows
    auto gate_sums = [&]() { return reinterpret_cast<const float*>(Vs + kC * VP); };

    f32x16 O = zero16(), D = zero16();
    bf16x8 afr[2];
    // partial phi_Q S over this wave's feature half; phi_Q . z over its z
    // tile. The phi_Q fragment reads run QD products ahead (pinned).
    auto inter = [&]() {
      constexpr int NQ = 2 * FH, QD = NQ < 2 ? NQ : 2;
      bf16x8 qf[QD];
#pragma unroll
      for (int i = 0; i < QD; ++i) qf[i] = frag_p16_sep(Qs, QPAD, 0, f0 * 32 + i * 16, lane);
#pragma unroll
      for (int idx = 0; idx < NQ; ++idx) {
        const int j = idx >> 1, h = idx & 1;
        if (AUG && j >= nlive) break;  // wave-uniform: the rest of the half is dead tiles
        const bf16x8 qa = qf[idx % QD];
        if (idx + QD < NQ) qf[idx % QD] = frag_p16_sep(Qs, QPAD, 0, f0 * 32 + (idx + QD) * 16, lane);
        O = mfma32x32x16(qa, acc_frag(S[j], h), O);
        if (a.normalize && has_z && j == zj) D = mfma32x32x16(qa, acc_frag(Z, h), D);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    __builtin_amdgcn_sched_barrier(0);
    if (CAUSAL && half == 0) {
      // masked A^T = phi_K phi_Q^T (keys x queries)
      // fragment reads run AD k-steps ahead of the MFMA chain (pinned: the
      // scheduler would otherwise sink each read next to its MFMA and expose
      // the LDS latency on every step); AUG: over the live features only
      constexpr int KS = (AUG ? kAugTiles * 32 : M) / 16, AD = KS < 3 ? KS : 3;
      f32x16 At = zero16();
      bf16x8 fk[AD], fq[AD];
#pragma unroll
      for (int i = 0; i < AD; ++i) {
        fk[i] = frag_nat(Ks, MP, 0, i * 16, lane);
        fq[i] = frag_nat(Qs, QPAD, 0, i * 16, lane);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka = fk[ks % AD], qb = fq[ks % AD];
        if (ks + AD < KS) {
          fk[ks % AD] = frag_nat(Ks, MP, 0, (ks + AD) * 16, lane);
          fq[ks % AD] = frag_nat(Qs, QPAD, 0, (ks + AD) * 16, lane);
        }
        At = mfma32x32x16(ka, qb, At);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (GATED) {
        // A_qk = exp(L_q - L_k) phi_Q,q . phi_K,k for key k <= query q
        // (ANTI: exp(L_k - L_q) for key k >= query q)
        const float* gls = gate_sums();
        float Lr[16];
        gate_rows(gls, hh, Lr);
        const float Lq = gls[c32];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (ANTI)
              At[4 * i + e] = 8 * i + e < lim ? 0.f : At[4 * i + e] * __expf(Lr[4 * i + e] - Lq);
            else
              At[4 * i + e] = 8 * i + e > lim ? 0.f : At[4 * i + e] * __expf(Lq - Lr[4 * i + e]);
          }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)  // zero keys after the query (ANTI: before it)
            if (ANTI ? 8 * i + e < lim : 8 * i + e > lim) At[4 * i + e] = 0.f;
      }
      afr[0] = acc_frag(At, 0);
      afr[1] = acc_frag(At, 1);
      if (a.normalize && dvt == 0) {  // row sums of the rounded weights A V uses
        float rs = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 u = __builtin_bit_cast(u32x4, afr[h]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            rs += __uint_as_float(u[q] << 16) + __uint_as_float(u[q] & 0xFFFF0000u);
        }
        rs += __shfl_xor(rs, 32);
        if (hh == 0) rsum[c32] = rs;
      }
      if constexpr (!GATED) {
#pragma unroll
        for (int ks = 0; ks < kC / 16; ++ks)
          O = mfma32x32x16(afr[ks], frag_tr(Vs, VP, ks * 16, dvt * 32, lane), O);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (GATED) {
      // The carried state reaches query q with weight exp(L_q): a row scale
      // of phi_Q S and phi_Q . z, applied to the accumulators before A V
      // joins them. Element k of a tile is row 8(k/4) + 4hh + k%4; lane i
      // of each 16-lane row takes exp(L) of element i's row, and a DPP row
      // broadcast from lane k hands it to every lane (folded into the
      // multiply).
      inter();
      const int i16 = lane & 15;
      const float* gls = gate_sums();
      const float Lrow = gls[8 * (i16 >> 2) + 4 * hh + (i16 & 3)];
      float ef;
      if constexpr (ANTI) {  // exp(T - L_q): the chunk's last valid sum T
        const int valid = t1 - c0 < kC ? static_cast<int>(t1 - c0) : kC;
        ef = __expf(gls[valid - 1] - Lrow);
      } else {
        ef = __expf(Lrow);
      }
      scale_rows16(O, ef);
      scale_rows16(D, ef);
      __builtin_amdgcn_sched_barrier(0);
      if (half == 0) {
#pragma unroll
        for (int ks = 0; ks < kC / 16; ++ks)
          O = mfma32x32x16(afr[ks], frag_tr(Vs, VP, ks * 16, dvt * 32, lane), O);
      }
    } else {
      inter();
    }
    __builtin_amdgcn_sched_barrier(0);
    // publish: the 16 rows the partner wave finishes, and the z partial
    {
      // elements 8..15 are rows 16..31
#pragma unroll
      for (int e = 0; e < 8; ++e) xo[(w * 8 + e) * 64 + lane] = pick(O[8 + e], O[e], half == 0);
      if (a.normalize && has_z && c32 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) part[(8 * i + 4 * hh + e) * 8 + w] = D[4 * i + e];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (CAUSAL) {  // S += phi_K^T V, z += phi_K^T 1; phi_K reads run KD ahead
      constexpr int NK = (kC / 16) * FH, KD = NK < 2 ? NK : 2;
      bf16x8 kf[KD];
#pragma unroll
      for (int i = 0; i < KD; ++i) kf[i] = frag_tr(Ks, MP, (i / FH) * 16, (f0 + i % FH) * 32, lane);
      bf16x8 vb[kC / 16], zb[kC / 16];
#pragma unroll
      for (int ks = 0; ks < kC / 16; ++ks) {
        vb[ks] = frag_tr(Vs, VP, ks * 16, dvt * 32, lane);
        zb[ks] = ones;
      }
      if constexpr (GATED) {
        // S <- exp(T) S + phi_K^T diag(exp(T - L)) V, z likewise
        // (ANTI: keys carried with exp(L))
        const float* gls = gate_sums();
        const int valid = t1 - c0 < kC ? static_cast<int>(t1 - c0) : kC;  // rows in range
        const float T = gls[valid - 1];
        float wv[16];
        if constexpr (ANTI)
          per_row16(lane, hh, [&](int tok) { return tok < valid ? __expf(gls[tok]) : 0.f; }, wv);
        else
          gate_carry(gls, lane, hh, T, valid, wv);
#pragma unroll
        for (int ks = 0; ks < kC / 16; ++ks) {
          vb[ks] = scale_frag(vb[ks], wv + 8 * ks);
          zb[ks] = as_bf16x8(u32x4{pack_bf16x2(wv[8 * ks + 0], wv[8 * ks + 1]),
                                   pack_bf16x2(wv[8 * ks + 2], wv[8 * ks + 3]),
                                   pack_bf16x2(wv[8 * ks + 4], wv[8 * ks + 5]),
                                   pack_bf16x2(wv[8 * ks + 6], wv[8 * ks + 7])});
        }
        const float decay = __expf(T);
#pragma unroll
        for (int j = 0; j < FH; ++j) S[j] *= decay;
        Z *= decay;
      }
#pragma unroll
      for (int idx = 0; idx < NK; ++idx) {
        const int ks = idx / FH, j = idx % FH;
        const bf16x8 ka = kf[idx % KD];
        if (idx + KD < NK && (!AUG || (idx + KD) % FH < nlive))
          kf[idx % KD] = frag_tr(Ks, MP, ((idx + KD) / FH) * 16, (f0 + (idx + KD) % FH) * 32, lane);
        if (!AUG || j < nlive) {  // wave-uniform
          S[j] = mfma32x32x16(ka, vb[ks], S[j]);
          if (has_z && j == zj) Z = mfma32x32x16(ka, zb[ks], Z);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < nch) store(smem + ((c + 1) & 1) * G::BUF, wr, wrg);
    __syncthreads();
    // finish rows 16*half .. +15: own part + partner's part, normalise, store.
    // All LDS reads are issued before any arithmetic and the normalisation
    // branch covers the whole block, so the eight rows overlap instead of
    // running as eight dependent read-add-divide-store chains.
    {
      const int kept = half == 0 ? 0 : 8;
      const int partner = (1 - half) * NWD + dvt;
      // one batch of LDS reads: the partner's partial rows, and for the
      // denominator of row den_row its masked-weight row sum and z partials
      // (read whether or not they are used: the batch costs one round trip)
      float val[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] = xo[(partner * 8 + e) * 64 + lane];
      const int rq = den_row(kept, lane);
      const float rs = CAUSAL ? rsum[rq] : 0.f;
      const u32x4 lo = ld16(part + rq * 8), hi = ld16(part + rq * 8 + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] += pick(O[e], O[8 + e], half == 0);
      if (a.normalize && !DENOUT) {
        // v_rcp_f32 (1 ulp) and a product: far inside the bf16 operands' error
        scale_rows(val, __builtin_amdgcn_rcpf(den_sum<NWD, (FH < NWD ? FH : NWD)>(a.delta, rs, lo, hi)));
      }
      if constexpr (DENOUT) {
        // row q = lane of the first 32 lanes of wave 0: the same sum, in the
        // same order, from the exchange area (read only after the barrier)
        if (w == 0 && lane < kC && c0 + lane < t1) {
          den_out[bh * a.n + c0 + lane] = den_sum<NWD, (FH < NWD ? FH : NWD)>(
              a.delta, CAUSAL ? rsum[lane] : 0.f, ld16(part + lane * 8), ld16(part + lane * 8 + 4));
        }
      }
      // element e is row 8 * ((kept + e) / 4) + 4 * hh + e % 4 of the chunk; the
      // rows are written once and not read back here: non-temporal stores
      float* orow = Og + (c0 + 4 * hh) * DV + dvt * 32 + c32;
      if constexpr (OM != 0) {
        // destination row of this lane's first row c0 + 4hh, then rows r
        // further on (or back, reversed): wave-uniform offsets
        const int64_t tb = c0 + 4 * hh;
        const int64_t d0 = bh * a.n + ((OM & 1) ? a.n - 1 - tb : tb);
        constexpr int sgn = (OM & 1) ? -1 : 1;
        if constexpr ((OM & 2) != 0) {
          // lanes c32 and c32 ^ 1 hold the same rows of adjacent columns: a
          // DPP swap gives the even lane rows e, the odd lane rows e + 1 as
          // bf16 pairs (half the stores)
          uint32_t* ob = reinterpret_cast<uint32_t*>(outb + d0 * ldo + dvt * 32 + (c32 & ~1));
          const bool odd = (c32 & 1) != 0;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float send = odd ? val[e] : val[e + 1];
            const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(
                __float_as_int(send), 0xB1, 0xF, 0xF, false));  // quad_perm [1, 0, 3, 2]
            const int ee = odd ? e + 1 : e;
            const int r = 8 * ((kept + ee) >> 2) + (ee & 3);
            if (tb + r < t1)
              ob[sgn * r * (ldo / 2)] = odd ? pack_bf16x2(recv, val[e + 1]) : pack_bf16x2(val[e], recv);
          }
        } else {
          float* ob = out + d0 * DV + dvt * 32 + c32;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * ((kept + e) >> 2) + (e & 3);
            if (tb + r < t1) ob[sgn * r * DV] = val[e];
          }
        }
      } else if (c0 + kC <= t1) {  // whole chunk in range: no per-row checks
#pragma unroll
        for (int e = 0; e < 8; ++e) __builtin_nontemporal_store(val[e], &orow[(8 * ((kept + e) >> 2) + (e & 3)) * DV]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * ((kept + e) >> 2) + (e & 3);
          if (c0 + r + 4 * hh < t1) __builtin_nontemporal_store(val[e], &orow[r * DV]);
        }
      }
    }
  };

  u32x4 rA[LPT], rB[LPT];
  uint32_t gA = 0u, gB = 0u;
  load(chunk_at(0), rA, gA);
  load(chunk_at(1), rB, gB);
  // The prefix state must be in registers before the chunk loop: a wait for
  // it left to the compiler lands inside the loop and drains the chunk
  // prefetch on every chunk (and the scheduler sinks the state loads below a
  // plain s_waitcnt). An empty asm reading every state register makes the
  // wait happen here.
#pragma unroll
  for (int j = 0; j < FH; ++j) asm volatile("" : "+v"(S[j]));
  asm volatile("" : "+v"(Z));
  store(smem, rA, gA);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    step(c, rA, gA, rB, gB);
    if (c + 1 < nch) step(c + 1, rB, gB, rA, gA);
  }
}

// ============================================================================
// Fused pass 2: phi_Q projected inside the causal output pass
// ============================================================================
// phi_Q = featmap(Q) never reaches HBM (the pages' cost model is p*t small
// projections plus element-wise products, notes key design 2; here those
// projections run in the same kernel as the causal read-out). A workgroup
// walks its segment in blocks of 64 rows:
//   projection: wave w computes the 32-feature block w of the block's rows,
//     Y_{j,r} = X_Q Theta_{j,r} on MFMA with the X rows staged in LDS and the
//     Theta fragments streamed from the fragment-order copy (the layout the
//     feature-map kernel reads) straight into registers, then the Hadamard
//     product over j, the sum over r and the square in registers, rounded to
//     bf16 into an LDS block buffer. The products and the epilogue run in the
//     feature-map kernel's order, so phi_Q is bit for bit the one that kernel
//     stores;
//   read-out: the block's two 32-token chunks run exactly as attn_out32's
//     (same waves, same exchange, same arithmetic), phi_Q read from the block
//     buffer, phi_K and V streamed per chunk.
// The workgroup needs m = 2 dv (one feature block per wave).
template <int M, int DV, int D, int P, int T>
struct Fq32Geom {
  static constexpr int NWD = DV / 32;      // value-column tiles
  static constexpr int NW = 2 * NWD;       // waves
  static constexpr int NT = NW * 64;
  static constexpr int FT = M / 32;
  static constexpr int FH = FT / 2;
  static constexpr int RB = 2 * kC;        // rows per projected block
  static constexpr int KS = D / 16;        // 16-deep k-steps of the projection
  static constexpr int QPAD = M + 8, MP = lds_stride(M, 24), VP = lds_stride(DV, 32);
  static constexpr int XP = D + 8;         // X rows 16 bytes apart mod 256: b128 reads conflict-free
  static constexpr int QB = RB * QPAD;     // phi_Q block buffer (elements)
  static constexpr int XB = RB * XP;       // X_Q block buffer
  static constexpr int BUF = kC * MP + kC * VP;  // one chunk: phi_K, V
  static constexpr int KPc = kC * M / 8, VPc = kC * DV / 8;  // 16-byte pieces per chunk
  static constexpr int LPT = (KPc + VPc) / NT;
  static constexpr int LX = RB * D / 8 / NT;  // 16-byte X pieces per thread per block
  static constexpr int XO = NW * 8 * 64, PART = kC * 8, EXW = XO + PART + kC;
  static constexpr int NFR = T * P * KS;   // Theta fragments of one feature block
  static constexpr int TPD = 4;            // Theta fragments in flight per wave
  static constexpr bool STREAM_NT = true;  // phi_K, V and X loads marked non-temporal
  static constexpr size_t lds_bytes() { return 2ull * (QB + XB + 2 * BUF) + 2ull * EXW * 4; }
  static_assert(lds_bytes() <= 160 * 1024, "LDS per workgroup");
  static_assert(FT == NW, "one 32-feature block per wave in the projection");
  static_assert(D % 32 == 0 && FT % 2 == 0, "shape");
  static_assert(KPc % NT == 0 && VPc % NT == 0 && (RB * D / 8) % NT == 0, "even split");
  static_assert(NW <= 8, "z partial slots");
};

template <int M, int DV, int D, int P, int T>
__global__ __launch_bounds__(DV * 4) __attribute__((amdgpu_waves_per_eu(2)))
void attn_out32_fq(Seg32Args a, const uint16_t* __restrict__ xq,
                   const uint16_t* __restrict__ thpk, int64_t pk_hstride, int64_t H, int square,
                   const uint16_t* __restrict__ phik, const uint16_t* __restrict__ v,
                   const float* __restrict__ state, int64_t st_seg, int64_t st_bh,
                   float* __restrict__ out) {
  using G = Fq32Geom<M, DV, D, P, T>;
  constexpr int FH = G::FH, QPAD = G::QPAD, MP = G::MP, VP = G::VP, XP = G::XP, NT = G::NT;
  constexpr int NWD = G::NWD, KS = G::KS, LPT = G::LPT, LX = G::LX, KPc = G::KPc;
  constexpr int NFR = G::NFR, TPD = G::TPD < G::NFR ? G::TPD : G::NFR;
  extern __shared__ __align__(16) uint16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: see attn pass 1
  const int dvt = w % NWD, half = w / NWD;
  const int f0 = half * FH;
  const bool has_z = dvt < FH;
  const int zj = dvt;
  const int c32 = lane & 31, hh = lane >> 5;
  // XCD-aware work order: workgroups are dispatched to the 8 XCDs round
  // robin (id % 8), so workgroup id takes sequence bh = xcd * BH/8 + k / nseg
  // with k = id / 8: the workgroups on one XCD walk the segments of BH/8
  // sequences and their heads' Theta_Q stays in that XCD's L2 instead of
  // every XCD streaming every head's
  const int64_t BH = static_cast<int64_t>(gridDim.x) / a.nseg;
  const int64_t id = blockIdx.x;
  int64_t bh;
  int gseg;
  if (BH % 8 == 0) {
    const int64_t k = id / 8;
    bh = (id % 8) * (BH / 8) + k / a.nseg;
    gseg = static_cast<int>(k % a.nseg);
  } else {
    bh = id / a.nseg;
    gseg = static_cast<int>(id % a.nseg);
  }
  const int64_t t0 = gseg * a.seg_len;
  const int64_t t1 = min(a.n, t0 + a.seg_len);
  const uint16_t* Xg = xq + bh * a.n * D;
  const uint16_t* Kg = phik + bh * a.n * M;
  const uint16_t* Vg = v + bh * a.n * DV;
  float* Og = out + bh * a.n * DV;
  const float* Sin = state + bh * st_bh + gseg * st_seg;
  const int nch = static_cast<int>((t1 - t0 + kC - 1) / kC);
  uint16_t* Qb = smem;                 // [RB][QPAD] phi_Q of the current block
  uint16_t* Xs = Qb + G::QB;           // [RB][XP]   X_Q rows of the block to project
  uint16_t* cbuf = Xs + G::XB;         // 2 x [phi_K | V] chunk buffers
  float* exbase = reinterpret_cast<float*>(cbuf + 2 * G::BUF);

  f32x16 S[FH], Z;
#pragma unroll
  for (int j = 0; j < FH; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[j][4 * i + e] = Sin[((f0 + j) * 32 + 8 * i + 4 * hh + e) * DV + dvt * 32 + c32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Z[4 * i + e] = has_z ? Sin[static_cast<int64_t>(M) * DV + (f0 + zj) * 32 + 8 * i + 4 * hh + e] : 0.f;
  const bf16x8 ones = as_bf16x8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  // Raw buffer views of this segment's rows (zeros past the segment end) and
  // of this wave's feature block of the fragment-order Theta_Q: fragment
  // (r, j, ks) is 1 KiB at byte ((r * P + j) * KS + ks) * 1024, lane l's 16
  // bytes at 16 l.
  const uint32_t seg_rows = static_cast<uint32_t>(t1 - t0);
  const __amdgpu_buffer_rsrc_t rsx = make_rsrc(Xg + t0 * D, seg_rows * D * 2u);
  const __amdgpu_buffer_rsrc_t rsk = make_rsrc(Kg + t0 * M, seg_rows * M * 2u);
  const __amdgpu_buffer_rsrc_t rsv = make_rsrc(Vg + t0 * DV, seg_rows * DV * 2u);
  const int64_t h = bh % H;
  const __amdgpu_buffer_rsrc_t rst =
      make_rsrc(thpk + h * pk_hstride + static_cast<int64_t>(w) * NFR * 512, NFR * 1024u);

  auto load = [&](int c, u32x4 (&r)[LPT]) {
    int t = tid;  // opaque: per-piece offsets are rebuilt, not kept live
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int p = t + i * NT;
      if (i * NT < KPc)
        r[i] = G::STREAM_NT ? buf_ld16_nt(rsk, p * 16u, static_cast<uint32_t>(c) * (kC * M * 2u))
                     : buf_ld16(rsk, p * 16u, static_cast<uint32_t>(c) * (kC * M * 2u));
      else
        r[i] = G::STREAM_NT ? buf_ld16_nt(rsv, (p - KPc) * 16u, static_cast<uint32_t>(c) * (kC * DV * 2u))
                     : buf_ld16(rsv, (p - KPc) * 16u, static_cast<uint32_t>(c) * (kC * DV * 2u));
    }
  };
  auto store = [&](uint16_t* buf, const u32x4 (&r)[LPT]) {
    int t = tid;
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int p = t + i * NT;
      uint16_t* dst;
      if (i * NT < KPc) {
        dst = buf + (p / (M / 8)) * MP + (p % (M / 8)) * 8;
      } else {
        const int pp = p - KPc;
        dst = buf + kC * MP + (pp / (DV / 8)) * VP + (pp % (DV / 8)) * 8;
      }
      st16(dst, r[i]);
    }
  };
  // X_Q rows of block blk (64 rows from the segment's row 64 blk)
  auto load_x = [&](int blk, u32x4 (&r)[LX]) {
#pragma unroll
    for (int i = 0; i < LX; ++i)
      r[i] = G::STREAM_NT ? buf_ld16_nt(rsx, (tid + i * NT) * 16u, static_cast<uint32_t>(blk) * (G::RB * D * 2u))
                   : buf_ld16(rsx, (tid + i * NT) * 16u, static_cast<uint32_t>(blk) * (G::RB * D * 2u));
  };
  auto store_x = [&](const u32x4 (&r)[LX]) {
#pragma unroll
    for (int i = 0; i < LX; ++i) {
      const int p = tid + i * NT;
      st16(Xs + (p / (D / 8)) * XP + (p % (D / 8)) * 8, r[i]);
    }
  };

  // Projection of the block in Xs into Qb: feature block w, both 32-row
  // tiles. Loop order r, ks, j: each X fragment pair is read once per (r, ks)
  // and feeds P Theta fragments; Theta fragments stream TPD ahead.
  auto project = [&]() {
    auto toff = [](int f) {  // byte offset of the f-th fragment in loop order
      const int r = f / (KS * P), ks = (f / P) % KS, j = f % P;
      return static_cast<uint32_t>(((r * P + j) * KS + ks) * 1024);
    };
    // lane-dependent bases pass through an empty asm: hoisted out of the block
    // loop, every derived address of the unrolled projection stays live
    uint32_t tl = lane * 16u;
    asm volatile("" : "+v"(tl));
    int xl = c32 * XP + 8 * hh;
    asm volatile("" : "+v"(xl));
    const uint16_t* xb = Xs + xl;
    bf16x8 tf[TPD];
#pragma unroll
    for (int f = 0; f < TPD; ++f) tf[f] = as_bf16x8(buf_ld16(rst, tl, toff(f)));
    f32x16 sum[2] = {zero16(), zero16()};
#pragma unroll
    for (int r = 0; r < T; ++r) {
      f32x16 acc[P][2];
#pragma unroll
      for (int j = 0; j < P; ++j) acc[j][0] = acc[j][1] = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // X rows 0..31 and 32..63 of the block, k = 16 ks + 8 hh .. +7
        const bf16x8 x0 = as_bf16x8(ld16(xb + ks * 16));
        const bf16x8 x1 = as_bf16x8(ld16(xb + 32 * XP + ks * 16));
#pragma unroll
        for (int j = 0; j < P; ++j) {
          const int f = (r * KS + ks) * P + j;
          const bf16x8 ta = tf[f % TPD];
          if (f + TPD < NFR) tf[f % TPD] = as_bf16x8(buf_ld16(rst, tl, toff(f + TPD)));
          acc[j][0] = mfma32x32x16(ta, x0, acc[j][0]);
          acc[j][1] = mfma32x32x16(ta, x1, acc[j][1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Hadamard product over j, sum over r (the feature-map kernel's order)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        if constexpr (P == 1) {
          sum[rt] += acc[0][rt];
        } else {
          f32x16 prod = acc[0][rt];
#pragma unroll
          for (int j = 1; j + 1 < P; ++j) prod *= acc[j][rt];
#pragma unroll
          for (int e = 0; e < 16; ++e) sum[rt][e] = fmaf(prod[e], acc[P - 1][rt][e], sum[rt][e]);
        }
      }
      // the rank's epilogue happens here: left alone, the compiler sinks every
      // rank's products below the last rank's MFMAs and keeps all T ranks'
      // accumulators live at once
      asm volatile("" : "+v"(sum[0]), "+v"(sum[1]));
    }
    // square, round to bf16, regroup so each lane holds 16 contiguous bytes of
    // its row (lanes c32 and c32 + 32 share row c32), store into the block buffer
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x16 x = sum[rt];
      if (square) x *= x;
      uint32_t wv[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wv[i][0] = pack_bf16x2(x[4 * i], x[4 * i + 1]);
        wv[i][1] = pack_bf16x2(x[4 * i + 2], x[4 * i + 3]);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        swap_halves(wv[0][e], wv[1][e]);
        swap_halves(wv[2][e], wv[3][e]);
      }
      int ql = (rt * 32 + c32) * QPAD + w * 32 + 8 * hh;
      asm volatile("" : "+v"(ql));
      uint16_t* dst = Qb + ql;
      st16(dst, u32x4{wv[0][0], wv[0][1], wv[1][0], wv[1][1]});
      st16(dst + 16, u32x4{wv[2][0], wv[2][1], wv[3][0], wv[3][1]});
    }
  };

  // one chunk, as attn_out32's causal ungated step, except that chunk c+1
  // is requested at the start of chunk c (one ahead, into rc) and staged at
  // its end: no chunk load is in flight during a projection, which leaves
  // the projection its registers
  auto step = [&](int c, int qrow, u32x4 (&rc)[LPT], f32x16& O) {
    if (c + 1 < nch) load(c + 1, rc);
    int lbase = (c & 1) * G::BUF;
    asm volatile("" : "+v"(lbase));
    int lim = c32 - 4 * hh;  // key 8i+4hh+e reaches query c32 iff 8i+e <= lim
    asm volatile("" : "+v"(lim));
    int qbase = qrow * QPAD;
    asm volatile("" : "+v"(qbase));
    const uint16_t* Qs = Qb + qbase;
    const uint16_t* Ks = cbuf + lbase;
    const uint16_t* Vs = Ks + kC * MP;
    int exoff = (c & 1) * G::EXW;
    asm volatile("" : "+v"(exoff));
    float* ex = exbase + exoff;
    float* xo = ex;
    float* part = ex + G::XO;
    float* rsum = part + G::PART;

    O = zero16();
    f32x16 D2 = zero16();
    if (half == 0) {
      // masked A^T = phi_K phi_Q^T (keys x queries); reads AD k-steps ahead
      constexpr int KSA = M / 16, AD = KSA < 3 ? KSA : 3;
      f32x16 At = zero16();
      bf16x8 fk[AD], fq[AD];
#pragma unroll
      for (int i = 0; i < AD; ++i) {
        fk[i] = frag_nat(Ks, MP, 0, i * 16, lane);
        fq[i] = frag_nat(Qs, QPAD, 0, i * 16, lane);
      }
#pragma unroll
      for (int ks = 0; ks < KSA; ++ks) {
        const bf16x8 ka = fk[ks % AD], qb = fq[ks % AD];
        if (ks + AD < KSA) {
          fk[ks % AD] = frag_nat(Ks, MP, 0, (ks + AD) * 16, lane);
          fq[ks % AD] = frag_nat(Qs, QPAD, 0, (ks + AD) * 16, lane);
        }
        At = mfma32x32x16(ka, qb, At);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (8 * i + e > lim) At[4 * i + e] = 0.f;  // key after query
      bf16x8 afr[2];
      afr[0] = acc_frag(At, 0);
      afr[1] = acc_frag(At, 1);
      if (a.normalize && dvt == 0) {  // row sums of the rounded weights A V uses
        float rs = 0.f;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const u32x4 u = __builtin_bit_cast(u32x4, afr[hf]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            rs += __uint_as_float(u[q] << 16) + __uint_as_float(u[q] & 0xFFFF0000u);
        }
        rs += __shfl_xor(rs, 32);
        if (hh == 0) rsum[c32] = rs;
      }
#pragma unroll
      for (int ks = 0; ks < kC / 16; ++ks)
        O = mfma32x32x16(afr[ks], frag_tr(Vs, VP, ks * 16, dvt * 32, lane), O);
    }
    __builtin_amdgcn_sched_barrier(0);
    {  // partial phi_Q S over this wave's feature half; phi_Q . z over its z tile
      constexpr int NQ = 2 * FH, QD = NQ < 2 ? NQ : 2;
      bf16x8 qf[QD];
#pragma unroll
      for (int i = 0; i < QD; ++i) qf[i] = frag_p16_sep(Qs, QPAD, 0, f0 * 32 + i * 16, lane);
#pragma unroll
      for (int idx = 0; idx < NQ; ++idx) {
        const int j = idx >> 1, hf = idx & 1;
        const bf16x8 qa = qf[idx % QD];
        if (idx + QD < NQ) qf[idx % QD] = frag_p16_sep(Qs, QPAD, 0, f0 * 32 + (idx + QD) * 16, lane);
        O = mfma32x32x16(qa, acc_frag(S[j], hf), O);
        if (a.normalize && has_z && j == zj) D2 = mfma32x32x16(qa, acc_frag(Z, hf), D2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    {  // publish: the 16 rows the partner wave finishes, and the z partial
#pragma unroll
      for (int e = 0; e < 8; ++e) xo[(w * 8 + e) * 64 + lane] = pick(O[8 + e], O[e], half == 0);
      if (a.normalize && has_z && c32 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) part[(8 * i + 4 * hh + e) * 8 + w] = D2[4 * i + e];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    {  // S += phi_K^T V, z += phi_K^T 1; phi_K reads run KD ahead
      constexpr int NK = (kC / 16) * FH, KD = NK < 2 ? NK : 2;
      bf16x8 kf[KD];
#pragma unroll
      for (int i = 0; i < KD; ++i) kf[i] = frag_tr(Ks, MP, (i / FH) * 16, (f0 + i % FH) * 32, lane);
      bf16x8 vb[kC / 16];
#pragma unroll
      for (int ks = 0; ks < kC / 16; ++ks) vb[ks] = frag_tr(Vs, VP, ks * 16, dvt * 32, lane);
#pragma unroll
      for (int idx = 0; idx < NK; ++idx) {
        const int ks = idx / FH, j = idx % FH;
        const bf16x8 ka = kf[idx % KD];
        if (idx + KD < NK)
          kf[idx % KD] = frag_tr(Ks, MP, ((idx + KD) / FH) * 16, (f0 + (idx + KD) % FH) * 32, lane);
        S[j] = mfma32x32x16(ka, vb[ks], S[j]);
        if (has_z && j == zj) Z = mfma32x32x16(ka, ones, Z);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < nch) store(cbuf + ((c + 1) & 1) * G::BUF, rc);
  };
  // finish rows 16 half .. +15 of chunk c (after the chunk's barrier)
  auto finish = [&](int c, const f32x16& O) {
    int exoff = (c & 1) * G::EXW;
    asm volatile("" : "+v"(exoff));
    const float* ex = exbase + exoff;
    const float* xo = ex;
    const float* part = ex + G::XO;
    const float* rsum = part + G::PART;
    const int64_t c0 = t0 + static_cast<int64_t>(c) * kC;
    const int kept = half == 0 ? 0 : 8;
    const int partner = (1 - half) * NWD + dvt;
    float val[8];  // as attn_out32's finish: one batch of LDS reads
#pragma unroll
    for (int e = 0; e < 8; ++e) val[e] = xo[(partner * 8 + e) * 64 + lane];
    const int rq = den_row(kept, lane);
    const float rs = rsum[rq];
    const u32x4 lo = ld16(part + rq * 8), hi = ld16(part + rq * 8 + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) val[e] += pick(O[e], O[8 + e], half == 0);
    if (a.normalize)
      scale_rows(val, __builtin_amdgcn_rcpf(den_sum<NWD, (FH < NWD ? FH : NWD)>(a.delta, rs, lo, hi)));
    // rows written once: non-temporal stores, as in attn_out32
    float* orow = Og + (c0 + 4 * hh) * DV + dvt * 32 + c32;
    if (c0 + kC <= t1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) __builtin_nontemporal_store(val[e], &orow[(8 * ((kept + e) >> 2) + (e & 3)) * DV]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * ((kept + e) >> 2) + (e & 3);
        if (c0 + r + 4 * hh < t1) __builtin_nontemporal_store(val[e], &orow[r * DV]);
      }
    }
  };

  u32x4 rc[LPT], rx[LX];
  load(0, rc);
  load_x(0, rx);
#pragma unroll
  for (int j = 0; j < FH; ++j) asm volatile("" : "+v"(S[j]));
  asm volatile("" : "+v"(Z));
  store(cbuf, rc);
  store_x(rx);
  __syncthreads();
  // Block blk: project its 64 rows (Xs -> Qb), barrier, then its two chunks.
  // The next block's X rows are loaded during the first chunk and stored
  // before that chunk's barrier (Xs is free once the projection's barrier
  // has passed); Qb is rewritten only after the second chunk's barrier, when
  // no wave reads it any more.
  const int nblk = (nch + 1) / 2;
  for (int blk = 0; blk < nblk; ++blk) {
    const int c = 2 * blk;
    project();
    __syncthreads();
    if (blk + 1 < nblk) load_x(blk + 1, rx);
    {
      f32x16 O;
      step(c, 0, rc, O);
      if (blk + 1 < nblk) store_x(rx);
      __syncthreads();
      finish(c, O);
    }
    if (c + 1 < nch) {
      f32x16 O;
      step(c + 1, kC, rc, O);
      __syncthreads();
      finish(c + 1, O);
    }
  }
}

// Chunk-local inclusive sums of the log gates: L[bh][t] = sum of g[bh][t']
// over t' from the start of t's 32-token chunk (chunks start at multiples of
// 32) to t, rows gl_ld(n) apart. The padding t in [n, gl_ld(n)) is written
// too (g taken as 0 there, so it repeats the last sum): the passes read whole
// 32-token chunks and every value they read is finite. One 32-lane group
// scans one chunk with lane shuffles.
__global__ __launch_bounds__(256) void gate_cumsum32(int64_t n, int64_t nch, int64_t total,
                                                     const float* __restrict__ g,
                                                     float* __restrict__ L) {
  const int64_t id = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  const int l = threadIdx.x & 31;
  const int64_t bh = id / nch, tok = (id % nch) * kC + l;
  const bool live = id < total;
  float x = live && tok < n ? g[bh * n + tok] : 0.f;
#pragma unroll
  for (int o = 1; o < kC; o <<= 1) {
    const float y = __shfl_up(x, o, kC);
    if (l >= o) x += y;
  }
  if (live) L[bh * nch * kC + tok] = x;
}

template <int M, int DV, bool GATED, bool ANCHOR = false, bool VSTR = false, bool AUG = false>
hipError_t launch_state_t(const AttnShape& s, const uint16_t* k, const uint16_t* v, const float* gl,
                          float* gseg, float* seg, hipStream_t st, int vld = 0, int kald = 0,
                          int kone = 0) {
  using G = Seg32Geom<M, DV>;
  Seg32Args a{s.n, s.seg_len, s.nseg, s.normalize, s.delta, gl, gseg, 0, kald, 0, kone};
  const size_t lds = 2ull * (kC * G::MP + kC * G::VP + (GATED ? kGL : 0)) * sizeof(uint16_t);
  auto* kern = seg_state32<M, DV, GATED, ANCHOR, VSTR, AUG>;
  const hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>(s.nseg), static_cast<unsigned>(s.BH));
  LLOPS_LAUNCH(GATED ? "seg_state_gated" : "seg_state_bf16", st, kern, grid, dim3(G::NT), lds, st,
               a, k, v, seg, vld);
  return hipGetLastError();
}

template <int M, int DV, bool CAUSAL, bool GATED, bool DENOUT = false, int OM = 0,
          bool VSTR = false, bool ANTI = false, bool AUG = false>
hipError_t launch_out_t(const AttnShape& s, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const float* gl, const float* state, int64_t ss,
                        int64_t sb, float* out, hipStream_t st, float* den = nullptr,
                        uint16_t* outb = nullptr, int ldo = 0, int vld = 0, int qald = 0,
                        int qone = 0, int kald = 0, int kone = 0) {
  using G = Out32Geom<M, DV, GATED>;
  Seg32Args a{s.n, s.seg_len, s.nseg, s.normalize, s.delta, gl, nullptr, qald, kald, qone, kone};
  const size_t lds = G::lds_bytes();
  if ((s.anti != 0) != ANTI) return hipErrorInvalidValue;
  auto* kern = attn_out32<M, DV, CAUSAL, GATED, DENOUT, OM, VSTR, ANTI, AUG>;
  const hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>(s.nseg), static_cast<unsigned>(s.BH));
  LLOPS_LAUNCH(GATED ? "attn_out_gated" : "attn_out_bf16", st, kern, grid, dim3(G::NT), lds, st,
               a, q, k, v, state, ss, sb, out, den, outb, ldo, vld);
  return hipGetLastError();
}

template <int M, int DV, int D, int P, int T>
hipError_t launch_fq_t(const AttnShape& s, const uint16_t* xq, const uint16_t* thpk,
                       int64_t pk_hstride, int64_t H, int square, const uint16_t* k,
                       const uint16_t* v, const float* state, int64_t ss, int64_t sb, float* out,
                       hipStream_t st) {
  using G = Fq32Geom<M, DV, D, P, T>;
  Seg32Args a{s.n, s.seg_len, s.nseg, s.normalize, s.delta, nullptr, nullptr};
  const size_t lds = G::lds_bytes();
  auto* kern = attn_out32_fq<M, DV, D, P, T>;
  const hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  if (s.BH * s.nseg > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(s.BH * s.nseg));  // one workgroup per (segment, sequence)
  LLOPS_LAUNCH("attn_out_fq", st, kern, grid, dim3(G::NT), lds, st, a, xq, thpk, pk_hstride, H,
               square, k, v, state, ss, sb, out);
  return hipGetLastError();
}

int key32(const AttnShape& s) {
  if (s.seg_len % kC != 0) return 0;
  // buffer views of one segment's rows need byte offsets below 2^31
  if (s.seg_len * (s.m > s.dv ? s.m : s.dv) * 2 >= (int64_t{1} << 31)) return 0;
  return s.m * 1000 + s.dv;
}

}  // namespace

bool attn32_supported(const AttnShape& s) {
  switch (key32(s)) {
    case 256128:
    case 128064:
    case 64064: return true;
    default: return false;
  }
}

hipError_t launch_seg_state32(const AttnShape& s, const uint16_t* phik, const uint16_t* v,
                              float* seg, hipStream_t st) {
  switch (key32(s)) {
    case 256128: return launch_state_t<256, 128, false>(s, phik, v, nullptr, nullptr, seg, st);
    case 128064: return launch_state_t<128, 64, false>(s, phik, v, nullptr, nullptr, seg, st);
    case 64064: return launch_state_t<64, 64, false>(s, phik, v, nullptr, nullptr, seg, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_out32(const AttnShape& s, const uint16_t* phiq, const uint16_t* phik,
                             const uint16_t* v, const float* state, int64_t st_seg,
                             int64_t st_bh, float* out, hipStream_t st) {
  const float* g = nullptr;
  if (s.anti) {  // anti-causal, fp32 rows (the backward's dV pass)
    if (!s.causal) return hipErrorInvalidValue;
    switch (key32(s)) {
      case 256128: return launch_out_t<256, 128, true, false, false, 0, false, true>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st);
      case 128064: return launch_out_t<128, 64, true, false, false, 0, false, true>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st);
      case 64064: return launch_out_t<64, 64, true, false, false, 0, false, true>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (key32(s) * 2 + (s.causal ? 1 : 0)) {
    case 256128 * 2 + 1: return launch_out_t<256, 128, true, false>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st);
    case 256128 * 2: return launch_out_t<256, 128, false, false>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st);
    case 128064 * 2 + 1: return launch_out_t<128, 64, true, false>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st);
    case 128064 * 2: return launch_out_t<128, 64, false, false>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st);
    case 64064 * 2 + 1: return launch_out_t<64, 64, true, false>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st);
    case 64064 * 2: return launch_out_t<64, 64, false, false>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_out32_den(const AttnShape& s, const uint16_t* phiq, const uint16_t* phik,
                                 const uint16_t* v, const float* state, int64_t st_seg,
                                 int64_t st_bh, float* out, float* den, hipStream_t st) {
  if (!s.normalize || !den) return hipErrorInvalidValue;
  const float* g = nullptr;
  switch (key32(s) * 2 + (s.causal ? 1 : 0)) {
    case 256128 * 2 + 1: return launch_out_t<256, 128, true, false, true>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st, den);
    case 256128 * 2: return launch_out_t<256, 128, false, false, true>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st, den);
    case 128064 * 2 + 1: return launch_out_t<128, 64, true, false, true>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st, den);
    case 128064 * 2: return launch_out_t<128, 64, false, false, true>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st, den);
    case 64064 * 2 + 1: return launch_out_t<64, 64, true, false, true>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st, den);
    case 64064 * 2: return launch_out_t<64, 64, false, false, true>(s, phiq, phik, v, g, state, st_seg, st_bh, out, st, den);
    default: return hipErrorInvalidValue;
  }
}

template <int M, int DV>
hipError_t launch_out_om(const AttnShape& s, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const float* state, int64_t ss, int64_t sb,
                         float* out, uint16_t* outb, int ldo, int rev, hipStream_t st,
                         int vld) {
  const int om = (outb ? 2 : 0) | (rev ? 1 : 0);
  const float* g = nullptr;
  if (s.anti) {  // the backward's suffix passes: bf16 rows in place from a value slice
    if (!s.causal || om != 2 || !vld) return hipErrorInvalidValue;
    return launch_out_t<M, DV, true, false, false, 2, true, true>(s, q, k, v, g, state, ss, sb, out, st, nullptr, outb, ldo, vld);
  }
  if (vld) {  // value rows vld apart: the backward's bf16 passes only
    if (om == 2 && !s.causal)
      return launch_out_t<M, DV, false, false, false, 2, true>(s, q, k, v, g, state, ss, sb, out, st, nullptr, outb, ldo, vld);
    if (om == 2)
      return launch_out_t<M, DV, true, false, false, 2, true>(s, q, k, v, g, state, ss, sb, out, st, nullptr, outb, ldo, vld);
    if (om == 3 && s.causal)
      return launch_out_t<M, DV, true, false, false, 3, true>(s, q, k, v, g, state, ss, sb, out, st, nullptr, outb, ldo, vld);
    return hipErrorInvalidValue;
  }
  if (!s.causal) {
    if (om != 2) return hipErrorInvalidValue;
    return launch_out_t<M, DV, false, false, false, 2>(s, q, k, v, g, state, ss, sb, out, st, nullptr, outb, ldo);
  }
  switch (om) {
    case 1: return launch_out_t<M, DV, true, false, false, 1>(s, q, k, v, g, state, ss, sb, out, st, nullptr, outb, ldo);
    case 2: return launch_out_t<M, DV, true, false, false, 2>(s, q, k, v, g, state, ss, sb, out, st, nullptr, outb, ldo);
    case 3: return launch_out_t<M, DV, true, false, false, 3>(s, q, k, v, g, state, ss, sb, out, st, nullptr, outb, ldo);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_out32_to(const AttnShape& s, const uint16_t* phiq, const uint16_t* phik,
                                const uint16_t* v, const float* state, int64_t st_seg,
                                int64_t st_bh, float* out, uint16_t* outb, int ldo, int rev,
                                hipStream_t st, int vld) {
  if (outb ? ldo < s.dv : !out) return hipErrorInvalidValue;
  if (vld && (vld < s.dv || s.n * vld * 2 >= (int64_t{1} << 31))) return hipErrorInvalidValue;
  switch (key32(s)) {
    case 256128: return launch_out_om<256, 128>(s, phiq, phik, v, state, st_seg, st_bh, out, outb, ldo, rev, st, vld);
    case 128064: return launch_out_om<128, 64>(s, phiq, phik, v, state, st_seg, st_bh, out, outb, ldo, rev, st, vld);
    case 64064: return launch_out_om<64, 64>(s, phiq, phik, v, state, st_seg, st_bh, out, outb, ldo, rev, st, vld);
    default: return hipErrorInvalidValue;
  }
}

// (d, p, t) of the fused output pass per (m, dv): m = 2 dv, one 32-feature
// block per wave
int fq_key(const AttnShape& s, int d, int p, int t) {
  if (!s.causal) return 0;
  const int k = key32(s);
  if (k == 256128 && d == 128 && p == 2 && t == 4) return 1;
  if (k == 128064 && d == 64 && p == 3 && t == 8) return 2;
  return 0;
}

bool attn32_fq_supported(const AttnShape& s, int d, int p, int t) {
  // X rows of a segment are addressed through a 32-bit buffer view
  return fq_key(s, d, p, t) != 0 && s.seg_len * d * 2 < (int64_t{1} << 31);
}

hipError_t launch_attn_out32_fq(const AttnShape& s, int d, int p, int t, const uint16_t* xq,
                                const uint16_t* thpk, int64_t pk_hstride, int64_t H, int square,
                                const uint16_t* phik, const uint16_t* v, const float* state,
                                int64_t st_seg, int64_t st_bh, float* out, hipStream_t st) {
  if (!attn32_fq_supported(s, d, p, t) || H < 1 || s.anti) return hipErrorInvalidValue;
  switch (fq_key(s, d, p, t)) {
    case 1: return launch_fq_t<256, 128, 128, 2, 4>(s, xq, thpk, pk_hstride, H, square, phik, v, state, st_seg, st_bh, out, st);
    case 2: return launch_fq_t<128, 64, 64, 3, 8>(s, xq, thpk, pk_hstride, H, square, phik, v, state, st_seg, st_bh, out, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_seg_state32_v(const AttnShape& s, const uint16_t* phik, const uint16_t* v,
                                int vld, float* seg, hipStream_t st) {
  if (vld < s.dv || s.n * vld * 2 >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  switch (key32(s)) {
    case 256128: return launch_state_t<256, 128, false, false, true>(s, phik, v, nullptr, nullptr, seg, st, vld);
    case 128064: return launch_state_t<128, 64, false, false, true>(s, phik, v, nullptr, nullptr, seg, st, vld);
    case 64064: return launch_state_t<64, 64, false, false, true>(s, phik, v, nullptr, nullptr, seg, st, vld);
    default: return hipErrorInvalidValue;
  }
}

// a narrow row of ald bf16 (and a one at column ald) within the live tiles
bool aug_ok(const AttnShape& s, int ald, int one) {
  return ald > 0 && ald % 8 == 0 && ald + (one ? 1 : 0) <= kAugTiles * 32 &&
         s.seg_len * ald * 2 < (int64_t{1} << 31) && s.n * ald * 2 < (int64_t{1} << 31);
}

bool aug32_supported(const AttnShape& s) { return key32(s) == 256128; }

hipError_t launch_seg_state32_aug(const AttnShape& s, const uint16_t* phik, int kald, int kone,
                                  const uint16_t* v, int vld, float* seg, hipStream_t st) {
  if (!aug32_supported(s) || !aug_ok(s, kald, kone) || vld < s.dv ||
      s.n * vld * 2 >= (int64_t{1} << 31))
    return hipErrorInvalidValue;
  return launch_state_t<256, 128, false, false, true, true>(s, phik, v, nullptr, nullptr, seg, st,
                                                            vld, kald, kone);
}

hipError_t launch_attn_out32_aug(const AttnShape& s, const uint16_t* phiq, int qald, int qone,
                                 const uint16_t* phik, int kald, int kone, const uint16_t* v,
                                 int vld, const float* state, int64_t st_seg, int64_t st_bh,
                                 uint16_t* outb, int ldo, hipStream_t st) {
  if (!aug32_supported(s) || !aug_ok(s, qald, qone) || !aug_ok(s, kald, kone) || !outb ||
      vld < s.dv || s.n * vld * 2 >= (int64_t{1} << 31))
    return hipErrorInvalidValue;
  const float* g = nullptr;
  if (s.anti) {
    if (!s.causal) return hipErrorInvalidValue;
    return launch_out_t<256, 128, true, false, false, 2, true, true, true>(
        s, phiq, phik, v, g, state, st_seg, st_bh, nullptr, st, nullptr, outb, ldo, vld, qald,
        qone, kald, kone);
  }
  if (s.causal)
    return launch_out_t<256, 128, true, false, false, 2, true, false, true>(
        s, phiq, phik, v, g, state, st_seg, st_bh, nullptr, st, nullptr, outb, ldo, vld, qald,
        qone, kald, kone);
  return launch_out_t<256, 128, false, false, false, 2, true, false, true>(
      s, phiq, phik, v, g, state, st_seg, st_bh, nullptr, st, nullptr, outb, ldo, vld, qald, qone,
      kald, kone);
}

hipError_t launch_seg_state32_gated_aug(const AttnShape& s, const uint16_t* phik, int kald, int kone,
                                        const uint16_t* v, int vld, const float* gl, float* gseg,
                                        float* seg, bool anchored, hipStream_t st) {
  if (s.anti || !aug32_supported(s) || !aug_ok(s, kald, kone) || vld < s.dv ||
      s.n * vld * 2 >= (int64_t{1} << 31))
    return hipErrorInvalidValue;
  if (anchored)
    return launch_state_t<256, 128, true, true, true, true>(s, phik, v, gl, gseg, seg, st, vld,
                                                            kald, kone);
  return launch_state_t<256, 128, true, false, true, true>(s, phik, v, gl, gseg, seg, st, vld,
                                                           kald, kone);
}

hipError_t launch_attn_out32_gated_aug(const AttnShape& s, const uint16_t* phiq, int qald, int qone,
                                       const uint16_t* phik, int kald, int kone,
                                       const uint16_t* v, int vld, const float* gl,
                                       const float* state, float* out, hipStream_t st) {
  if (!s.causal || !aug32_supported(s) || !aug_ok(s, qald, qone) || !aug_ok(s, kald, kone) ||
      vld < s.dv || s.n * vld * 2 >= (int64_t{1} << 31))
    return hipErrorInvalidValue;
  const int64_t per = 256 * 128 + 256;
  if (s.anti)  // suffix sums over start-anchored segment states (slot g + 1)
    return launch_out_t<256, 128, true, true, false, 0, true, true, true>(
        s, phiq, phik, v, gl, state, per, per * s.nseg, out, st, nullptr, nullptr, 0, vld, qald,
        qone, kald, kone);
  return launch_out_t<256, 128, true, true, false, 0, true, false, true>(
      s, phiq, phik, v, gl, state, per, per * s.nseg, out, st, nullptr, nullptr, 0, vld, qald, qone,
      kald, kone);
}

hipError_t launch_gate_cumsum32(int64_t BH, int64_t n, const float* g, float* L, hipStream_t st) {
  const int64_t nch = (n + kC - 1) / kC, total = BH * nch;
  if (total == 0) return hipSuccess;
  if ((total + 7) / 8 > 0x7fffffffLL) return hipErrorInvalidValue;
  LLOPS_LAUNCH("gate_cumsum32", st, gate_cumsum32, dim3(static_cast<unsigned>((total + 7) / 8)),
               dim3(256), 0, st, n, nch, total, g, L);
  return hipGetLastError();
}

hipError_t launch_seg_state32_gated(const AttnShape& s, const uint16_t* phik, const uint16_t* v,
                                    const float* gl, float* gseg, float* seg, hipStream_t st) {
  if (s.anti) return hipErrorInvalidValue;  // decayed sums depend on the direction
  switch (key32(s)) {
    case 256128: return launch_state_t<256, 128, true>(s, phik, v, gl, gseg, seg, st);
    case 128064: return launch_state_t<128, 64, true>(s, phik, v, gl, gseg, seg, st);
    case 64064: return launch_state_t<64, 64, true>(s, phik, v, gl, gseg, seg, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_seg_state32_anchored(const AttnShape& s, const uint16_t* phik,
                                      const uint16_t* v, const float* gl, float* gseg, float* seg,
                                      hipStream_t st) {
  if (s.anti) return hipErrorInvalidValue;
  switch (key32(s)) {
    case 256128: return launch_state_t<256, 128, true, true>(s, phik, v, gl, gseg, seg, st);
    case 128064: return launch_state_t<128, 64, true, true>(s, phik, v, gl, gseg, seg, st);
    case 64064: return launch_state_t<64, 64, true, true>(s, phik, v, gl, gseg, seg, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_out32_gated(const AttnShape& s, const uint16_t* phiq, const uint16_t* phik,
                                   const uint16_t* v, const float* gl, const float* state,
                                   float* out, hipStream_t st) {
  if (!s.causal) return hipErrorInvalidValue;
  const int64_t per = static_cast<int64_t>(s.m) * s.dv + s.m;
  switch (key32(s)) {
    case 256128: return launch_out_t<256, 128, true, true>(s, phiq, phik, v, gl, state, per, per * s.nseg, out, st);
    case 128064: return launch_out_t<128, 64, true, true>(s, phiq, phik, v, gl, state, per, per * s.nseg, out, st);
    case 64064: return launch_out_t<64, 64, true, true>(s, phiq, phik, v, gl, state, per, per * s.nseg, out, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_seg_state32_gated_v(const AttnShape& s, const uint16_t* phik, const uint16_t* v,
                                      int vld, const float* gl, float* gseg, float* seg,
                                      bool anchored, hipStream_t st) {
  if (vld < s.dv || s.n * vld * 2 >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  switch (key32(s) * 2 + (anchored ? 1 : 0)) {
    case 256128 * 2: return launch_state_t<256, 128, true, false, true>(s, phik, v, gl, gseg, seg, st, vld);
    case 256128 * 2 + 1: return launch_state_t<256, 128, true, true, true>(s, phik, v, gl, gseg, seg, st, vld);
    case 128064 * 2: return launch_state_t<128, 64, true, false, true>(s, phik, v, gl, gseg, seg, st, vld);
    case 128064 * 2 + 1: return launch_state_t<128, 64, true, true, true>(s, phik, v, gl, gseg, seg, st, vld);
    case 64064 * 2: return launch_state_t<64, 64, true, false, true>(s, phik, v, gl, gseg, seg, st, vld);
    case 64064 * 2 + 1: return launch_state_t<64, 64, true, true, true>(s, phik, v, gl, gseg, seg, st, vld);
    default: return hipErrorInvalidValue;
  }
}

template <int M, int DV>
hipError_t launch_out_gated_to(const AttnShape& s, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const float* gl, const float* state,
                               float* out, int rev, int vld, hipStream_t st) {
  const int64_t per = static_cast<int64_t>(M) * DV + M;
  if (s.anti) {  // suffix sums over start-anchored segment states (slot g + 1)
    if (rev) return hipErrorInvalidValue;
    if (vld)
      return launch_out_t<M, DV, true, true, false, 0, true, true>(s, q, k, v, gl, state, per, per * s.nseg, out, st, nullptr, nullptr, 0, vld);
    return launch_out_t<M, DV, true, true, false, 0, false, true>(s, q, k, v, gl, state, per, per * s.nseg, out, st);
  }
  if (vld && !rev)
    return launch_out_t<M, DV, true, true, false, 0, true>(s, q, k, v, gl, state, per, per * s.nseg, out, st, nullptr, nullptr, 0, vld);
  if (rev && !vld)
    return launch_out_t<M, DV, true, true, false, 1>(s, q, k, v, gl, state, per, per * s.nseg, out, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_out32_gated_to(const AttnShape& s, const uint16_t* phiq,
                                      const uint16_t* phik, const uint16_t* v, const float* gl,
                                      const float* state, float* out, int rev, int vld,
                                      hipStream_t st) {
  if (!s.causal) return hipErrorInvalidValue;
  if (vld && (vld < s.dv || s.n * vld * 2 >= (int64_t{1} << 31))) return hipErrorInvalidValue;
  switch (key32(s)) {
    case 256128: return launch_out_gated_to<256, 128>(s, phiq, phik, v, gl, state, out, rev, vld, st);
    case 128064: return launch_out_gated_to<128, 64>(s, phiq, phik, v, gl, state, out, rev, vld, st);
    case 64064: return launch_out_gated_to<64, 64>(s, phiq, phik, v, gl, state, out, rev, vld, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_out32_gated_den(const AttnShape& s, const uint16_t* phiq,
                                       const uint16_t* phik, const uint16_t* v, const float* gl,
                                       const float* state, float* out, float* den,
                                       hipStream_t st) {
  if (!s.causal || !s.normalize || !den) return hipErrorInvalidValue;
  const int64_t per = static_cast<int64_t>(s.m) * s.dv + s.m;
  switch (key32(s)) {
    case 256128: return launch_out_t<256, 128, true, true, true>(s, phiq, phik, v, gl, state, per, per * s.nseg, out, st, den);
    case 128064: return launch_out_t<128, 64, true, true, true>(s, phiq, phik, v, gl, state, per, per * s.nseg, out, st, den);
    case 64064: return launch_out_t<64, 64, true, true, true>(s, phiq, phik, v, gl, state, per, per * s.nseg, out, st, den);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace llops
