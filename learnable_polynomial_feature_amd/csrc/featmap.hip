// LLoPS feature map  phi(X) = sum_r prod_j X Theta_{j,r}  [squared after the r-sum]
// (papernotes.org LLoPS notes, key design 2; arXiv 2610.14219 Sec. 3).
//
// Three kernels: featmap_fast (bf16, (d, p, t) fixed at compile time, 32x32x16
// MFMA; described at its definition below) takes the shapes it is
// instantiated for; featmap_mfma (bf16, any shape the validation allows) and
// featmap_f32_kernel (fp32 inputs) take the rest.
//
// featmap_mfma: each workgroup owns 256 rows (4 waves x 64) of one head. A wave
// keeps its X rows resident as MFMA A-fragments for the whole kernel and
// walks the features 16 at a time; for every 16-feature block the Theta
// columns of all (j, r) pairs are staged, transposed to k-major rows, into a
// double-buffered LDS ring. The p*t projections of one feature block land in
// the same lane/register slots (one 16x16 accumulator per (j, r)), so the
// Hadamard product over j, the sum over r and the optional square run in
// registers and only phi (1/(p*t) of the projection output) is stored.
#include "device.h"
#include "kernels.h"

namespace llops {
namespace {

struct FeatArgs {
  FeatJob job[2];
  int64_t B, H, n;
  int p, t, m;
  int64_t theta_hstride;  // elements between heads' Theta blocks (0 = shared)
  int square, out_bf16;
  int fsplit;             // feature-block groups per row tile
  int fb_per_split;       // 16-feature blocks per group
  int tr;                 // CP ranks staged per LDS buffer
};

constexpr int kRowsPerWave = 64;

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void featmap_mfma(FeatArgs a) {
  constexpr int KS = (D + 31) / 32;  // 32-wide k-steps
  constexpr int LDSROW = D + 8;      // padded bf16 row (16 B pad: conflict-free b128 reads)
  constexpr int NT = NW * 64;
  constexpr int SB_PER_BLK = D / 4;  // 8x8 sub-blocks per (j, r) block of D x 16
  extern __shared__ __align__(16) uint16_t smem[];

  const FeatJob job = a.job[blockIdx.z];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int tile = blockIdx.x / a.fsplit;
  const int fs = blockIdx.x - tile * a.fsplit;
  const int64_t h = blockIdx.y;
  const int64_t R = a.B * a.n;
  const int64_t wrow0 = (int64_t)tile * (NW * kRowsPerWave) + wave * kRowsPerWave;

  // row r of head h lives at sequence row rho = (b*H + h)*n + tk, b = r / n.
  auto rho_of = [&](int64_t r) -> int64_t {
    const int64_t b = (a.B == 1) ? 0 : r / a.n;
    return (b * a.H + h) * a.n + (r - b * a.n);
  };

  // ---- X fragments: lane holds row (rt*16 + c16), k = ks*32 + 8g .. +7
  const uint16_t* X = static_cast<const uint16_t*>(job.X);
  bf16x8 xf[4][KS];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int64_t r = wrow0 + rt * 16 + c16;
    const bool ok = r < R;
    const uint16_t* src = X + (ok ? rho_of(r) : 0) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k0 = ks * 32 + g * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok && (D % 32 == 0 || k0 < D)) v = ld16(src + k0);
      xf[rt][ks] = as_bf16x8(v);
    }
  }
  // ---- output rows of this lane: rt*16 + 4g + i, stored as offsets from obase
  const int64_t obase = rho_of(wrow0 < R ? wrow0 : 0);
  int orel[4][4];
  bool ook[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = wrow0 + rt * 16 + g * 4 + i;
      ook[rt][i] = r < R;
      orel[rt][i] = ook[rt][i] ? static_cast<int>(rho_of(r) - obase) : 0;
    }

  const int FB = a.m / 16;
  const int fb_begin = fs * a.fb_per_split;
  const int fb_end = min(FB, fb_begin + a.fb_per_split);
  const int nrg = (a.t + a.tr - 1) / a.tr;
  const int nstages = (fb_end - fb_begin) * nrg;
  if (nstages <= 0) return;
  const uint16_t* th = static_cast<const uint16_t*>(job.theta) + h * a.theta_hstride;
  const int bufelems = a.p * a.tr * 16 * LDSROW;

  // ---- stage (fb, rg): Theta_{j, r0+rr}[:, fb*16 .. +15] for all j, rr
  u32x4 pre[8];
  auto stage_geom = [&](int s, int& fb, int& r0, int& trs) {
    fb = fb_begin + s / nrg;
    const int rg = s - (s / nrg) * nrg;
    r0 = rg * a.tr;
    trs = min(a.tr, a.t - r0);
  };
  auto load_stage = [&](int s) {
    int fb, r0, trs;
    stage_geom(s, fb, r0, trs);
    const int nsb = a.p * trs * SB_PER_BLK;
    if (tid < nsb) {
      const int blk = tid / SB_PER_BLK, rem = tid - blk * SB_PER_BLK;
      const int kb = rem >> 1, fh = rem & 1;
      const int j = blk / trs, rr = blk - j * trs;
      const uint16_t* src =
          th + ((static_cast<int64_t>(j) * a.t + r0 + rr) * D + kb * 8) * a.m + fb * 16 + fh * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) pre[i] = ld16(src + static_cast<int64_t>(i) * a.m);
    }
  };
  auto write_stage = [&](int s, uint16_t* buf) {
    int fb, r0, trs;
    stage_geom(s, fb, r0, trs);
    const int nsb = a.p * trs * SB_PER_BLK;
    if (tid < nsb) {
      const int blk = tid / SB_PER_BLK, rem = tid - blk * SB_PER_BLK;
      const int kb = rem >> 1, fh = rem & 1;
      u32x4 tr[8];
      transpose8x8(pre, tr);
      uint16_t* dst = buf + (blk * 16 + fh * 8) * LDSROW + kb * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) st16(dst + e * LDSROW, tr[e]);
    }
  };
  (void)NT;

  load_stage(0);
  write_stage(0, smem);
  __syncthreads();

  f32x4 sum[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) sum[rt] = zero4();

  for (int s = 0; s < nstages; ++s) {
    const bool more = s + 1 < nstages;
    if (more) load_stage(s + 1);
    const uint16_t* buf = smem + (s & 1) * bufelems;
    int fb, r0, trs;
    stage_geom(s, fb, r0, trs);
    for (int rr = 0; rr < trs; ++rr) {
      f32x4 prod[4];
      for (int j = 0; j < a.p; ++j) {
        f32x4 acc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt] = zero4();
        const uint16_t* brow = buf + ((j * trs + rr) * 16 + c16) * LDSROW;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int k0 = ks * 32 + g * 8;
          u32x4 bv = {0u, 0u, 0u, 0u};
          if (D % 32 == 0 || k0 < D) bv = ld16(brow + k0);
          const bf16x8 b = as_bf16x8(bv);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) acc[rt] = mfma16x16x32(xf[rt][ks], b, acc[rt]);
        }
        if (j == 0) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) prod[rt] = acc[rt];
        } else {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) prod[rt] *= acc[rt];
        }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) sum[rt] += prod[rt];
    }
    if (r0 + trs == a.t) {  // last rank group of this feature block: epilogue
      const int col = fb * 16 + c16;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 v = sum[rt];
        if (a.square) v *= v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (!ook[rt][i]) continue;
          const int64_t off = (obase + orel[rt][i]) * a.m + col;
          if (a.out_bf16)
            static_cast<uint16_t*>(job.phi)[off] = f32_to_bf16(v[i]);
          else
            static_cast<float*>(job.phi)[off] = v[i];
        }
        sum[rt] = zero4();
      }
    }
    if (more) write_stage(s + 1, smem + ((s + 1) & 1) * bufelems);
    __syncthreads();
  }
}

// ---- fp32 SIMT feature map --------------------------------------------------
struct FeatArgsF {
  FeatJob job[2];
  int64_t B, H, n;
  int d, p, t, m;
  int64_t theta_hstride;
  int square;
};

__global__ __launch_bounds__(256) void featmap_f32_kernel(FeatArgsF a) {
  extern __shared__ float xs[];  // [16][d]
  const FeatJob job = a.job[blockIdx.z];
  const int64_t h = blockIdx.y % a.H;
  const int64_t R = a.B * a.n;
  const int fy = threadIdx.x >> 4, fx = threadIdx.x & 15;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 16;
  const float* X = static_cast<const float*>(job.X);
  auto rho_of = [&](int64_t r) -> int64_t {
    const int64_t b = r / a.n;
    return (b * a.H + h) * a.n + (r - b * a.n);
  };
  for (int e = threadIdx.x; e < 16 * a.d; e += 256) {
    const int rr = e / a.d, k = e - rr * a.d;
    const int64_t r = r0 + rr;
    xs[e] = (r < R) ? X[rho_of(r) * a.d + k] : 0.f;
  }
  __syncthreads();
  const float* th = static_cast<const float*>(job.theta) + h * a.theta_hstride;
  const int64_t r = r0 + fy;
  for (int f = fx; f < a.m; f += 16) {
    float acc = 0.f;
    for (int rk = 0; rk < a.t; ++rk) {
      float prod = 1.f;
      for (int j = 0; j < a.p; ++j) {
        const float* col = th + (static_cast<int64_t>(j) * a.t + rk) * a.d * a.m + f;
        float y = 0.f;
        for (int k = 0; k < a.d; ++k) y = fmaf(xs[fy * a.d + k], col[static_cast<int64_t>(k) * a.m], y);
        prod *= y;
      }
      acc += prod;
    }
    if (a.square) acc *= acc;
    if (r < R) static_cast<float*>(job.phi)[rho_of(r) * a.m + f] = acc;
  }
}

// ---- fast bf16 path: (d, p, t) known at compile time, 32x32x16 MFMA ----
//
// Theta is first repacked (pack_theta) into fragment order: for head h,
// 32-feature block fb, rank r, degree index j and 16-deep k-step ks, the
// 64 lanes' fragments of v_mfma_f32_32x32x16_bf16 lie next to each other
// (lane l: feature fb*32 + l%32, k = ks*16 + 8*(l/32) .. +7). One stage
// (fb, r) is then a contiguous P*d*64-byte block that workgroups copy into
// LDS with plain 16-byte loads, and fragment reads from LDS are lane-linear
// (bank-conflict free, no padding).
//
// The MFMAs compute the transposed tile (features x rows): Theta fragments
// are the A operand and the wave's register-resident X rows the B operand.
// A lane then holds one row's features 8i + 4*(l/32) + e (i, e < 4); one
// v_permlane32_swap per register pair gives every lane 16 contiguous bytes
// of phi, so the epilogue stores straight to global memory.
//
// A workgroup of 4 waves owns 256 rows of one head; each wave keeps 2 row
// tiles of 32 rows of X in registers. Stages run one rank at a time through
// a 2-slot LDS ring. In the middle of stage s (after the j = 0 MFMAs) each
// thread moves its share of stage s+1 from registers into the free slot and
// issues the loads of stage s+2, so a whole stage covers the load latency
// and one register set suffices. 32 KiB of LDS (d = 128, p = 2) and <= 256
// VGPRs let two workgroups share a CU, so one workgroup's barrier and VALU
// epilogue overlap the other's MFMAs.
struct FastArgs {
  FeatJob job[2];
  int64_t B, H, n;
  int m;
  int64_t pk_hstride;  // packed elements between heads (0 = shared)
  int square;
  int fsplit;          // feature-block groups per row tile (grid.x = tiles * fsplit)
  int fb_per;          // 32-feature blocks per group
};

constexpr int kFastRT = 2;                         // 32-row tiles per wave
constexpr int kFastNW = 4;                         // waves per workgroup
constexpr int kFastRows = kFastNW * kFastRT * 32;  // rows per workgroup

template <int D, int P>
struct FastGeom {
  static constexpr int KS = D / 16;
  static constexpr int NF = P * KS;                // fragments per stage
  static constexpr int STAGE = NF * 512;           // bf16 elements per stage
  static constexpr int LPT = NF * 64 / (kFastNW * 64);  // 16-byte loads per thread per stage
  static constexpr int FD = NF < 6 ? NF : 6;       // fragment reads in flight
  static constexpr size_t lds_bytes() { return 2ull * STAGE * 2; }
};

// theta [H'][p][t][d][m] -> packed [H'][m/32][t][p][d/16][64 lanes][8];
// blockIdx.y picks one of up to two (theta, packed) pairs
struct PackArgs {
  const uint16_t* th[2];
  uint16_t* pk[2];
};
__global__ __launch_bounds__(256) void pack_theta_kernel(PackArgs pa, int64_t total, int P, int T,
                                                         int D, int m) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const uint16_t* __restrict__ th = pa.th[blockIdx.y];
  uint16_t* __restrict__ pk = pa.pk[blockIdx.y];
  const int KS = D / 16, FB = m / 32;
  const int lane = static_cast<int>(idx & 63);
  int64_t q = idx >> 6;
  const int ks = static_cast<int>(q % KS);
  q /= KS;
  const int j = static_cast<int>(q % P);
  q /= P;
  const int r = static_cast<int>(q % T);
  q /= T;
  const int fb = static_cast<int>(q % FB);
  const int64_t h = q / FB;
  const int k0 = ks * 16 + (lane >> 5) * 8;
  const uint16_t* src = th + (((h * P + j) * T + r) * D + k0) * m + fb * 32 + (lane & 31);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(src[(2 * i) * static_cast<int64_t>(m)]) |
           (static_cast<uint32_t>(src[(2 * i + 1) * static_cast<int64_t>(m)]) << 16);
  st16(pk + idx * 8, u32x4{w[0], w[1], w[2], w[3]});
}

template <int D, int P, int T, bool OUT_BF16>
__global__ __launch_bounds__(kFastNW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void featmap_fast(FastArgs a) {
  using G = FastGeom<D, P>;
  constexpr int RT = kFastRT;
  constexpr int KS = G::KS;
  constexpr int NF = G::NF;
  constexpr int FD = G::FD;
  constexpr int LPT = G::LPT;
  static_assert(D % 32 == 0, "D must be a multiple of 32");
  static_assert((NF * 64) % (kFastNW * 64) == 0, "a stage splits evenly over the threads");
  extern __shared__ __align__(16) uint16_t smem[];

  const FeatJob job = a.job[blockIdx.z];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, c32 = lane & 31;
  const int64_t h = blockIdx.y;
  const int64_t R = a.B * a.n;
  // few rows (decode-sized batches): the feature blocks of a row tile are
  // split over a.fsplit workgroups, fb_per blocks each
  const int tile = blockIdx.x / a.fsplit;
  const int fb0 = (blockIdx.x - tile * a.fsplit) * a.fb_per;
  const int FB = min(a.m / 32, fb0 + a.fb_per) - fb0;  // blocks of this workgroup
  if (FB <= 0) return;
  const int64_t wrow0 = static_cast<int64_t>(tile) * kFastRows + wave * (RT * 32);

  const uint16_t* pk = static_cast<const uint16_t*>(job.theta_pk) + h * a.pk_hstride +
                       static_cast<int64_t>(fb0) * T * G::STAGE;
  const int nstages = FB * T;  // stage s = (fb, r) = (s / T, s % T), fb local
  // piece i of stage s: buffer load at a loop-invariant 32-bit lane offset
  // plus a scalar stage offset (no per-stage address registers, so the
  // compiler never reuses load destinations as address temporaries)
  const uint32_t lane_off = static_cast<uint32_t>(tid) * 16u;
  const __amdgpu_buffer_rsrc_t pk_rsrc =
      make_rsrc(pk, static_cast<uint32_t>(nstages) * G::STAGE * 2u);
  auto load_stage = [&](int s, u32x4 (&v)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      v[i] = buf_ld16(pk_rsrc, lane_off,
                      static_cast<uint32_t>(s) * (G::STAGE * 2u) + i * (kFastNW * 64u * 16u));
  };
  auto write_stage = [&](uint16_t* buf, const u32x4 (&v)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) st16(buf + (i * kFastNW * 64 + tid) * 8, v[i]);
  };

  // stage 0 goes straight to slot 0; stage 1 waits in registers
  u32x4 reg[LPT];
  load_stage(0, reg);
  write_stage(smem, reg);
  load_stage(nstages > 1 ? 1 : 0, reg);

  // ---- X fragments (B operand): lane holds row rt*32 + c32, k = ks*16 + 8*hh .. +7
  const uint16_t* X = static_cast<const uint16_t*>(job.X);
  bf16x8 xf[RT][KS];
  int64_t rowoff[RT];  // element offset of the lane's phi row, -1 past the end
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t r = wrow0 + rt * 32 + c32;
    const bool ok = r < R;
    int64_t rho = 0;
    if (ok) {
      const int64_t b = r / a.n;
      rho = (b * a.H + h) * a.n + (r - b * a.n);
    }
    rowoff[rt] = ok ? rho * a.m : -1;
    const uint16_t* src = X + rho * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      xf[rt][ks] = as_bf16x8(ok ? ld16(src + ks * 16 + hh * 8) : u32x4{0u, 0u, 0u, 0u});
  }
  // drain every load here: a wait for the X fragments left to the compiler
  // lands inside the stage loop and would drain the Theta prefetch each stage
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const uint16_t* fbase = smem + lane * 8;
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  uint8_t* out = static_cast<uint8_t*>(job.phi) + static_cast<int64_t>(fb0) * 32 * ESZ;
  constexpr int NQ = OUT_BF16 ? 2 : 4;  // 16-byte pieces per lane per row tile
  // phi of finished feature blocks, rounded and regrouped so piece q of
  // tile rt is 16 contiguous bytes at byte q*32 + 16*hh of the lane's row.
  // bf16 rows hold two 32-feature blocks per 128-byte line: the blocks are
  // stored in pairs (cv0 = even block, cv1 = odd block) so each line is
  // written whole while it is in L2; stored one at a time, a line's halves
  // lie four stages apart and some lines reach HBM twice.
  constexpr int PAIR = OUT_BF16 ? 2 : 1;
  u32x4 cv0[RT][NQ], cv1[RT][NQ];
  auto finish = [&](const f32x16 (&sum)[RT], u32x4 (&cv)[RT][NQ]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x16 v = sum[rt];
      if (a.square) v *= v;
      if (OUT_BF16) {
        // lane (hh, c32) holds features 8i + 4hh + e of row c32; after the
        // swaps hh = 0 lanes own features 0..7 and 16..23, hh = 1 lanes
        // 8..15 and 24..31 (lanes c32 and c32 + 32 share a row)
        uint32_t w[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w[i][0] = pack_bf16x2(v[4 * i], v[4 * i + 1]);
          w[i][1] = pack_bf16x2(v[4 * i + 2], v[4 * i + 3]);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          swap_halves(w[0][e], w[1][e]);
          swap_halves(w[2][e], w[3][e]);
        }
        cv[rt][0] = u32x4{w[0][0], w[0][1], w[1][0], w[1][1]};
        cv[rt][NQ - 1] = u32x4{w[2][0], w[2][1], w[3][0], w[3][1]};
      } else {
#pragma unroll
        for (int i = 0; i < NQ; ++i)
          cv[rt][i] = u32x4{__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]),
                            __float_as_uint(v[4 * i + 2]), __float_as_uint(v[4 * i + 3])};
      }
    }
  };
  auto emit = [&](int fb, const u32x4 (&cv)[RT][NQ]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      uint8_t* dst = out + (rowoff[rt] + fb * 32) * ESZ + hh * 16;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (rowoff[rt] >= 0) st16(dst + q * 32, cv[rt][q]);
    }
  };

  // One stage: MFMAs of stage s from slot s & 1. After the j = 0 block the
  // registers holding stage s+1 go to the other slot (free since the last
  // barrier), the previous PAIR feature blocks' phi is stored if
  // store_fb >= 0 (blocks store_fb ..), and stage s+2 is requested. The
  // stores go before the loads: waits for loads count in issue order, so a
  // store issued after a load would be waited for together with it half a
  // stage later.
  auto stage = [&](int s, f32x16 (&sum)[RT], int store_fb) {
    const uint16_t* buf = fbase + (s & 1) * G::STAGE;
    bf16x8 fr[NF];
#pragma unroll
    for (int i = 0; i < FD; ++i) fr[i] = as_bf16x8(ld16(buf + i * 512));
    f32x16 prod[RT];
#pragma unroll
    for (int j = 0; j < P; ++j) {
      f32x16 acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int fi = j * KS + ks;
        if (fi + FD < NF) fr[fi + FD] = as_bf16x8(ld16(buf + (fi + FD) * 512));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32x32x16(fr[fi], xf[rt][ks], acc[rt]);
        // pin the read FD fragments ahead of its MFMAs (the scheduler would
        // otherwise sink it next to its use and expose the LDS latency)
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j == 0) {
        __builtin_amdgcn_sched_barrier(0);
        if (s + 1 < nstages) write_stage(smem + ((s + 1) & 1) * G::STAGE, reg);
        if (store_fb >= 0) {
          emit(store_fb, cv0);
          if (PAIR == 2) emit(store_fb + 1, cv1);
        }
        load_stage(s + 2 < nstages ? s + 2 : nstages - 1, reg);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (P == 1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sum[rt] += acc[rt];
      } else if (j == 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) prod[rt] = acc[rt];
      } else if (j + 1 < P) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) prod[rt] *= acc[rt];
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int e = 0; e < 16; ++e) sum[rt][e] = fmaf(prod[rt][e], acc[rt][e], sum[rt][e]);
      }
    }
    __syncthreads();
  };

  // stages stay rolled: unrolling lets the scheduler interleave stages and
  // exceed the register budget
  for (int fb = 0; fb < FB; fb += PAIR) {
    {
      f32x16 sum[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sum[rt] = zero16();
#pragma unroll 1
      for (int r = 0; r < T; ++r) stage(fb * T + r, sum, r == 0 && fb >= PAIR ? fb - PAIR : -1);
      finish(sum, cv0);
    }
    if (PAIR == 2 && fb + 1 < FB) {
      f32x16 sum[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sum[rt] = zero16();
#pragma unroll 1
      for (int r = 0; r < T; ++r) stage((fb + 1) * T + r, sum, -1);
      finish(sum, cv1);
    }
  }
  // the last block or pair
  const int last = (FB - 1) / PAIR * PAIR;
  emit(last, cv0);
  if (PAIR == 2 && last + 1 < FB) emit(last + 1, cv1);
}

// ---- few rows per head (decode-sized batches): Theta in its natural layout ----
//
// With a few hundred rows per head the projection is bound by reading Theta
// once. A workgroup owns one 32-feature block of one head and every row: it
// stages Theta_{j,r}[:, block] for all (j, r) side by side in LDS rows of d
// (natural layout, 16-byte loads) and 32 rows of X per wave, and reads both
// operands in natural k-order (the Theta side with the transposing LDS read), so
// Theta needs no fragment-order copy and no repacking launch.
constexpr int kSmallRows = 1024;  // rows per head up to which this path runs

struct SmallArgs {
  FeatJob job[2];
  int64_t B, H, n;
  int m;
  int64_t th_hstride;  // Theta elements between heads (0 = shared)
  int square;
};

template <int D, int P, int T>
struct SmallGeom {
  static constexpr int PT = P * T;
  static constexpr int TW = PT * 32 + 32;  // Theta row stride (elements): rows 64 bytes apart mod 256
  static constexpr size_t lds_bytes() { return 1ull * D * TW * 2; }
};

// Row r of a head's flattened (batch, position) rows -> its row of the
// [B][H][n] tensor, for r < 2^32 (a 32-bit division: the 64-bit one expands
// to a long instruction sequence per call).
__device__ __forceinline__ int64_t head_row(uint32_t r, uint32_t n, int64_t H, int64_t h) {
  const uint32_t b = r / n;
  return (static_cast<int64_t>(b) * H + h) * n + (r - b * n);
}

template <int D, int P, int T, bool OUT_BF16>
__global__ __launch_bounds__(256) void featmap_small(SmallArgs a) {
  using G = SmallGeom<D, P, T>;
  constexpr int PT = G::PT, TW = G::TW, KS = D / 16, NF = P * KS;
  static_assert(PT % 2 == 0, "Theta rows need an even block count to stay conflict free");
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* Ts = smem;           // [D][TW]: Theta_{j,r}[k][block] at column (j*T + r) * 32
  // XCD-aware work order: the workgroups of one (head, job) pair -- one per
  // 32-feature block -- go to one XCD (workgroups reach the 8 XCDs round
  // robin, id % 8), so the 128-byte Theta rows the neighbouring blocks each
  // read half of, and the pair's X rows, are fetched once into that XCD's L2
  // (32-bit index arithmetic: the grid has m/32 * H * jobs < 2^31 workgroups)
  const uint32_t FB = static_cast<uint32_t>(a.m / 32);
  const uint32_t pairs = gridDim.x / FB;
  const uint32_t id = blockIdx.x;
  uint32_t pair, fb;
  if (pairs % 8 == 0) {
    const uint32_t k = id / 8;
    pair = (id % 8) * (pairs / 8) + k / FB;
    fb = k % FB;
  } else {
    pair = id / FB;
    fb = id % FB;
  }
  const uint32_t H32 = static_cast<uint32_t>(a.H);
  const FeatJob job = a.job[pair / H32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, c32 = lane & 31;
  const int64_t h = pair % H32;
  const int64_t R = a.B * a.n;

  const uint16_t* th = static_cast<const uint16_t*>(job.theta) + h * a.th_hstride;
  const uint16_t* X = static_cast<const uint16_t*>(job.X);
  const uint32_t nr = static_cast<uint32_t>(a.n);  // R <= kSmallRows: rows fit 32 bits
  // X fragments of 32 rows, straight from global memory in natural k-order:
  // lane row t0 + c32, k = 16ks + 8hh + 0..7, one 16-byte load per k-step
  // (rows clamped to R - 1 >= 0; zeroed past the end when taken). These
  // loads are requests-bound (every instruction touches 32 rows), so the
  // wave's first tile is issued ahead of Theta's loads and overlaps them.
  auto issue_x = [&](int64_t t0, u32x4 (&xr)[KS]) {
    const int64_t r = t0 + c32 < R ? t0 + c32 : R - 1;
    const uint16_t* src = X + head_row(static_cast<uint32_t>(r), nr, a.H, h) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) xr[ks] = ld16(src + ks * 16);
  };
  auto take_x = [&](int64_t t0, const u32x4 (&xr)[KS], bf16x8 (&xf)[KS]) {
    const bool ok = t0 + c32 < R;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) xf[ks] = as_bf16x8(ok ? xr[ks] : u32x4{0u, 0u, 0u, 0u});
  };
  const int64_t tw = static_cast<int64_t>(w) * 32;  // the wave's first row tile
  u32x4 xr[KS];
  issue_x(tw, xr);
  // all of a thread's Theta loads are issued before its first LDS store
  constexpr int TL = PT * D * 4 / 256;  // 16-byte pieces per thread
  static_assert((PT * D * 4) % 256 == 0, "Theta block splits evenly over the threads");
  {
    u32x4 tv[TL];
#pragma unroll
    for (int i = 0; i < TL; ++i) {
      const int idx = tid + 256 * i, q = idx & 3, k = (idx >> 2) % D, jr = (idx >> 2) / D;
      tv[i] = ld16(th + (static_cast<int64_t>(jr) * D + k) * a.m + fb * 32 + q * 8);
    }
#pragma unroll
    for (int i = 0; i < TL; ++i) {
      const int idx = tid + 256 * i, q = idx & 3, k = (idx >> 2) % D, jr = (idx >> 2) / D;
      st16(Ts + k * TW + jr * 32 + q * 8, tv[i]);
    }
  }
  __syncthreads();

  uint8_t* out = static_cast<uint8_t*>(job.phi);
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  for (int64_t t0 = tw; t0 < R; t0 += 4 * 32) {
    if (t0 != tw) issue_x(t0, xr);
    bf16x8 xf[KS];
    take_x(t0, xr, xf);
    f32x16 sum = zero16();
#pragma unroll 1
    for (int r = 0; r < T; ++r) {
      // Theta fragments of rank r (natural k-order, as X's), (j, ks)
      // flattened, read two ahead (pinned)
      bf16x8 fr[3];
      fr[0] = frag_tr_nat(Ts, TW, 0, r * 32, lane);
      if (NF > 1) fr[1] = frag_tr_nat(Ts, TW, (1 % KS) * 16, ((1 / KS) * T + r) * 32, lane);
      f32x16 prod, acc;
#pragma unroll
      for (int fi = 0; fi < NF; ++fi) {
        const int j = fi / KS, ks = fi % KS;
        if (fi + 2 < NF)
          fr[(fi + 2) % 3] = frag_tr_nat(Ts, TW, ((fi + 2) % KS) * 16, (((fi + 2) / KS) * T + r) * 32, lane);
        acc = mfma32x32x16(xf[ks], fr[fi % 3], ks == 0 ? zero16() : acc);
        __builtin_amdgcn_sched_barrier(0);
        if (ks == KS - 1) prod = j == 0 ? acc : prod * acc;
      }
      sum += prod;
    }
    if (a.square) sum *= sum;
    // element 4i+e: row t0 + 8i + 4hh + e, feature fb*32 + c32
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = t0 + 8 * i + 4 * hh + e;
        if (r < R) {
          uint8_t* dst = out + (head_row(static_cast<uint32_t>(r), nr, a.H, h) * a.m + fb * 32 + c32) * ESZ;
          if (OUT_BF16)
            *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16(sum[4 * i + e]);
          else
            *reinterpret_cast<float*>(dst) = sum[4 * i + e];
        }
      }
  }
}

template <int D, int P, int T, bool OUT_BF16>
hipError_t launch_small_t(const FeatShape& s, const FeatJob* jobs, int njobs, hipStream_t st) {
  using G = SmallGeom<D, P, T>;
  SmallArgs a{};
  a.job[0] = jobs[0];
  a.job[1] = njobs > 1 ? jobs[1] : jobs[0];
  a.B = s.B;
  a.H = s.H;
  a.n = s.n;
  a.m = s.m;
  a.th_hstride = s.theta_per_head ? static_cast<int64_t>(P) * T * D * s.m : 0;
  a.square = s.square;
  if (s.H > 65535) return hipErrorInvalidValue;
  if (s.B * s.n == 0) return hipSuccess;  // no rows (the kernel reads row R - 1 of a head)
  auto* k = featmap_small<D, P, T, OUT_BF16>;
  const hipError_t e = allow_lds(k, G::lds_bytes());
  if (e != hipSuccess) return e;
  // one workgroup per (32-feature block, head, job), ordered in the kernel
  dim3 grid(static_cast<unsigned>(static_cast<int64_t>(s.m / 32) * s.H * njobs));
  LLOPS_LAUNCH("featmap_bf16", st, k, grid, dim3(256), G::lds_bytes(), st, a);
  return hipGetLastError();
}

template <int D, int P, int T>
hipError_t launch_small(const FeatShape& s, const FeatJob* jobs, int njobs, hipStream_t st) {
  return s.out_bf16 ? launch_small_t<D, P, T, true>(s, jobs, njobs, st)
                    : launch_small_t<D, P, T, false>(s, jobs, njobs, st);
}

template <int D, int P, int T, bool OUT_BF16>
hipError_t launch_fast_t(const FeatShape& s, const FeatJob* jobs, int njobs, hipStream_t st) {
  using G = FastGeom<D, P>;
  FastArgs a{};
  a.job[0] = jobs[0];
  a.job[1] = njobs > 1 ? jobs[1] : jobs[0];
  a.B = s.B;
  a.H = s.H;
  a.n = s.n;
  a.m = s.m;
  a.pk_hstride = s.theta_per_head ? static_cast<int64_t>(P) * T * D * s.m : 0;
  a.square = s.square;
  const int64_t tiles = (s.B * s.n + kFastRows - 1) / kFastRows;
  // under ~1024 workgroups, split the feature blocks to fill the chip
  const int FB = s.m / 32;
  int fsplit = 1;
  const int64_t wgs = tiles * s.H * njobs;
  if (wgs > 0 && wgs < 1024) {
    const int64_t want = (1024 + wgs - 1) / wgs;
    fsplit = static_cast<int>(want < FB ? want : FB);
  }
  a.fb_per = (FB + fsplit - 1) / fsplit;
  a.fsplit = (FB + a.fb_per - 1) / a.fb_per;
  if (tiles * a.fsplit > 0x7fffffffLL || s.H > 65535) return hipErrorInvalidValue;
  // repack Theta of every job into its fragment-order buffer
  const int64_t th_heads = s.theta_per_head ? s.H : 1;
  const int64_t total = th_heads * P * T * D * s.m / 8;
  // one launch for both jobs (the second is skipped when it repeats the first)
  PackArgs pa{};
  int npack = 0;
  for (int jb = 0; jb < njobs; ++jb) {
    if (jb == 1 && jobs[1].theta == jobs[0].theta && jobs[1].theta_pk == jobs[0].theta_pk) break;
    pa.th[npack] = static_cast<const uint16_t*>(jobs[jb].theta);
    pa.pk[npack] = static_cast<uint16_t*>(jobs[jb].theta_pk);
    ++npack;
  }
  LLOPS_LAUNCH("pack_theta", st, pack_theta_kernel,
               dim3(static_cast<unsigned>((total + 255) / 256), static_cast<unsigned>(npack)), dim3(256), 0,
               st, pa, total, P, T, D, s.m);
  const size_t lds = G::lds_bytes();
  auto* k = featmap_fast<D, P, T, OUT_BF16>;
  const hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>(tiles * a.fsplit), static_cast<unsigned>(s.H), njobs);
  LLOPS_LAUNCH("featmap_bf16", st, k, grid, dim3(kFastNW * 64), lds, st, a);
  return hipGetLastError();
}

template <int D, int P, int T>
hipError_t launch_fast(const FeatShape& s, const FeatJob* jobs, int njobs, hipStream_t st) {
  return s.out_bf16 ? launch_fast_t<D, P, T, true>(s, jobs, njobs, st)
                    : launch_fast_t<D, P, T, false>(s, jobs, njobs, st);
}

int fast_key(const FeatShape& s) {
  if (s.B * s.n < 1 || s.m % 32 != 0) return 0;
  const int key = s.d * 10000 + s.p * 100 + s.t;
  switch (key) {
    case 1280204:
    case 1280201:
    case 1280401:
    case 640204:
    case 640201:
    case 640401:
    case 640308: return key;
    default: return 0;
  }
}

bool small_rows(const FeatShape& s) { return s.B * s.n <= kSmallRows; }

bool try_fast(const FeatShape& s, const FeatJob* jobs, int njobs, hipStream_t st, hipError_t* err) {
  if (small_rows(s)) {
    switch (fast_key(s)) {
      case 1280204: *err = launch_small<128, 2, 4>(s, jobs, njobs, st); return true;
      case 1280201: *err = launch_small<128, 2, 1>(s, jobs, njobs, st); return true;
      case 1280401: *err = launch_small<128, 4, 1>(s, jobs, njobs, st); return true;
      case 640204: *err = launch_small<64, 2, 4>(s, jobs, njobs, st); return true;
      case 640201: *err = launch_small<64, 2, 1>(s, jobs, njobs, st); return true;
      case 640401: *err = launch_small<64, 4, 1>(s, jobs, njobs, st); return true;
      case 640308: *err = launch_small<64, 3, 8>(s, jobs, njobs, st); return true;
      default: return false;
    }
  }
  // callers without scratch for the repacked Theta take the generic kernel
  for (int jb = 0; jb < njobs; ++jb)
    if (!jobs[jb].theta_pk) return false;
  switch (fast_key(s)) {
    case 1280204: *err = launch_fast<128, 2, 4>(s, jobs, njobs, st); return true;
    case 1280201: *err = launch_fast<128, 2, 1>(s, jobs, njobs, st); return true;
    case 1280401: *err = launch_fast<128, 4, 1>(s, jobs, njobs, st); return true;
    case 640201: *err = launch_fast<64, 2, 1>(s, jobs, njobs, st); return true;
    case 640401: *err = launch_fast<64, 4, 1>(s, jobs, njobs, st); return true;
    case 640204: *err = launch_fast<64, 2, 4>(s, jobs, njobs, st); return true;
    case 640308: *err = launch_fast<64, 3, 8>(s, jobs, njobs, st); return true;
    default: return false;
  }
}

}  // namespace

hipError_t launch_pack_theta(const FeatShape& s, const void* theta, void* pk, hipStream_t st) {
  if (!fast_key(s) || small_rows(s) || !theta || !pk) return hipErrorInvalidValue;
  const int64_t th_heads = s.theta_per_head ? s.H : 1;
  const int64_t total = th_heads * s.p * s.t * s.d * s.m / 8;
  PackArgs pa{};
  pa.th[0] = static_cast<const uint16_t*>(theta);
  pa.pk[0] = static_cast<uint16_t*>(pk);
  LLOPS_LAUNCH("pack_theta", st, pack_theta_kernel,
               dim3(static_cast<unsigned>((total + 255) / 256), 1u), dim3(256), 0, st, pa, total,
               s.p, s.t, s.d, s.m);
  return hipGetLastError();
}

size_t featmap_pack_bytes(const FeatShape& s) {
  if (!fast_key(s) || small_rows(s)) return 0;
  const int64_t th_heads = s.theta_per_head ? s.H : 1;
  return static_cast<size_t>(th_heads) * s.p * s.t * s.d * s.m * sizeof(uint16_t);
}

namespace {

template <int D>
hipError_t launch_d(const FeatArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  const hipError_t e = allow_lds(featmap_mfma<D, 4>, lds);
  if (e != hipSuccess) return e;
  LLOPS_LAUNCH("featmap_bf16", st, (featmap_mfma<D, 4>), grid, dim3(256), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_featmap_bf16(const FeatShape& s, const FeatJob* jobs, int njobs,
                               hipStream_t st) {
  hipError_t fast_err = hipSuccess;
  if (try_fast(s, jobs, njobs, st, &fast_err)) return fast_err;
  FeatArgs a{};
  a.job[0] = jobs[0];
  a.job[1] = njobs > 1 ? jobs[1] : jobs[0];
  a.B = s.B;
  a.H = s.H;
  a.n = s.n;
  a.p = s.p;
  a.t = s.t;
  a.m = s.m;
  a.theta_hstride = s.theta_per_head ? static_cast<int64_t>(s.p) * s.t * s.d * s.m : 0;
  a.square = s.square;
  a.out_bf16 = s.out_bf16;
  // ranks per stage: one 8x8 sub-block per thread, LDS ring <= 72 KiB
  const int ldsrow = s.d + 8;
  int tr = 1024 / (s.p * s.d);
  const int tr_lds = (36 * 1024) / (s.p * 16 * ldsrow * 2);
  tr = tr < tr_lds ? tr : tr_lds;
  tr = tr < s.t ? tr : s.t;
  if (tr < 1) return hipErrorInvalidValue;
  a.tr = tr;
  const int64_t R = s.B * s.n;
  const int64_t tiles = (R + 255) / 256;
  const int FB = s.m / 16;
  // few row tiles (decode-sized batches): split the feature blocks across workgroups
  int fsplit = 1;
  const int64_t wgs = tiles * s.H * njobs;
  if (wgs < 1024) {
    int64_t want = (1024 + wgs - 1) / wgs;
    fsplit = static_cast<int>(want < FB ? want : FB);
  }
  a.fb_per_split = (FB + fsplit - 1) / fsplit;
  a.fsplit = (FB + a.fb_per_split - 1) / a.fb_per_split;
  if (tiles * a.fsplit > 0x7fffffffLL || s.H > 65535) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(tiles * a.fsplit), static_cast<unsigned>(s.H), njobs);
  const size_t lds = 2ull * s.p * tr * 16 * ldsrow * sizeof(uint16_t);
  // every d the validation admits for bf16 (a multiple of 16 up to 256); the
  // kernel zeroes both operands past d when d is not a multiple of 32
  switch (s.d) {
    case 16: return launch_d<16>(a, grid, lds, st);
    case 32: return launch_d<32>(a, grid, lds, st);
    case 48: return launch_d<48>(a, grid, lds, st);
    case 64: return launch_d<64>(a, grid, lds, st);
    case 80: return launch_d<80>(a, grid, lds, st);
    case 96: return launch_d<96>(a, grid, lds, st);
    case 112: return launch_d<112>(a, grid, lds, st);
    case 128: return launch_d<128>(a, grid, lds, st);
    case 144: return launch_d<144>(a, grid, lds, st);
    case 160: return launch_d<160>(a, grid, lds, st);
    case 176: return launch_d<176>(a, grid, lds, st);
    case 192: return launch_d<192>(a, grid, lds, st);
    case 208: return launch_d<208>(a, grid, lds, st);
    case 224: return launch_d<224>(a, grid, lds, st);
    case 240: return launch_d<240>(a, grid, lds, st);
    case 256: return launch_d<256>(a, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_featmap_f32(const FeatShape& s, const FeatJob* jobs, int njobs,
                              hipStream_t st) {
  FeatArgsF a{};
  a.job[0] = jobs[0];
  a.job[1] = njobs > 1 ? jobs[1] : jobs[0];
  a.B = s.B;
  a.H = s.H;
  a.n = s.n;
  a.d = s.d;
  a.p = s.p;
  a.t = s.t;
  a.m = s.m;
  a.theta_hstride = s.theta_per_head ? static_cast<int64_t>(s.p) * s.t * s.d * s.m : 0;
  a.square = s.square;
  const int64_t R = s.B * s.n;
  const int64_t tiles = (R + 15) / 16;
  if (tiles > 0x7fffffffLL || s.H > 65535) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(s.H), njobs);
  LLOPS_LAUNCH("featmap_f32", st, featmap_f32_kernel, grid, dim3(256), 16 * s.d * sizeof(float), st, a);
  return hipGetLastError();
}

}  // namespace llops
