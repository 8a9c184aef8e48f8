// LLoPS feature map  phi(X) = sum_r prod_j X Theta_{j,r}  [squared after the r-sum]
// (papernotes.org LLoPS notes, key design 2; arXiv 2610.14219 Sec. 3).
//
// bf16 path: each workgroup owns 256 rows (4 waves x 64) of one head. A wave
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
  const int lane = tid & 63, wave = tid >> 6;
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
  switch (s.d) {
    case 16: return launch_d<16>(a, grid, lds, st);
    case 32: return launch_d<32>(a, grid, lds, st);
    case 48: return launch_d<48>(a, grid, lds, st);
    case 64: return launch_d<64>(a, grid, lds, st);
    case 96: return launch_d<96>(a, grid, lds, st);
    case 128: return launch_d<128>(a, grid, lds, st);
    case 192: return launch_d<192>(a, grid, lds, st);
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
