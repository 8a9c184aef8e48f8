// LLoPS feature-map backward. For an upstream gradient dphi, the gradients of
// L = sum(dphi * phi) with respect to X and Theta, by the chain rule through
// phi = [sum_r prod_j X Theta_{j,r}]^(2 if square) (LLoPS notes, key design 2;
// Theta is trained end to end, notes' training strategy):
//   Y_{j,r} = X Theta_{j,r},   s = sum_r prod_j Y_{j,r},   ds = dphi * 2s (square) or dphi
//   dY_{j,r} = ds * prod_{j' != j} Y_{j',r}
//   dX = sum_{j,r} dY_{j,r} Theta_{j,r}^T,   dTheta_{j,r} = X^T dY_{j,r}
//
// Both kernels stage one 32-feature block of every Theta_{j,r} side by side
// in LDS rows of d, in Theta's natural layout, and recompute Y on 32x32x16
// MFMA from it: nothing of size n x p*t*m is stored. Operands are read in P16
// k-order (device.h), so recomputed tiles feed the next product from
// registers.
//
// dX (featmap_bwd_dx): a workgroup owns 128 rows (32 per wave) of one head and
// keeps their dX tile (rows x d) in registers. Per feature block it
// recomputes s in the transposed orientation (features x rows), forms ds,
// recomputes each rank's Y, and adds dY_{j,r} Theta_{j,r}^T: dY as the A
// operand straight from its accumulator, Theta^T read from the staged rows.
//
// dTheta (featmap_bwd_dth): a workgroup owns one feature block, one head and
// one chunk of rows, and walks the chunk 32 rows at a time with the rows
// staged in LDS. Y is recomputed in the natural orientation (rows x
// features), so dY^T is an A operand from registers and X (read transposed
// from LDS) the B operand. With t = 4 each wave takes one rank and the waves
// swap their rank's product through LDS to form s; with t = 1 every wave
// computes the one rank and takes a quarter of the d columns. The workgroup
// writes its chunk's partial dTheta; featmap_bwd_reduce sums the chunks (and
// the heads, for a shared Theta) in a fixed order and transposes.
#include "device.h"
#include "kernels.h"

namespace llops {
namespace {

struct BwdArgs {
  const uint16_t* X;      // [B][H][n][d] bf16
  const uint16_t* theta;  // [H'][p][t][d][m] bf16
  const void* dphi;       // [B][H][n][m], fp32 or bf16
  float* dX;              // [B][H][n][d]
  float* part;            // dTheta partials [chunk][H][p][t][m][d]
  int64_t B, H, n;
  int m;
  int64_t th_hstride;     // Theta elements between heads (0 = shared)
  int square;
  int chunks;             // row chunks per head (dTheta kernel)
  int64_t chunk_rows;     // rows per chunk, a multiple of the kernel's step
};

template <int D, int P, int T>
struct BwdGeom {
  static constexpr int PT = P * T;
  static constexpr int KS = D / 16;        // 16-deep k-steps over d
  static constexpr int DT = D / 32;        // 32-wide tiles of d
  static constexpr int TW = PT * 32 + 16;  // staged Theta row stride: rows shift by 8 banks
  static constexpr int XW = D + 16;        // staged X row stride: rows shift by 8 banks
  static constexpr int RB = T == 4 ? 32 : 128;  // rows per step of the dTheta kernel
  static constexpr size_t theta_lds() { return 1ull * D * TW * 2; }
  static constexpr size_t x_lds() { return 1ull * RB * XW * 2; }
  static constexpr size_t exch_lds() { return T == 4 ? 4ull * 16 * 64 * 4 : 0; }
  static_assert(PT % 2 == 0, "staged Theta rows need an even block count to stay conflict free");
  static_assert((PT * D * 4) % 256 == 0, "a Theta block splits evenly over the threads");
};

// Theta_{j,r}[k][fb*32 + c] -> Ts[k][(j*T + r)*32 + c]; all loads of a thread
// are issued before its first LDS store.
template <int D, int PT>
__device__ __forceinline__ void stage_theta(uint16_t* Ts, int TW, const uint16_t* th, int m,
                                            int fb, int tid) {
  constexpr int TL = PT * D * 4 / 256;
  u32x4 tv[TL];
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    const int idx = tid + 256 * i, q = idx & 3, k = (idx >> 2) % D, jr = (idx >> 2) / D;
    tv[i] = ld16(th + (static_cast<int64_t>(jr) * D + k) * m + fb * 32 + q * 8);
  }
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    const int idx = tid + 256 * i, q = idx & 3, k = (idx >> 2) % D, jr = (idx >> 2) / D;
    st16(Ts + k * TW + jr * 32 + q * 8, tv[i]);
  }
}

// Sequence row of head h for row r of the head's [B*n] rows.
__device__ __forceinline__ int64_t rho_of(int64_t r, int64_t h, const BwdArgs& a) {
  const int64_t b = r / a.n;
  return (b * a.H + h) * a.n + (r - b * a.n);
}

// ---------------------------------------------------------------------------
// dX
// ---------------------------------------------------------------------------
// GB: dphi is bf16 (else fp32).
template <int D, int P, int T, bool GB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void featmap_bwd_dx(BwdArgs a) {
  using G = BwdGeom<D, P, T>;
  constexpr int KS = G::KS, DT = G::DT, TW = G::TW, PT = G::PT;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* Ts = smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, c32 = lane & 31;
  const int64_t h = blockIdx.y;
  const int64_t R = a.B * a.n;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 128 + w * 32;  // this wave's rows

  // X fragments (B operand of the transposed recompute): lane row t0 + c32,
  // k = 16ks + {4hh..4hh+3, 8+4hh..8+4hh+3}; zeros past the end
  bf16x8 xf[KS];
  const bool ok = t0 + c32 < R;
  const int64_t rho = rho_of(ok ? t0 + c32 : R - 1, h, a);
  {
    const uint16_t* src = a.X + rho * D + 4 * hh;
    u32x2 lo[KS], hi[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      lo[ks] = *reinterpret_cast<const u32x2*>(src + ks * 16);
      hi[ks] = *reinterpret_cast<const u32x2*>(src + ks * 16 + 8);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      xf[ks] = as_bf16x8(ok ? u32x4{lo[ks][0], lo[ks][1], hi[ks][0], hi[ks][1]}
                            : u32x4{0u, 0u, 0u, 0u});
  }
  const uint16_t* th = a.theta + h * a.th_hstride;

  // Y_{j,r} of the staged feature block, transposed: element 4i+e is
  // feature 8i + 4hh + e of row t0 + c32
  auto y_of = [&](int j, int r) {
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = mfma32x32x16(frag_tr(Ts, TW, ks * 16, (j * T + r) * 32, lane), xf[ks], acc);
    return acc;
  };

  f32x16 dx[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dx[dt] = zero16();
  const int FB = a.m / 32;
  for (int fb = 0; fb < FB; ++fb) {
    // upstream gradient of this lane's row, features fb*32 + 8i + 4hh + {0..3}
    f32x16 g;
    {
      const int64_t base = rho * a.m + fb * 32 + 4 * hh;
      if constexpr (GB) {
        u32x2 gv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          gv[i] = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.dphi) + base + 8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            g[4 * i + e] = __uint_as_float(e & 1 ? gv[i][e >> 1] & 0xffff0000u : gv[i][e >> 1] << 16);
      } else {
        f32x4 gv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          gv[i] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.dphi) + base + 8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) g[4 * i + e] = gv[i][e];
      }
    }
    __syncthreads();  // every wave is done with the previous block's Theta
    stage_theta<D, PT>(Ts, TW, th, a.m, fb, tid);
    __syncthreads();
    f32x16 ds = g;
    if (a.square) {
      f32x16 s = zero16();
#pragma unroll 1
      for (int r = 0; r < T; ++r) {
        f32x16 prod = y_of(0, r);
#pragma unroll
        for (int j = 1; j < P; ++j) prod *= y_of(j, r);
        s += prod;
      }
      ds *= 2.f * s;
    }
    if (!ok) ds = zero16();
#pragma unroll 1
    for (int r = 0; r < T; ++r) {
      f32x16 y[P];
#pragma unroll
      for (int j = 0; j < P; ++j) y[j] = y_of(j, r);
#pragma unroll
      for (int j = 0; j < P; ++j) {
        f32x16 dy = ds;
#pragma unroll
        for (int jj = 0; jj < P; ++jj)
          if (jj != j) dy *= y[jj];
        // dX[rows][d] += dY[rows][f] Theta^T[f][d]: dY as the A operand (lane
        // row, k = features in P16 order), Theta^T from the staged rows of d
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const bf16x8 af = acc_frag(dy, hf);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            dx[dt] = mfma32x32x16(af, frag_p16(Ts, TW, dt * 32, (j * T + r) * 32 + hf * 16, lane),
                                  dx[dt]);
        }
      }
    }
  }
  // dx[dt] element 4i+e: row t0 + 8i + 4hh + e, column dt*32 + c32
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t r = t0 + 8 * i + 4 * hh + e;
      if (r < R) {
        float* dst = a.dX + rho_of(r, h, a) * D + c32;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) dst[dt * 32] = dx[dt][4 * i + e];
      }
    }
}

// ---------------------------------------------------------------------------
// dTheta partials
// ---------------------------------------------------------------------------
template <int D, int P, int T, bool GB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void featmap_bwd_dth(BwdArgs a) {
  using G = BwdGeom<D, P, T>;
  constexpr int KS = G::KS, DT = G::DT, TW = G::TW, XW = G::XW, PT = G::PT;
  static_assert(T == 1 || T == 4, "one rank per wave (t = 4) or one rank for all (t = 1)");
  constexpr int RB = G::RB;                 // rows per step
  constexpr int XL = RB * (D / 8) / 256;    // 16-byte pieces of a step's X per thread
  static_assert(XL >= 1 && RB * (D / 8) % 256 == 0, "a step's rows split evenly over the threads");
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* Ts = smem;
  uint16_t* Xs = smem + D * TW;
  float* exch = reinterpret_cast<float*>(Xs + RB * XW);  // [wave][4][64][4] (t = 4)
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, c32 = lane & 31;
  // Workgroups go to the 8 XCDs in turn; renumber them so that the m/32
  // feature blocks of one (chunk, head), which read the same rows of X, run
  // on one XCD and share its L2.
  const int FB = a.m / 32;
  const int64_t N = static_cast<int64_t>(gridDim.x);
  int64_t L = blockIdx.x;
  if (N % 8 == 0) L = (L % 8) * (N / 8) + L / 8;
  const int fb = static_cast<int>(L % FB);
  const int chunk = static_cast<int>((L / FB) % a.chunks);
  const int64_t h = L / (static_cast<int64_t>(FB) * a.chunks);
  const int64_t R = a.B * a.n;
  const int64_t r0 = chunk * a.chunk_rows;
  const int64_t r1 = min(R, r0 + a.chunk_rows);
  const int rk = T == 4 ? w : 0;       // the rank this wave recomputes
  const int wr = T == 4 ? 0 : 32 * w;  // this wave's first row within a step

  stage_theta<D, PT>(Ts, TW, a.theta + h * a.th_hstride, a.m, fb, tid);

  f32x16 acc[P][DT];
#pragma unroll
  for (int j = 0; j < P; ++j)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[j][dt] = zero16();

  // X of one step, row-major; rows past the chunk read its last row
  u32x4 xv[XL];
  auto load_x = [&](int64_t t0) {
#pragma unroll
    for (int it = 0; it < XL; ++it) {
      const int idx = tid + 256 * it, rr = idx / (D / 8), q = idx % (D / 8);
      const int64_t r = t0 + rr < r1 ? t0 + rr : r1 - 1;
      xv[it] = ld16(a.X + rho_of(r, h, a) * D + q * 8);
    }
  };
  load_x(r0);
  for (int64_t t0 = r0; t0 < r1; t0 += RB) {
    __syncthreads();  // the previous step's X and exchange reads are done
#pragma unroll
    for (int it = 0; it < XL; ++it) {
      const int idx = tid + 256 * it, rr = idx / (D / 8), q = idx % (D / 8);
      st16(Xs + rr * XW + q * 8, t0 + rr < r1 ? xv[it] : u32x4{0u, 0u, 0u, 0u});
    }
    __syncthreads();
    // upstream gradient: element 4i+e is row t0 + wr + 8i + 4hh + e, feature fb*32 + c32
    f32x16 g;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = t0 + wr + 8 * i + 4 * hh + e;
        const int64_t idx = rho_of(r < r1 ? r : r1 - 1, h, a) * a.m + fb * 32 + c32;
        g[4 * i + e] = GB ? bf16_to_f32(static_cast<const uint16_t*>(a.dphi)[idx])
                          : static_cast<const float*>(a.dphi)[idx];
      }
    load_x(t0 + RB < r1 ? t0 + RB : t0);  // next step's rows, in flight during this one
    // Y_{j,rk} in the natural orientation: element 4i+e is row wr + 8i + 4hh + e
    // of the step, lane column c32 is feature fb*32 + c32
    f32x16 y[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
      y[j] = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        y[j] = mfma32x32x16(frag_p16(Xs, XW, wr, ks * 16, lane),
                            frag_tr(Ts, TW, ks * 16, (j * T + rk) * 32, lane), y[j]);
    }
    f32x16 ds = g;
    if (a.square) {
      f32x16 s = y[0];
#pragma unroll
      for (int j = 1; j < P; ++j) s *= y[j];
      if constexpr (T == 4) {  // s = sum of the four waves' rank products
#pragma unroll
        for (int q = 0; q < 4; ++q)
          st16(exch + ((w * 4 + q) * 64 + lane) * 4,
               u32x4{__float_as_uint(s[4 * q]), __float_as_uint(s[4 * q + 1]),
                     __float_as_uint(s[4 * q + 2]), __float_as_uint(s[4 * q + 3])});
        __syncthreads();
        s = zero16();
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 u = ld16(exch + ((v * 4 + q) * 64 + lane) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[4 * q + e] += __uint_as_float(u[e]);
          }
      }
      ds *= 2.f * s;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t0 + wr + 8 * i + 4 * hh + e >= r1) ds[4 * i + e] = 0.f;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      f32x16 dy = ds;
#pragma unroll
      for (int jj = 0; jj < P; ++jj)
        if (jj != j) dy *= y[jj];
      // dTheta^T[f][d] += dY^T[f][rows] X[rows][d]: dY^T as the A operand
      // (lane feature, k = rows in P16 order), X read transposed from LDS
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8 af = acc_frag(dy, hf);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[j][dt] = mfma32x32x16(af, frag_tr(Xs, XW, wr + hf * 16, dt * 32, lane), acc[j][dt]);
      }
    }
  }
  // partial dTheta^T tile: element 4i+e is feature fb*32 + 8i + 4hh + e, lane
  // column c32 is d = dt*32 + c32; layout [slot][H][p][t][m][d], one slot per
  // chunk (t = 4) or per chunk and wave (t = 1)
  const int64_t slot = T == 4 ? chunk : static_cast<int64_t>(chunk) * 4 + w;
#pragma unroll
  for (int j = 0; j < P; ++j)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float* dst = a.part + (((((slot * a.H + h) * P + j) * T + rk) * a.m) + fb * 32) * D +
                   dt * 32 + c32;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(8 * i + 4 * hh + e) * D] = acc[j][dt][4 * i + e];
    }
}

// dtheta[h'][j][r][d][f] = sum over slots (and heads, for a shared Theta) of
// part[slot][h][j][r][f][d], summed in a fixed order; 32 x 32 tiles are
// transposed through LDS so reads and writes are both row contiguous. With
// no slots (no rows) it writes zeros.
__global__ __launch_bounds__(256) void featmap_bwd_reduce(const float* __restrict__ part,
                                                          float* __restrict__ dtheta, int slots,
                                                          int64_t H, int heads_per_out, int PT,
                                                          int D, int m) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const int ftiles = m / 32;
  const int ftile = static_cast<int>(blockIdx.x % ftiles), dtile = blockIdx.y;
  const int64_t hjr = blockIdx.x / ftiles;  // (h', jr)
  const int64_t ho = hjr / PT, jr = hjr % PT;
  const int64_t slab = static_cast<int64_t>(m) * D;  // one (h, j, r) block of part
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int f = ftile * 32 + ty + 8 * k, d = dtile * 32 + tx;
    float acc = 0.f;
    for (int c = 0; c < slots; ++c)
      for (int hi = 0; hi < heads_per_out; ++hi) {
        const int64_t h = ho * heads_per_out + hi;
        acc += part[((static_cast<int64_t>(c) * H + h) * PT + jr) * slab +
                    static_cast<int64_t>(f) * D + d];
      }
    tile[ty + 8 * k][tx] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = dtile * 32 + ty + 8 * k, f = ftile * 32 + tx;
    dtheta[(ho * PT + jr) * slab + static_cast<int64_t>(d) * m + f] = tile[tx][ty + 8 * k];
  }
}

int bwd_key(const FeatShape& s) {
  if (s.m % 32 != 0) return 0;
  const int key = s.d * 10000 + s.p * 100 + s.t;
  switch (key) {
    case 1280204:
    case 1280201:
    case 640204:
    case 640201: return key;
    default: return 0;
  }
}

// Row chunks of the dTheta kernel: about 1024 workgroups in all, each chunk
// a whole number of the kernel's steps (32 rows for t = 4, 128 for t = 1)
// and at least 1024 rows, so that a workgroup reads more X and dphi than it
// writes partial dTheta.
struct BwdPlan {
  int chunks;
  int64_t chunk_rows;
  int slots;  // partial dTheta slots: chunks, or 4 per chunk for t = 1
};

BwdPlan bwd_plan(const FeatShape& s) {
  const int64_t step = s.t == 4 ? 32 : 128;
  const int64_t R = s.B * s.n;
  const int64_t steps = (R + step - 1) / step;
  const int64_t wgs = static_cast<int64_t>(s.m / 32) * s.H;
  int64_t c = wgs > 0 ? (1024 + wgs - 1) / wgs : 1;
  if (c > (R + 1023) / 1024) c = (R + 1023) / 1024;
  if (c > steps) c = steps;
  BwdPlan p{};
  if (c < 1) return p;  // no rows
  const int64_t per = (steps + c - 1) / c;
  p.chunk_rows = per * step;
  p.chunks = static_cast<int>((steps + per - 1) / per);
  p.slots = s.t == 4 ? p.chunks : 4 * p.chunks;
  return p;
}

template <int D, int P, int T, bool GB>
hipError_t launch_bwd_t(const FeatShape& s, const BwdArgs& a, float* dtheta, hipStream_t st) {
  using G = BwdGeom<D, P, T>;
  const int64_t R = s.B * s.n;
  const int64_t hout = s.theta_per_head ? s.H : 1;
  const int hpo = s.theta_per_head ? 1 : static_cast<int>(s.H);
  const int slots = T == 4 ? a.chunks : 4 * a.chunks;
  if (R > 0) {
    const int64_t tiles = (R + 127) / 128;
    if (tiles > 0x7fffffffLL || s.H > 65535) return hipErrorInvalidValue;
    auto* kx = featmap_bwd_dx<D, P, T, GB>;
    hipError_t e = allow_lds(kx, G::theta_lds());
    if (e != hipSuccess) return e;
    LLOPS_LAUNCH("featmap_bwd_dx", st, kx,
                 dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(s.H)), dim3(256),
                 G::theta_lds(), st, a);
    const size_t lds = G::theta_lds() + G::x_lds() + G::exch_lds();
    auto* kt = featmap_bwd_dth<D, P, T, GB>;
    e = allow_lds(kt, lds);
    if (e != hipSuccess) return e;
    const int64_t wgs = static_cast<int64_t>(s.m / 32) * a.chunks * s.H;
    if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
    LLOPS_LAUNCH("featmap_bwd_dth", st, kt, dim3(static_cast<unsigned>(wgs)), dim3(256), lds, st,
                 a);
  }
  const int64_t rx = hout * P * T * (s.m / 32);
  if (rx > 0x7fffffffLL) return hipErrorInvalidValue;
  LLOPS_LAUNCH("featmap_bwd_reduce", st, featmap_bwd_reduce,
               dim3(static_cast<unsigned>(rx), static_cast<unsigned>(D / 32)),
               dim3(256), 0, st, a.part, dtheta, R > 0 ? slots : 0, s.H, hpo, P * T, D, s.m);
  return hipGetLastError();
}

template <int D, int P, int T>
hipError_t launch_bwd_g(const FeatShape& s, const BwdArgs& a, int dphi_bf16, float* dtheta,
                        hipStream_t st) {
  return dphi_bf16 ? launch_bwd_t<D, P, T, true>(s, a, dtheta, st)
                   : launch_bwd_t<D, P, T, false>(s, a, dtheta, st);
}

}  // namespace

bool featmap_bwd_supported(const FeatShape& s) { return bwd_key(s) != 0; }

size_t featmap_bwd_ws_bytes(const FeatShape& s) {
  if (!bwd_key(s)) return 0;
  const BwdPlan p = bwd_plan(s);
  return static_cast<size_t>(p.slots) * s.H * s.p * s.t * s.m * s.d * sizeof(float);
}

hipError_t launch_featmap_bwd(const FeatShape& s, const void* X, const void* theta,
                              const void* dphi, int dphi_bf16, float* dX, float* dtheta,
                              void* ws, hipStream_t st) {
  const BwdPlan p = bwd_plan(s);
  BwdArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.theta = static_cast<const uint16_t*>(theta);
  a.dphi = dphi;
  a.dX = dX;
  a.part = static_cast<float*>(ws);
  a.B = s.B;
  a.H = s.H;
  a.n = s.n;
  a.m = s.m;
  a.th_hstride = s.theta_per_head ? static_cast<int64_t>(s.p) * s.t * s.d * s.m : 0;
  a.square = s.square;
  a.chunks = p.chunks;
  a.chunk_rows = p.chunk_rows;
  switch (bwd_key(s)) {
    case 1280204: return launch_bwd_g<128, 2, 4>(s, a, dphi_bf16, dtheta, st);
    case 1280201: return launch_bwd_g<128, 2, 1>(s, a, dphi_bf16, dtheta, st);
    case 640204: return launch_bwd_g<64, 2, 4>(s, a, dphi_bf16, dtheta, st);
    case 640201: return launch_bwd_g<64, 2, 1>(s, a, dphi_bf16, dtheta, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace llops
