// LLoPS feature-map backward. For an upstream gradient dphi, the gradients of
// L = sum(dphi * phi) with respect to X and Theta, by the chain rule through
// phi = [sum_r prod_j X Theta_{j,r}]^(2 if square) (LLoPS notes, key design 2;
// Theta is trained end to end, notes' training strategy):
//   Y_{j,r} = X Theta_{j,r},   s = sum_r prod_j Y_{j,r},   ds = dphi * 2s (square) or dphi
//   dY_{j,r} = ds * prod_{j' != j} Y_{j',r}
//   dX = sum_{j,r} dY_{j,r} Theta_{j,r}^T,   dTheta_{j,r} = X^T dY_{j,r}
//
// Both kernels recompute Y on 32x32x16 MFMA from one 32-feature block of
// every Theta_{j,r} at a time: nothing of size n x p*t*m is stored.
//
// dX (featmap_bwd_dx): a workgroup of 8 waves owns 256 rows (32 per wave) of
// one head and keeps their dX tile (rows x d) in registers. Per feature block
// it recomputes every Y_{j,r} once in the transposed orientation (features x
// rows; pass 1), forms s and ds, keeps the Y tiles as bf16 pairs, and adds
// dY_{j,r} Theta_{j,r}^T (pass 2): dY as the A operand straight from
// registers. A small kernel first copies Theta into fragment order
// (pack_bwd_theta); pass 1 reads each 1 KiB fragment with lane-linear
// 16-byte LDS reads, pass 2 reads the same block transposed, and blocks are
// double-buffered in LDS, each landing by direct buffer-to-LDS copies while
// the previous one is used. With t > 1 and a squared map the kernel also
// stores ds for the dTheta kernel, in its own register order (32 contiguous
// bytes per lane).
//
// dTheta (featmap_bwd_dth): a workgroup owns one feature block, one head and
// one chunk of rows. Each wave keeps the Theta fragments of its rank in
// registers for the whole chunk and walks the chunk a step of rows at a time
// through three LDS row buffers. Y is recomputed in the natural orientation
// (rows x features), so dY^T is an A operand from registers and X (read
// transposed from LDS) the B operand. With t = 4 the four waves take one rank
// each over the same 32 rows and read ds from the dX kernel; with t = 1 each
// wave takes its own 32 of a 128-row step and forms s itself (one swizzled
// copy of the step's rows serves both its read patterns, xswz). A bf16
// gradient of whole steps travels with the X rows: each step's tile is staged
// once per workgroup and read back transposed by every wave. The workgroup
// writes its chunk's partial dTheta (one per wave for t = 1);
// featmap_bwd_reduce sums the partials (and the heads, for a shared Theta) in
// a fixed order and transposes.
#include <algorithm>
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace llops {
namespace {

struct BwdArgs {
  const uint16_t* X;      // [B][H][n][d] bf16
  const uint16_t* theta;  // [H'][p][t][d][m] bf16
  const void* dphi;       // [B][H][n][m], fp32 or bf16
  float* dX;              // [B][H][n][d]
  float* part;            // dTheta partials [slot][H][p][t][m][d]
  // ds of the squared map when t > 1 (else null), bf16 in the dX kernel's
  // register order: [H][ds_tph 32-row tiles][m/32][64 lanes][16]
  uint16_t* ds;
  int64_t ds_tph;         // ds tiles per head: 8 per 256-row workgroup of the dX kernel
  const uint16_t* pk;     // Theta^T fragments (pack_bwd_theta), [H'][m/32][t][p][d/16][64][8]
  int64_t pk_hstride;     // packed elements between heads (0 = shared)
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
  // Row strides of the dTheta kernel's staged blocks (elements). Transposing
  // reads (4 rows x 32 bytes per 16 lanes) are conflict free when rows sit
  // 64 bytes apart modulo 256 (measured: a 32-byte shift takes twice the LDS
  // cycles); 16-byte row reads (frag_nat, 16 lanes a cycle) when rows sit 16
  // bytes apart modulo 256.
  static constexpr int TW = PT * 32 + 32;  // staged Theta, read transposed
  static constexpr int XW = T == 1 ? D : D + 32;  // staged X (t = 1: unpadded, swizzled)
  static constexpr int RB = T == 4 ? 32 : 128;  // rows per step of the dTheta kernel
  static constexpr size_t theta_lds() { return 1ull * D * TW * 2; }
  static constexpr int XP = D + 8;          // second copy of staged X (t = 4), read as rows
  // One feature block of packed Theta: PT * KS fragments of 64 lanes x 8
  // elements (1 KiB); the dX kernel double-buffers it in LDS.
  static constexpr int NFR = PT * KS;
  static constexpr int BLK = NFR * 512;
  static constexpr size_t x_lds() {         // three row buffers, each with a gradient tile
    return 3ull * RB * ((T == 4 ? XW + XP : XW) + 32) * 2;
  }
  static_assert(PT % 2 == 0, "staged Theta rows need an even block count to stay conflict free");
  static_assert((PT * D * 4) % 256 == 0, "a Theta block splits evenly over the threads");
};

// Theta_{j,r}[k][fb*32 + c] -> Ts[k][(j*T + r)*32 + c] (row stride TW); NT
// threads, and all loads of a thread are issued before its first LDS store.
template <int D, int PT, int NT = 256>
__device__ __forceinline__ void stage_theta(uint16_t* Ts, int TW, const uint16_t* th, int m,
                                            int fb, int tid) {
  static_assert((PT * D * 4) % NT == 0, "a Theta block splits evenly over the threads");
  constexpr int TL = PT * D * 4 / NT;
  u32x4 tv[TL];
  // piece idx: 16 bytes of staged row k = idx / (4 PT) at column
  // 8 * (idx % (4 PT)); consecutive lanes fill a row
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    const int idx = tid + NT * i, k = idx / (4 * PT), pc = idx % (4 * PT);
    tv[i] = ld16(th + (static_cast<int64_t>(pc >> 2) * D + k) * m + fb * 32 + (pc & 3) * 8);
  }
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    const int idx = tid + NT * i, k = idx / (4 * PT), pc = idx % (4 * PT);
    st16(Ts + k * TW + pc * 8, tv[i]);
  }
}

// With t = 1 the dTheta kernel keeps one copy of each step's 128 rows of X
// (no room for a second) and reads it both ways: 16-byte row pieces (16 rows
// a cycle) and transposing reads (4 rows x 64 bytes a cycle, 4 rows aligned
// to 4). Rows are unpadded, and 16-byte chunk c of row r sits at chunk
// c ^ xswz(r): any 16 consecutive rows put one chunk in 16 different groups
// of 4 banks, and the 4 rows of a transposing read put their 4 chunks of a
// 32-column block in 4 different ones.
template <int D>
__device__ __forceinline__ int xswz(int r) {
  static_assert(D == 64 || D == 128, "rows of 8 or 16 chunks");
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int xswz_at(int r, int col) {  // element offset of (r, col)
  return r * D + (((col >> 3) ^ xswz<D>(r)) << 3) + (col & 7);
}
// frag_nat and frag_tr_nat's counterparts on a swizzled block
template <int D>
__device__ __forceinline__ bf16x8 frag_nat_swz(const uint16_t* base, int rbase, int kbase,
                                               int lane) {
  return as_bf16x8(ld16(base + xswz_at<D>(rbase + (lane & 31), kbase + 8 * (lane >> 5))));
}
template <int D>
__device__ __forceinline__ bf16x8 frag_tr_swz(const uint16_t* base, int kbase, int cbase, int lane) {
  const int s = lane & 15, G = lane >> 4;
  const int row = kbase + 4 * (G >> 1) + (s >> 2);
  const int col = cbase + (G & 1) * 16 + 4 * (s & 3);
  const uint2 lo = lds_tr64(base + xswz_at<D>(row, col));
  const uint2 hi = lds_tr64(base + xswz_at<D>(row + 8, col));
  return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
}

// Row t of a head's B*n rows is token i of sequence b, stored at sequence row
// (b*H + h)*n + i. A cursor holds (b, i) of a wave-uniform row t0, so the
// rows t0 + o nearby need no division: with n >= span (the largest o + 1)
// they cross at most one sequence boundary.
struct RowCursor {
  int64_t b, i;
};

__device__ __forceinline__ RowCursor cursor_at(int64_t t, const BwdArgs& a) {
  const int64_t b = t / a.n;
  return RowCursor{b, t - b * a.n};
}

__device__ __forceinline__ RowCursor cursor_advance(RowCursor c, int64_t by, const BwdArgs& a) {
  c.i += by;
  while (c.i >= a.n) {  // wave-uniform; one pass when n >= by
    c.i -= a.n;
    ++c.b;
  }
  return c;
}

template <bool ONE_WRAP>
__device__ __forceinline__ int64_t rho_near(const RowCursor& c, int64_t o, int64_t h,
                                            const BwdArgs& a) {
  int64_t i = c.i + o, b = c.b;
  if constexpr (ONE_WRAP) {
    const bool wrap = i >= a.n;
    i = wrap ? i - a.n : i;
    b = wrap ? b + 1 : b;
  } else {
    const int64_t q = i / a.n;
    b += q;
    i -= q * a.n;
  }
  return (b * a.H + h) * a.n + i;
}

// ---------------------------------------------------------------------------
// dX
// ---------------------------------------------------------------------------
// Theta^T in fragment order for the dX kernel. Fragment b = (r*P + j)*KS + ks
// of feature block fb is the A operand of Y^T = Theta^T X^T: lane l holds
// Theta_{j,r}[16ks + 8(l/32) + e][32fb + l%32], e < 8 (k = d in natural
// order), as one 16-byte chunk. Chunks sit at swizzled places within the
// fragment (packed_chunk) so that both reads of the dX kernel are free of LDS
// bank conflicts (64 banks of 4 bytes): its pass 1 reads each lane's chunk
// whole, its pass 2 reads 8-byte halves of chunks transposed (see
// featmap_bwd_dx). One thread packs one chunk.
__host__ __device__ constexpr int packed_chunk(int l, int odd) {
  // l = 32h + c: chunk 32h + (c & 16) + ((c + 8h) & 15), with bit 2 flipped
  // in fragments of odd ks. Any 16 consecutive lanes still take 16 different
  // chunks mod 16 (a 16-byte read serves 16 lanes a cycle, pass 1). The 16
  // (h, c) pairs of one transposed read, c in 4 consecutive features, take 8
  // chunks whole, and the other 16 lanes of the same cycle read the same
  // features of fragment ks + 1: the flip moves those to the other 8 chunks
  // mod 16 (pass 2).
  return (32 * (l >> 5) + (l & 16) + (((l & 31) + 8 * (l >> 5)) & 15)) ^ (odd ? 4 : 0);
}

__global__ __launch_bounds__(256) void pack_bwd_theta(const uint16_t* __restrict__ th,
                                                      uint16_t* __restrict__ pk, int64_t total,
                                                      int P, int T, int D, int m) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int KS = D / 16, NFR = P * T * KS, FB = m / 32;
  const int lane = static_cast<int>(idx & 63), hh = lane >> 5, c = lane & 31;
  const int64_t f = idx >> 6;  // fragment index over heads and blocks
  const int b = static_cast<int>(f % NFR);
  const int fb = static_cast<int>((f / NFR) % FB);
  const int64_t h = f / (static_cast<int64_t>(NFR) * FB);
  const int ks = b % KS, j = (b / KS) % P, r = b / (KS * P);
  const uint16_t* src = th + h * P * T * static_cast<int64_t>(D) * m +
                        ((static_cast<int64_t>(j) * T + r) * D + ks * 16 + 8 * hh) * m + fb * 32 + c;
  uint32_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = static_cast<uint32_t>(src[(2 * i) * static_cast<int64_t>(m)]) |
           (static_cast<uint32_t>(src[(2 * i + 1) * static_cast<int64_t>(m)]) << 16);
  st16(pk + (f * 64 + packed_chunk(lane, ks & 1)) * 8, u32x4{v[0], v[1], v[2], v[3]});
}

// LDS address of a shared-memory pointer, for the direct buffer-to-LDS copy
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_addr(uint16_t* p) {
  return reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(p));
}

// ds_read_b64_tr_b16 through an address-space cast, which keeps the pointer's
// shared array visible to the compiler (a cast through an integer hides it,
// and a read of unknown origin waits for every buffer-to-LDS copy in flight)
__device__ __forceinline__ uint2 tr64(const uint16_t* p) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, v);
}

// Every buffer-to-LDS copy this wave issued has landed.
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// GB: dphi is bf16 (else fp32).
// OW: n >= 32, so a wave's 32 rows cross at most one sequence boundary.
// SQ: the map is squared; with t > 1 the kernel then also stores ds (bf16)
// for the dTheta kernel.
//
// Per feature block the workgroup reads one packed Theta block from LDS in
// two ways: pass 1 takes fragment (r, j, ks) as the A operand of Y^T; pass 2
// needs Theta_{j,r} as the B operand of dY Theta^T (column d, k = features
// in P16 order), which is the same data transposed: two ds_read_b64_tr_b16
// per operand, each lane supplying 4 consecutive d of one feature (8 bytes of
// a chunk). Blocks are double-buffered: block fb+1 is copied into the other
// buffer while block fb is used, and one barrier per block separates them.
template <int D, int P, int T, bool GB, bool OW, bool SQ>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void featmap_bwd_dx(BwdArgs a) {
  using G = BwdGeom<D, P, T>;
  constexpr int KS = G::KS, DT = G::DT, PT = G::PT, NFR = G::NFR, BLK = G::BLK;
  constexpr bool WDS = SQ && T > 1;
  static_assert(NFR % 8 == 0, "a block's fragments split evenly over the 8 waves");
  // The two block buffers are distinct shared arrays, and the feature-block
  // loop below is unrolled by two so that every read names its buffer: the
  // compiler can then tell that a read of one never waits for the copy into
  // the other.
  __shared__ __align__(16) uint16_t LA[BLK];
  __shared__ __align__(16) uint16_t LB[BLK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, c32 = lane & 31;
  const int64_t h = blockIdx.y;
  const int64_t R = a.B * a.n;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 256 + w * 32;  // this wave's rows

  // X fragments (B operand of the transposed recompute): lane row t0 + c32,
  // k = 16ks + 8hh .. +7; zeros past the end
  bf16x8 xf[KS];
  const bool ok = t0 + c32 < R;
  const int64_t tb = t0 < R ? t0 : R - 1;  // a wave past the end reads the last row
  const RowCursor cur = cursor_at(tb, a);
  const int64_t rho = rho_near<OW>(cur, ok ? c32 : R - 1 - tb, h, a);
  {
    const uint16_t* src = a.X + rho * D + 8 * hh;
    u32x4 v[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) v[ks] = ld16(src + ks * 16);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) xf[ks] = as_bf16x8(ok ? v[ks] : u32x4{0u, 0u, 0u, 0u});
  }

  // This head's packed Theta, block fb at byte fb * NFR KiB; wave w copies
  // fragments w, w + 8, ... of a block, 16 bytes per lane.
  const __amdgpu_buffer_rsrc_t rpk =
      make_rsrc(a.pk + h * a.pk_hstride, static_cast<uint32_t>(a.m / 32) * (NFR * 1024u));
  auto copy_block = [&](uint16_t* dst, int fb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NFR / 8; ++i) {
      const int f = w + 8 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rpk, lds_addr(dst + f * 512), 16, lane * 16u,
                                               static_cast<uint32_t>(fb * NFR + f) * 1024u, 0, 0);
    }
  };
  // pass 1: this lane's chunk of a fragment of even (a_off) or odd ks
  const int a_off = packed_chunk(lane, 0) * 8, a_odd = packed_chunk(lane, 1) * 8;
  // pass 2: in the 16-lane group g4 = lane/16 of a transposing read, lane s
  // supplies d = 32dt + 16(g4 & 1) + 4(s & 3) .. +3 (fragment ks = 2dt + (g4 & 1),
  // lane half (s & 3) / 2, chunk half (s & 1)) of feature row
  // 16hf + 4(g4 / 2) + s / 4, and 8 rows further for the second read
  const int g4 = lane >> 4, s4 = lane & 15;
  auto b_off = [&](int c) {
    return (g4 & 1) * 512 + packed_chunk(32 * ((s4 & 3) >> 1) + c, g4 & 1) * 8 + (s4 & 1) * 4;
  };
  const int crow = 4 * (g4 >> 1) + (s4 >> 2);
  const int b_lo0 = b_off(crow), b_hi0 = b_off(crow + 8);
  const int b_lo1 = b_off(16 + crow), b_hi1 = b_off(24 + crow);

  // upstream gradient of this lane's row, features fb*32 + 8i + 4hh + {0..3},
  // as raw bits until ds is formed
  u32x4 gr[GB ? 2 : 4];
  auto load_g = [&](int fb) __attribute__((always_inline)) {
    const int64_t base = rho * a.m + fb * 32 + 4 * hh;
    if constexpr (GB) {
      const uint16_t* src = static_cast<const uint16_t*>(a.dphi) + base;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(src + 16 * i);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(src + 16 * i + 8);
        gr[i] = u32x4{v0[0], v0[1], v1[0], v1[1]};
      }
    } else {
      const float* src = static_cast<const float*>(a.dphi) + base;
#pragma unroll
      for (int i = 0; i < 4; ++i) gr[i] = ld16(src + 8 * i);
    }
  };
  auto g_at = [&](int i, int e) __attribute__((always_inline)) {
    if constexpr (GB) {
      const uint32_t u = gr[i / 2][2 * (i % 2) + e / 2];
      return __uint_as_float(e & 1 ? u & 0xffff0000u : u << 16);
    } else {
      return __uint_as_float(gr[i][e]);
    }
  };

  f32x16 dx[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dx[dt] = zero16();
  const int FB = a.m / 32;
  // ds of the previous block, stored at the top of the next iteration, ahead
  // of the copies: memory operations count down in issue order, so a wait
  // for a store (before its registers are reused) placed after the copies
  // would also wait for them. Block 0's tile first takes zeros, overwritten
  // in order by the same lanes.
  u32x4 dsp[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
  auto store_ds = [&](int fb) __attribute__((always_inline)) {
    if constexpr (WDS) {  // this wave's 32 x 32 tile, 32 contiguous bytes per lane
      uint16_t* dst = a.ds + ((h * a.ds_tph + t0 / 32) * FB + fb) * 1024 + lane * 16;
      st16(dst, dsp[0]);
      st16(dst + 8, dsp[1]);
    }
  };
  // one feature block: blk holds it, nxt takes the next one
  auto block = [&](const uint16_t* blk, uint16_t* nxt, int fb) __attribute__((always_inline)) {
    // lane offsets made opaque per block, so the fragment addresses of the
    // two buffers are formed here (base + immediate) instead of being
    // hoisted out of the loop into registers of their own
    int ao = a_off, ao1 = a_odd, bl0 = b_lo0, bh0 = b_hi0, bl1 = b_lo1, bh1 = b_hi1;
    asm volatile("" : "+v"(ao), "+v"(ao1), "+v"(bl0), "+v"(bh0), "+v"(bl1), "+v"(bh1));
    store_ds(fb > 0 ? fb - 1 : 0);
    // the gradient next, so that waiting for it leaves the copies below in
    // flight
    load_g(fb);
    // the next block lands in the other buffer, last read before the
    // previous barrier (the last block copies itself again: a branch here
    // costs the allocator registers)
    copy_block(nxt, fb + 1 < FB ? fb + 1 : fb);

    // Pass 1, rank by rank: Y_{j,r} transposed (element 4i+e is feature
    // 8i + 4hh + e of row t0 + c32), its P chains interleaved over k, kept as
    // bf16 pairs; s for a squared map. Theta fragments are read two MFMAs
    // ahead.
    constexpr int NA = PT * KS;
    auto read_a = [&](int idx) __attribute__((always_inline)) {
      // idx = (r*KS + ks)*P + j
      const int j = idx % P, ks = (idx / P) % KS, r = idx / (P * KS);
      return as_bf16x8(
          *reinterpret_cast<const u32x4*>(blk + ((r * P + j) * KS + ks) * 512 + (ks & 1 ? ao1 : ao)));
    };
    uint32_t yb[PT][8];
    f32x16 s = zero16();
    f32x16 yv[P];
    bf16x8 fr[3];
    fr[0] = read_a(0);
    fr[1] = read_a(1);
#pragma unroll
    for (int r = 0; r < T; ++r) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < P; ++j) {
          const int idx = (r * KS + ks) * P + j;
          if (idx + 2 < NA) fr[(idx + 2) % 3] = read_a(idx + 2);
          __builtin_amdgcn_sched_barrier(0);
          yv[j] = mfma32x32x16(fr[idx % 3], xf[ks], ks == 0 ? zero16() : yv[j]);
          __builtin_amdgcn_sched_barrier(0);
        }
      if constexpr (SQ) {
        f32x16 prod = yv[0];
#pragma unroll
        for (int jj = 1; jj < P; ++jj) prod *= yv[jj];
        s += prod;
      }
#pragma unroll
      for (int jj = 0; jj < P; ++jj)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          yb[jj * T + r][k] = pack_bf16x2(yv[jj][2 * k], yv[jj][2 * k + 1]);
    }
    f32x16 ds;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float gv = g_at(i, e);
        ds[4 * i + e] = ok ? (SQ ? 2.f * s[4 * i + e] * gv : gv) : 0.f;
      }
    if constexpr (WDS) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        dsp[q] = u32x4{pack_bf16x2(ds[8 * q + 0], ds[8 * q + 1]),
                       pack_bf16x2(ds[8 * q + 2], ds[8 * q + 3]),
                       pack_bf16x2(ds[8 * q + 4], ds[8 * q + 5]),
                       pack_bf16x2(ds[8 * q + 6], ds[8 * q + 7])};
    }
    // Pass 2, over (r, j): dY_{j,r} = ds * prod_{j' != j} Y_{j',r} in
    // registers, then dX[rows][d] += dY[rows][f] Theta^T[f][d]: dY as the A
    // operand (lane row, k = features in P16 order), Theta^T by transposing
    // reads of the block, two MFMAs ahead.
    constexpr int NB = PT * 2 * DT;
    auto read_b = [&](int idx) __attribute__((always_inline)) {
      const int q = idx / (2 * DT), hf = (idx / DT) % 2, dt = idx % DT;
      const uint16_t* base = blk + (q * KS + 2 * dt) * 512;
      const uint2 lo = tr64(base + (hf ? bl1 : bl0));
      const uint2 hi = tr64(base + (hf ? bh1 : bh0));
      return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
    };
    fr[0] = read_b(0);
    fr[1] = read_b(1);
    bf16x8 af[2];
#pragma unroll
    for (int q = 0; q < PT; ++q)
#pragma unroll
    for (int hd = 0; hd < 2 * DT; ++hd) {
      const int idx = q * 2 * DT + hd, hf = hd / DT, dt = hd % DT, r = q / P, j = q % P;
      if (idx + 2 < NB) fr[(idx + 2) % 3] = read_b(idx + 2);
      if (hf == 0 && dt == 0) {
        f32x16 dy = ds;
#pragma unroll
        for (int jj = 0; jj < P; ++jj) {
          if (jj == j) continue;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t u = yb[jj * T + r][k];
            dy[2 * k] *= __uint_as_float(u << 16);
            dy[2 * k + 1] *= __uint_as_float(u & 0xffff0000u);
          }
        }
        af[0] = acc_frag(dy, 0);
        af[1] = acc_frag(dy, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      dx[dt] = mfma32x32x16(af[hf], fr[idx % 3], dx[dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_copies();
    __syncthreads();  // the next block has landed; every wave is done with this one
  };
  copy_block(LA, 0);
  wait_copies();
  __syncthreads();
  for (int fb = 0;; fb += 2) {
    block(LA, LB, fb);
    if (fb + 1 >= FB) break;
    block(LB, LA, fb + 1);
    if (fb + 2 >= FB) break;
  }
  store_ds(FB - 1);
  // dx[dt] element 4i+e: row t0 + 8i + 4hh + e, column dt*32 + c32
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int o = 8 * i + 4 * hh + e;
      if (t0 + o < R) {
        float* dst = a.dX + rho_near<OW>(cur, o, h, a) * D + c32;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) dst[dt * 32] = dx[dt][4 * i + e];
      }
    }
}

// ---------------------------------------------------------------------------
// dTheta partials
// ---------------------------------------------------------------------------
// RM, how a step's rows map to sequence rows: 2 = n is a multiple of the
// step, so a step's rows are consecutive in memory; 1 = n >= the step, so a
// step crosses at most one sequence boundary; 0 = any n.
// GB: the gradient read (dphi, or ds from the dX kernel) is bf16.
// With t = 4 and a squared map the gradient read is ds itself; with t = 1
// and a squared map each wave forms s from its own (only) rank.
template <int D, int P, int T, bool GB, int RM, bool DS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void featmap_bwd_dth(BwdArgs a) {
  static_assert(!DS || GB, "ds is bf16");
  using G = BwdGeom<D, P, T>;
  constexpr int KS = G::KS, DT = G::DT, TW = G::TW, XW = G::XW, PT = G::PT;
  static_assert(T == 1 || T == 4, "one rank per wave (t = 4) or one rank for all (t = 1)");
  constexpr int RB = G::RB;                 // rows per step
  constexpr int XL = RB * (D / 8) / 256;    // 16-byte pieces of a step's X per thread
  static_assert(XL >= 1 && RB * (D / 8) % 256 == 0, "a step's rows split evenly over the threads");
  // LDS: the staged Theta block at the start; once each wave holds its
  // rank's Theta fragments in registers, the same bytes hold three steps'
  // rows of X.
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* Ts = smem;
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
  const void* gsrc = DS ? static_cast<const void*>(a.ds) : a.dphi;
  const bool own_s = T == 1 && a.square;
  // element of ds for head-local row t, feature fb*32 + f (the dX kernel's
  // tile order: lane 32 (f/4 % 2) + t % 32, element 4 (f/8) + f % 4)
  auto ds_at = [&](int64_t t, int f) __attribute__((always_inline)) {
    return ((h * a.ds_tph + (t >> 5)) * FB + fb) * 1024 +
           (32 * ((f >> 2) & 1) + (t & 31)) * 16 + 4 * (f >> 3) + (f & 3);
  };
  // GT: a bf16 gradient whose step rows are consecutive travels with the X
  // rows: each step's RB x 32 tile is requested once per workgroup (8 bytes
  // per thread and 32 rows), staged in LDS, and each wave reads its 16 values
  // with two transposing reads instead of 16 two-byte loads of its own.
  constexpr bool GT = GB && RM == 2;
  constexpr int GL = GT ? RB / 32 : 1;  // 8-byte gradient pieces per thread and step
  // ds tile pieces (GT, DS): wave w moves rows 8w .. 8w + 7, lane l the 8
  // bytes at 8l of them (row 8w + l/8, features 4 (l % 8) .. + 3: elements
  // 4 ((l/2) % 4) .. + 3 of dX lane 32 (l % 2) + row), so its 64 shared-memory
  // stores fill 512 contiguous bytes in lane order
  const int ds_row = 8 * w + (lane >> 3);

  stage_theta<D, PT>(Ts, TW, a.theta + h * a.th_hstride, a.m, fb, tid);
  __syncthreads();
  // B operands of Y_{j,rk} = X Theta_{j,rk}: Theta rows 16ks.. in natural k
  // order (to pair with X rows read as 16-byte pieces), lane column c32 =
  // feature fb*32 + c32; held for the whole chunk
  bf16x8 tf[P][KS];
#pragma unroll
  for (int j = 0; j < P; ++j)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) tf[j][ks] = frag_tr_nat(Ts, TW, ks * 16, (j * T + rk) * 32, lane);

  f32x16 acc[P][DT];
#pragma unroll
  for (int j = 0; j < P; ++j)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[j][dt] = zero16();

  // A step's X (row-major), requested two steps ahead, and its gradient
  // (element 4i+e: row wr + 8i + 4hh + e of the step, feature fb*32 + c32),
  // requested one step ahead and kept as raw bits until the step widens it.
  // Requests never pass the chunk's last step (RM 2: whole steps); with
  // other RM a partial step's rows past the chunk read as its last row.
  u32x4 xv[XL];
  u32x2 gv[GL];  // GT: this thread's pieces of a step's gradient tile
  uint32_t gn[GT ? 1 : 16];
  constexpr uint32_t ES = GB ? 2 : 4;
  // RM 2: the first row (in [B][H][n] order) of the step whose X was
  // requested last, and the offset of its ds tile, kept incrementally by
  // advance() below: a step never straddles two sequences, so stepping is an
  // add (and a hop to the next sequence), not a division and 64-bit products
  int64_t xrow = 0, dsoff = 0;
  auto load_x = [&](const RowCursor& c, int64_t t) __attribute__((always_inline)) {
    if constexpr (RM == 2) {  // the step's rows are consecutive in memory
      (void)c;
      (void)t;
      const int64_t row0 = xrow;  // whole steps: RB rows each
      const auto rx = make_rsrc(a.X + row0 * D, static_cast<uint32_t>(RB) * D * 2u);
#pragma unroll
      for (int it = 0; it < XL; ++it) xv[it] = buf_ld16(rx, (tid + 256u * it) * 16u, 0u);
      if constexpr (GT && DS) {  // the step is one 2 KiB tile of ds
        static_assert(GL == 1, "ds exists for t = 4 only: one piece per thread");
        const auto rg = make_rsrc(a.ds + dsoff, 2048u);
        gv[0] = buf_ld8(rg, ((32 * (lane & 1) + ds_row) * 16 + 4 * ((lane >> 1) & 3)) * 2u);
      } else if constexpr (GT) {  // piece idx: row idx / 8, features fb*32 + 4 (idx % 8) .. + 3
        const auto rg = make_rsrc(static_cast<const uint16_t*>(gsrc) + row0 * a.m,
                                  static_cast<uint32_t>(RB) * static_cast<uint32_t>(a.m) * 2u);
#pragma unroll
        for (int it = 0; it < GL; ++it) {
          const uint32_t idx = tid + 256u * it;
          gv[it] = buf_ld8(rg, ((idx >> 3) * static_cast<uint32_t>(a.m) + fb * 32 + (idx & 7) * 4) * 2u);
        }
      }
    } else {
#pragma unroll
      for (int it = 0; it < XL; ++it) {
        const int idx = tid + 256 * it, rr = idx / (D / 8), q = idx % (D / 8);
        const int64_t o = t + rr < r1 ? rr : r1 - 1 - t;
        xv[it] = ld16(a.X + rho_near<RM == 1>(c, o, h, a) * D + q * 8);
      }
    }
  };
  auto load_g = [&](const RowCursor& c, int64_t t) __attribute__((always_inline)) {
    if constexpr (GT) {
      (void)c;
      (void)t;
    } else if constexpr (RM == 2) {
      (void)c;
      (void)t;
      const auto rg = make_rsrc(static_cast<const char*>(gsrc) + xrow * a.m * ES,
                                static_cast<uint32_t>(RB) * static_cast<uint32_t>(a.m) * ES);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t off =
              ((wr + 8 * i + 4 * hh + e) * static_cast<uint32_t>(a.m) + fb * 32 + c32) * ES;
          gn[4 * i + e] = GB ? buf_ld2(rg, off) : buf_ld4(rg, off);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t r = wr + 8 * i + 4 * hh + e;
          const int64_t o = t + r < r1 ? r : r1 - 1 - t;
          const int64_t idx =
              DS ? ds_at(t + o, c32) : rho_near<RM == 1>(c, o, h, a) * a.m + fb * 32 + c32;
          gn[4 * i + e] = GB ? static_cast<uint32_t>(static_cast<const uint16_t*>(gsrc)[idx])
                             : __float_as_uint(static_cast<const float*>(gsrc)[idx]);
        }
    }
  };
  // LDS per row buffer: the rows with stride XW (read transposed, B operands
  // of the dTheta product) and, for t = 4, again with stride XP (read as A
  // operands of Y); each stride keeps its own read pattern free of bank
  // conflicts. With t = 1 one swizzled copy (xswz) serves both.
  constexpr int XP = T == 4 ? G::XP : XW;
  constexpr int XBW = T == 4 ? RB * (XW + XP) : RB * XW;  // X rows of one buffer
  constexpr int BUFW = XBW + RB * 32;                      // then the gradient tile (GT)
  auto xbuf = [&](int k) __attribute__((always_inline)) { return smem + k * BUFW; };
  auto pbuf = [&](int k) __attribute__((always_inline)) {
    return T == 4 ? smem + k * BUFW + RB * XW : smem + k * BUFW;
  };
  // gradient tile: RB rows of 32 features, rows 64 bytes apart (conflict free
  // for the transposing reads)
  auto gbuf = [&](int k) __attribute__((always_inline)) { return smem + k * BUFW + XBW; };
  // piece `it` of the step's rows into buffer k
  auto store_piece = [&](int k, int64_t t, int it) __attribute__((always_inline)) {
    const int idx = tid + 256 * it, rr = idx / (D / 8), q = idx % (D / 8);
    // rows past the chunk read as zeros; with whole steps (RM 2) a step past
    // the chunk is never read, so its rows need no masking
    const u32x4 v = RM == 2 || t + rr < r1 ? xv[it] : u32x4{0u, 0u, 0u, 0u};
    if constexpr (T == 1) {
      st16(xbuf(k) + xswz_at<D>(rr, q * 8), v);
    } else {
      st16(xbuf(k) + rr * XW + q * 8, v);
      st16(pbuf(k) + rr * XP + q * 8, v);
    }
  };
  // the step's gradient tile (GT) into buffer k
  auto store_gtile = [&](int k) __attribute__((always_inline)) {
    if constexpr (GT && DS) {  // this thread's piece: row ds_row, features 4 (lane % 8) ..
      *reinterpret_cast<u32x2*>(gbuf(k) + ds_row * 32 + 4 * (lane & 7)) = gv[0];  // RM 2
    } else if constexpr (GT) {
#pragma unroll
      for (int it = 0; it < GL; ++it) {
        const int idx = tid + 256 * it, rr = idx >> 3;
        *reinterpret_cast<u32x2*>(gbuf(k) + rr * 32 + (idx & 7) * 4) = gv[it];  // RM 2
      }
    }
  };
  auto store_x = [&](int k, int64_t t) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < XL; ++it) store_piece(k, t, it);
    store_gtile(k);
  };
  auto widen = [&]() __attribute__((always_inline)) {
    f32x16 v = zero16();
    if constexpr (!GT) {
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = __uint_as_float(GB ? gn[k] << 16 : gn[k]);
    }
    return v;
  };
  // a step's gradient from its staged tile (two transposing reads, rows in
  // P16 order): element 4i+e is row wr + 8i + 4hh + e, column fb*32 + c32
  auto tile_g = [&](const u32x4& lo, const u32x4& hi) __attribute__((always_inline)) {
    f32x16 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(lo[q] << 16);
      v[2 * q + 1] = __uint_as_float(lo[q] & 0xffff0000u);
      v[8 + 2 * q] = __uint_as_float(hi[q] << 16);
      v[8 + 2 * q + 1] = __uint_as_float(hi[q] & 0xffff0000u);
    }
    return v;
  };
  // the cursor of the last step whose X was requested (it stays on the
  // chunk's last step once there)
  RowCursor cx = cursor_at(r0, a);
  int64_t tx = r0;
  const int64_t hop = RB + (a.H - 1) * a.n;  // RM 2: last step of a sequence -> next one's first
  if constexpr (RM == 2) {
    xrow = (cx.b * a.H + h) * a.n + cx.i;
    if constexpr (GT && DS) dsoff = ds_at(r0, 0);
  }
  auto advance = [&]() __attribute__((always_inline)) {
    if constexpr (RM == 2) {  // branch-free (selects), so the step stays one basic block
      const bool more = tx + RB < r1;
      tx += more ? RB : 0;
      const int64_t i = cx.i + (more ? RB : 0);  // n is a multiple of RB: i lands on n exactly
      const bool wrap = i >= a.n;
      cx.i = wrap ? 0 : i;
      cx.b += wrap ? 1 : 0;
      xrow += more ? (wrap ? hop : RB) : 0;
      if constexpr (GT && DS) dsoff += more ? FB * 1024 : 0;  // one 32-row ds tile per step
    } else if (tx + RB < r1) {
      tx += RB;
      cx = cursor_advance(cx, RB, a);
    }
  };

  // Three row buffers in rotation: step i reads buffer i%3 (its Y and dTheta
  // operands) and buffer (i+1)%3 (the next step's Y operands, read while
  // this step's products run), and fills buffer (i+2)%3, which was last read
  // before the previous barrier.
  load_x(cx, tx);  // step 0
  load_g(cx, tx);
  __syncthreads();  // every wave holds its Theta fragments: Ts may be overwritten
  store_x(0, r0);
  f32x16 g = widen();
  advance();
  load_x(cx, tx);  // step 1
  store_x(1, r0 + RB);
  load_g(cx, tx);
  advance();
  load_x(cx, tx);  // step 2
  __syncthreads();
  // this wave's X fragments: A operands of Y (row wr + lane%32, k = 16ks..
  // in natural order, one 16-byte read: t = 4 from the second copy) and B
  // operands of the dTheta product (k = rows wr + 16hf.., column dt*32 + c32)
  auto x_rows = [&](const uint16_t* buf, int ks) __attribute__((always_inline)) {
    if constexpr (T == 1)
      return frag_nat_swz<D>(buf, wr, ks * 16, lane);
    else
      return frag_nat(buf, XP, wr, ks * 16, lane);
  };
  bf16x8 xa[KS], xb[2][DT];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) xa[ks] = x_rows(pbuf(0), ks);
  int cur = 0, nxt = 1, fut = 2;
  // One step. With one wave per SIMD nothing else hides a wave's non-MFMA
  // work. With t = 1 (IL) the work that does not depend on this step's
  // products runs between them: the rows two steps ahead go into the free
  // buffer (last read before the previous barrier) one piece per Y k-step,
  // the next requests are issued between the rank's dTheta products, and the
  // dTheta product's X operands are read in two halves, so that at most 15
  // LDS reads are in flight (the range of the wait counter). With t = 4 the
  // stores and requests stay at the end of the step: its 32-row steps are
  // short, and rows requested half a step before they are stored arrive
  // late (measured: 2.29 against 2.10 ms; t = 1, 0.78 against 0.83 ms).
  constexpr bool IL = T == 1;
  auto read_xb = [&](int hf) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      xb[hf][dt] = T == 1 ? frag_tr_swz<D>(xbuf(cur), wr + hf * 16, dt * 32, lane)
                          : frag_tr(xbuf(cur), XW, wr + hf * 16, dt * 32, lane);
  };
  for (int64_t t0 = r0; t0 < r1; t0 += RB) {
    // Y_{j,rk} in the natural orientation: element 4i+e is row wr + 8i + 4hh + e
    // of the step, lane column c32 is feature fb*32 + c32. The first products
    // go ahead of the step's first reads: their accumulators are then live,
    // so no read's address is formed in them (a product writing a register a
    // read in flight still takes its address from waits for that read).
    f32x16 y[P];
#pragma unroll
    for (int j = 0; j < P; ++j) y[j] = zero16();
    u32x4 gtl, gth;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int j = 0; j < P; ++j) y[j] = mfma32x32x16(xa[ks], tf[j][ks], y[j]);
      auto read_rest = [&]() __attribute__((always_inline)) {
        read_xb(1);
        if constexpr (GT) {
          gtl = __builtin_bit_cast(u32x4, frag_tr(gbuf(cur), 32, wr, 0, lane));
          gth = __builtin_bit_cast(u32x4, frag_tr(gbuf(cur), 32, wr + 16, 0, lane));
        }
      };
      if (ks == 0) {
        __builtin_amdgcn_sched_barrier(0);
        read_xb(0);
        if constexpr (IL) store_gtile(fut);
        else read_rest();
      }
      if (IL && ks < XL) store_piece(fut, t0 + 2 * RB, ks);
      if (IL && ks == KS / 2) read_rest();
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next step's Y operands, in flight during this step's products
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) xa[ks] = x_rows(pbuf(nxt), ks);
    f32x16 ds;
    if constexpr (GT)
      ds = tile_g(gtl, gth);
    else
      ds = g;
    if (own_s) {
      f32x16 s = y[0];
#pragma unroll
      for (int j = 1; j < P; ++j) s *= y[j];
      ds *= 2.f * s;
    }
    if constexpr (RM != 2) {  // rows past the chunk (RM 2 steps are always whole)
      const int64_t left = r1 - t0 - wr - 4 * hh;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) ds[4 * i + e] = 8 * i + e < left ? ds[4 * i + e] : 0.f;
    }
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
        for (int dt = 0; dt < DT; ++dt) acc[j][dt] = mfma32x32x16(af, xb[hf][dt], acc[j][dt]);
      }
      if (IL && j == 0) {
        __builtin_amdgcn_sched_barrier(0);
        // the next step's gradient is widened and the one after it
        // requested; rows three steps ahead requested
        g = widen();
        load_g(cx, tx);
        advance();
        load_x(cx, tx);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!IL) {
      // rows two steps ahead into the free buffer; the next step's gradient
      // is widened and the one after it requested; rows three steps ahead
      // requested
      store_x(fut, t0 + 2 * RB);
      g = widen();
      load_g(cx, tx);
      advance();
      load_x(cx, tx);
    }
    const int k = cur;
    cur = nxt;
    nxt = fut;
    fut = k;
    __syncthreads();  // the stored rows are visible; this step's buffer is free
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
    const int64_t tiles = (R + 255) / 256;
    if (tiles > 0x7fffffffLL || s.H > 65535) return hipErrorInvalidValue;
    // with t > 1 and a squared map the dX kernel also stores ds (bf16) for
    // the dTheta kernel, which then reads it in place of dphi
    const bool wds = T > 1 && s.square;
    const int64_t pk_total = hout * P * T * D * s.m / 8;  // 16-byte chunks of packed Theta
    // the dX kernel addresses one head's packed Theta through a 32-bit range
    if ((pk_total + 255) / 256 > 0x7fffffffLL || pk_total * 16 / hout > 0xffffffffLL || !a.pk)
      return hipErrorInvalidValue;
    LLOPS_LAUNCH("pack_bwd_theta", st, pack_bwd_theta,
                 dim3(static_cast<unsigned>((pk_total + 255) / 256)), dim3(256), 0, st, a.theta,
                 const_cast<uint16_t*>(a.pk), pk_total, P, T, D, s.m);
    auto* kx = s.n >= 32 ? (s.square ? featmap_bwd_dx<D, P, T, GB, true, true>
                                     : featmap_bwd_dx<D, P, T, GB, true, false>)
                         : (s.square ? featmap_bwd_dx<D, P, T, GB, false, true>
                                     : featmap_bwd_dx<D, P, T, GB, false, false>);
    // the dX kernel's LDS (two packed blocks) is static
    LLOPS_LAUNCH("featmap_bwd_dx", st, kx,
                 dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(s.H)), dim3(512), 0,
                 st, a);
    const size_t lds = std::max(G::theta_lds(), G::x_lds());
    const int rm = s.n % G::RB == 0 ? 2 : s.n >= G::RB ? 1 : 0;
    constexpr bool DS = T > 1;  // the kernel reads ds (wds), which exists for t > 1 only
    auto* kt = wds ? (rm == 2 ? featmap_bwd_dth<D, P, T, true, 2, DS>
                      : rm == 1 ? featmap_bwd_dth<D, P, T, true, 1, DS>
                                : featmap_bwd_dth<D, P, T, true, 0, DS>)
                   : (rm == 2 ? featmap_bwd_dth<D, P, T, GB, 2, false>
                      : rm == 1 ? featmap_bwd_dth<D, P, T, GB, 1, false>
                                : featmap_bwd_dth<D, P, T, GB, 0, false>);
    const hipError_t e = allow_lds(kt, lds);
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

bool featmap_bwd_supported_impl(const FeatShape& s) { return bwd_key(s) != 0; }

// Scratch: the partial dTheta slots, then (t > 1, squared) ds in bf16, then
// Theta in the dX kernel's fragment order.
size_t bwd_part_bytes(const FeatShape& s) {
  const BwdPlan p = bwd_plan(s);
  const size_t b = static_cast<size_t>(p.slots) * s.H * s.p * s.t * s.m * s.d * sizeof(float);
  return (b + 255) / 256 * 256;
}

// ds tiles per head: one per 32 rows of every 256-row dX workgroup
int64_t bwd_ds_tph(const FeatShape& s) { return (s.B * s.n + 255) / 256 * 8; }

// ds in bf16 (t > 1, squared), in 32-row tiles of 32 x m
size_t bwd_ds_bytes(const FeatShape& s) {
  if (!(s.t > 1 && s.square) || s.B * s.n == 0) return 0;
  return static_cast<size_t>(s.H) * bwd_ds_tph(s) * 32 * s.m * sizeof(uint16_t);
}

// Theta in the dX kernel's fragment order (rows > 0 only)
size_t bwd_pack_bytes(const FeatShape& s) {
  if (static_cast<size_t>(s.B) * s.H * s.n == 0) return 0;
  const size_t th_heads = s.theta_per_head ? s.H : 1;
  const size_t b = th_heads * s.p * s.t * s.d * s.m * sizeof(uint16_t);
  return (b + 255) / 256 * 256;
}

}  // namespace

bool featmap_bwd_supported(const FeatShape& s) { return featmap_bwd_supported_impl(s); }

size_t featmap_bwd_ws_bytes(const FeatShape& s) {
  if (!bwd_key(s)) return 0;
  return bwd_part_bytes(s) + bwd_ds_bytes(s) + bwd_pack_bytes(s);
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
  a.ds = s.t > 1 && s.square && ws
             ? reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + bwd_part_bytes(s))
             : nullptr;
  a.ds_tph = bwd_ds_tph(s);
  if (ws && bwd_pack_bytes(s))
    a.pk = reinterpret_cast<const uint16_t*>(static_cast<char*>(ws) + bwd_part_bytes(s) +
                                             bwd_ds_bytes(s));
  a.pk_hstride = s.theta_per_head ? static_cast<int64_t>(s.p) * s.t * s.d * s.m : 0;
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
