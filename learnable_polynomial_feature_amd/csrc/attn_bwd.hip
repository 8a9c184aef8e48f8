// Element-wise and row-copy kernels of the causal linear-attention backward.
//
// For out = M V [/ (M 1 + delta)], M = tril(phi_Q phi_K^T), and an upstream
// gradient G of out, the chain rule (LLoPS paper, Sec. 1 form of the
// attention; the normalised numerator/denominator form of the Performer
// section of the low-rank-attention post, with SLAY's +delta) gives
//   dnum = G / den,  dden = -sum_v(G * out) / den      (plain: dnum = G, dden = 0)
//   dM = tril(dnum V^T + dden 1^T)
//   dphi_Q = dM phi_K,  dphi_K = dM^T phi_Q,  dV = M^T dnum.
// Each of the three is itself a causal (or, in reversed token order, causal)
// linear attention over features the library already contracts:
//   dphi_Q_i = sum_{j<=i} (a_i . b_j) phi_K_j   with a = [dnum | dden | 0], b = [V | 1 | 0];
//   dphi_K and dV are the same sums over i >= j, i.e. causal sums over the
//   reversed sequence.
// The host side (abi.cpp) runs them on the forward's segment kernels; the
// kernels here build a and b, reverse or slice rows, and scatter results.
#include "device.h"
#include "kernels.h"

namespace llops {
namespace {

// dst[bh][i'][doff + c] = src[bh][i][soff + c] for c < width, i' = n-1-i when
// reversing (else i); fp32 -> bf16 rounds to nearest even. Eight elements per
// thread; widths are multiples of 8, rows * width / 8 < 2^31.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void rows_copy(const TI* __restrict__ src, int sw, int soff,
                                                 TO* __restrict__ dst, int dw, int doff,
                                                 int width, int n, int rows, int rev) {
  const int q = width / 8;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * q) return;
  const int r = idx / q;
  const int c = (idx - r * q) * 8;
  const int bh = r / n, i = r - bh * n;
  const int64_t ro = rev ? static_cast<int64_t>(bh) * n + (n - 1 - i) : r;
  const TI* s = src + static_cast<int64_t>(r) * sw + soff + c;
  TO* d = dst + ro * dw + doff + c;
  if constexpr (sizeof(TI) == 2 && sizeof(TO) == 2) {
    st16(d, ld16(s));
  } else if constexpr (sizeof(TI) == 4 && sizeof(TO) == 4) {
    st16(d, ld16(s));
    st16(d + 4, ld16(s + 4));
  } else {  // fp32 -> bf16
    const u32x4 lo = ld16(s), hi = ld16(s + 4);
    st16(d, u32x4{pack_bf16x2(__uint_as_float(lo[0]), __uint_as_float(lo[1])),
                  pack_bf16x2(__uint_as_float(lo[2]), __uint_as_float(lo[3])),
                  pack_bf16x2(__uint_as_float(hi[0]), __uint_as_float(hi[1])),
                  pack_bf16x2(__uint_as_float(hi[2]), __uint_as_float(hi[3]))});
  }
}

// Column 0 of a [rows][16] bf16 block is 1, the rest 0: values whose causal
// sum is the denominator M 1.
__global__ __launch_bounds__(256) void fill_ones16(uint16_t* __restrict__ dst, int64_t rows) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= rows * 16) return;
  dst[idx] = (idx % 16) == 0 ? 0x3F80u : 0u;
}

// 32 lanes per row, eight rows per workgroup: from num (fp32 [rows][dv]),
// the plain causal sums den1 (fp32 [rows][16], column 0 = M 1), the upstream
// gradient G (fp32) and V (bf16), writes a = [dnum | dden | 0] and
// b = [V | 1 | 0] (bf16 [rows][MA]), with rev also in reversed row order
// (ra, rb), and dnum (bf16 [rows][dv]) reversed when rev, else in order. A
// lane owns 8 consecutive columns and writes them as one 16-byte store; dv
// and MA are multiples of 8, MA <= 256.
__global__ __launch_bounds__(256) void make_ab(const float* __restrict__ num,
                                              const float* __restrict__ den1,
                                              const float* __restrict__ G,
                                              const uint16_t* __restrict__ V, int dv, int MA,
                                              int64_t n, int64_t rows, int normalize, float delta,
                                              uint16_t* __restrict__ a, uint16_t* __restrict__ ra,
                                              uint16_t* __restrict__ b, uint16_t* __restrict__ rb,
                                              uint16_t* __restrict__ rdnum, int rev) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  const int l = threadIdx.x & 31;
  const bool live = r < rows;  // every lane joins the shuffles below
  const int64_t rc = live ? r : rows - 1;
  const int64_t bh = rc / n, i = rc - bh * n;
  const int64_t rr = rev ? bh * n + (n - 1 - i) : rc;
  const float den = normalize ? den1[rc * 16] + delta : 1.f;
  const float inv = 1.f / den;
  const int c0 = 8 * l;  // this lane's columns c0 .. c0+7
  float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float dot = 0.f;
  if (c0 < dv) {
    const u32x4 g0 = ld16(G + rc * dv + c0), g1 = ld16(G + rc * dv + c0 + 4);
    const u32x4 n0 = ld16(num + rc * dv + c0), n1 = ld16(num + rc * dv + c0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g[e] = __uint_as_float(g0[e]);
      g[4 + e] = __uint_as_float(g1[e]);
      dot += g[e] * (__uint_as_float(n0[e]) * inv) + g[4 + e] * (__uint_as_float(n1[e]) * inv);
    }
  }
  // dden = -(G . out) / den with out = num / den (sum over the row's 32 lanes)
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 32);
  const float dden = normalize ? -dot * inv : 0.f;
  if (!live || c0 >= MA) return;
  u32x4 av, bv;
  if (c0 + 8 <= dv) {
    av = u32x4{pack_bf16x2(g[0] * inv, g[1] * inv), pack_bf16x2(g[2] * inv, g[3] * inv),
               pack_bf16x2(g[4] * inv, g[5] * inv), pack_bf16x2(g[6] * inv, g[7] * inv)};
    bv = ld16(V + rc * dv + c0);
    st16(rdnum + rr * dv + c0, av);
  } else {  // c0 == dv: the dden and ones column, then zeros
    const bool first = c0 == dv;
    av = u32x4{first ? static_cast<uint32_t>(f32_to_bf16(dden)) : 0u, 0u, 0u, 0u};
    bv = u32x4{first ? 0x3F80u : 0u, 0u, 0u, 0u};
  }
  st16(a + rc * MA + c0, av);
  st16(b + rc * MA + c0, bv);
  if (rev) {
    st16(ra + rr * MA + c0, av);
    st16(rb + rr * MA + c0, bv);
  }
}

unsigned blocks_for(int64_t work, int per) {
  return static_cast<unsigned>((work + per - 1) / per);
}

template <typename TI, typename TO>
hipError_t rows_copy_t(const TI* src, int sw, int soff, TO* dst, int dw, int doff, int width,
                       int64_t n, int64_t rows, int rev, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (width % 8 || rows * (width / 8) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  LLOPS_LAUNCH("attn_bwd_rows", st, (rows_copy<TI, TO>),
               dim3(blocks_for(rows * (width / 8), 256)), dim3(256), 0, st, src, sw, soff, dst, dw,
               doff, width, static_cast<int>(n), static_cast<int>(rows), rev);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rows_copy_bf16(const uint16_t* src, int sw, int soff, uint16_t* dst, int dw,
                                 int doff, int width, int64_t n, int64_t rows, int rev,
                                 hipStream_t st) {
  return rows_copy_t(src, sw, soff, dst, dw, doff, width, n, rows, rev, st);
}

hipError_t launch_rows_copy_f32(const float* src, int sw, int soff, float* dst, int dw, int doff,
                                int width, int64_t n, int64_t rows, int rev, hipStream_t st) {
  return rows_copy_t(src, sw, soff, dst, dw, doff, width, n, rows, rev, st);
}

hipError_t launch_rows_copy_f32_bf16(const float* src, int sw, int soff, uint16_t* dst, int dw,
                                     int doff, int width, int64_t n, int64_t rows, int rev,
                                     hipStream_t st) {
  return rows_copy_t(src, sw, soff, dst, dw, doff, width, n, rows, rev, st);
}

hipError_t launch_fill_ones16(uint16_t* dst, int64_t rows, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  LLOPS_LAUNCH("attn_bwd_ones", st, fill_ones16, dim3(blocks_for(rows * 16, 256)), dim3(256), 0,
               st, dst, rows);
  return hipGetLastError();
}

hipError_t launch_make_ab(const float* num, const float* den1, const float* G, const uint16_t* V,
                          int dv, int MA, int64_t n, int64_t rows, int normalize, float delta,
                          uint16_t* a, uint16_t* ra, uint16_t* b, uint16_t* rb, uint16_t* rdnum,
                          int rev, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if ((rows + 7) / 8 > 0x7fffffffLL || dv % 8 || MA % 8 || MA > 256 || MA <= dv)
    return hipErrorInvalidValue;
  LLOPS_LAUNCH("attn_bwd_make_ab", st, make_ab, dim3(static_cast<unsigned>((rows + 7) / 8)),
               dim3(256), 0, st, num, den1, G, V, dv, MA, n, rows, normalize, delta, a, ra, b, rb,
               rdnum, rev);
  return hipGetLastError();
}

}  // namespace llops
