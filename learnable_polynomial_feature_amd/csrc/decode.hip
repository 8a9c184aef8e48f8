// LLoPS single-token decode step on the recurrent state (LLoPS paper Sec. 1:
// linear attention as a recurrent memory state updated token by token).
//   S += phi_K(k) v^T;  z += phi_K(k);  out = phi_Q(q)^T S [/(phi_Q(q)^T z + delta)]
// The state update precedes the read (inclusive of the new token). The gated
// form first scales S and z by a = exp(g) for a per-(batch, head) log gate g
// (the forgetting gates the LLoPS notes name as future work, limitations and
// outlook).
//
// One workgroup per (batch, head). The m x dv fp32 state is streamed once:
// each thread owns 4 adjacent columns (16-byte non-temporal loads/stores) of
// every (256 / (dv/4))-th row, updates them in registers and accumulates the
// read-out partial; partials are reduced across row groups in a fixed order.
// The kernel is bound by HBM bandwidth: 2 * m * dv * 4 bytes of state per
// (batch, head) against ~3 flops per state element.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace llops {
namespace {

template <bool VBF16>
__device__ __forceinline__ float4 load_v4(const void* v, int64_t idx) {
  if (VBF16) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(v) + idx);
    return make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                       __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(v) + idx);
  }
}

template <bool VBF16>
__device__ __forceinline__ float load_v1(const void* v, int64_t idx) {
  if (VBF16) return bf16_to_f32(static_cast<const uint16_t*>(v)[idx]);
  return static_cast<const float*>(v)[idx];
}

__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

constexpr int kDecodeMaxM = 1024;  // feature count the vector path stages in LDS

// Vector path: dv % 4 == 0, (dv / 4) divides 256, m <= kDecodeMaxM.
template <bool VBF16, bool GATED>
__global__ __launch_bounds__(256) void decode_state_vec(int m, int dv, const float* __restrict__ phiq,
                                                        const float* __restrict__ phik,
                                                        const void* __restrict__ v,
                                                        float* __restrict__ S, float* __restrict__ z,
                                                        float* __restrict__ out, int normalize,
                                                        float delta, const float* __restrict__ lg) {
  __shared__ float4 red4[256];
  __shared__ float red[4];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int CG = dv >> 2, RG = 256 / CG;
  const int cg = tid % CG, rg = tid / CG;
  const float* fq = phiq + bh * m;
  const float* fk = phik + bh * m;
  float* Sb = S + bh * static_cast<int64_t>(m) * dv;
  const float4 vv = load_v4<VBF16>(v, bh * dv + cg * 4);
  const float ga = GATED ? __expf(lg[bh]) : 1.f;  // state decay of this (batch, head)
  // phi_k and phi_q of this (batch, head) in LDS: the row loop then issues
  // only the state's vector loads and stores
  __shared__ float fks[kDecodeMaxM], fqs[kDecodeMaxM];
  for (int f = tid; f < m; f += 256) {
    fks[f] = fk[f];
    fqs[f] = fq[f];
  }
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto update = [&](f32x4& st, float kf, float qf) {
    if (GATED) st *= ga;
    st[0] = fmaf(kf, vv.x, st[0]);
    st[1] = fmaf(kf, vv.y, st[1]);
    st[2] = fmaf(kf, vv.z, st[2]);
    st[3] = fmaf(kf, vv.w, st[3]);
    acc.x = fmaf(qf, st[0], acc.x);
    acc.y = fmaf(qf, st[1], acc.y);
    acc.z = fmaf(qf, st[2], acc.z);
    acc.w = fmaf(qf, st[3], acc.w);
  };
  // Rows go in batches whose loads are all issued before the first store: in
  // a plain loop the compiler cannot move a row's load above the previous
  // row's store (it cannot prove they miss each other), so each thread would
  // keep one 16-byte load in flight. Batches of 32 rows (a thread's whole
  // share at m = 256, dv = 128) keep 512 bytes per thread in flight; smaller
  // batches take the rest. At 32 rows the kernel needs 256 VGPRs, one wave
  // per SIMD: fewer concurrent state streams measured faster than two waves
  // per SIMD with the same batch.
  int f = rg;
  auto batch = [&](auto u_c) {
    constexpr int U = decltype(u_c)::value;
    for (; f + (U - 1) * RG < m; f += U * RG) {
      f32x4* p[U];
      f32x4 st[U];
      float kf[U], qf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = reinterpret_cast<f32x4*>(Sb + static_cast<int64_t>(f + u * RG) * dv + cg * 4);
        st[u] = __builtin_nontemporal_load(p[u]);
        kf[u] = fks[f + u * RG];
        qf[u] = fqs[f + u * RG];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        update(st[u], kf[u], qf[u]);
        __builtin_nontemporal_store(st[u], p[u]);
      }
    }
  };
  batch(std::integral_constant<int, 32>{});
  batch(std::integral_constant<int, 8>{});
  batch(std::integral_constant<int, 1>{});
  red4[tid] = acc;
  // z update and the normaliser dot product
  float dpart = 0.f;
  for (int f = tid; f < m; f += 256) {
    const float zn = (GATED ? ga * z[bh * m + f] : z[bh * m + f]) + fk[f];
    z[bh * m + f] = zn;
    dpart = fmaf(fq[f], zn, dpart);
  }
  const float den = normalize ? block_sum(dpart, red) + delta : 1.f;  // has barriers
  __syncthreads();
  if (tid < CG) {
    float4 o = red4[tid];
    for (int r = 1; r < RG; ++r) {
      const float4 x = red4[r * CG + tid];
      o.x += x.x;
      o.y += x.y;
      o.z += x.z;
      o.w += x.w;
    }
    const float inv = normalize ? 1.f / den : 1.f;
    float* ob = out + bh * dv + tid * 4;
    ob[0] = o.x * inv;
    ob[1] = o.y * inv;
    ob[2] = o.z * inv;
    ob[3] = o.w * inv;
  }
}

// Generic path: any dv (one thread per column, rows split over 256/dv groups).
template <bool VBF16, bool GATED>
__global__ __launch_bounds__(256) void decode_state_gen(int m, int dv, const float* __restrict__ phiq,
                                                        const float* __restrict__ phik,
                                                        const void* __restrict__ v,
                                                        float* __restrict__ S, float* __restrict__ z,
                                                        float* __restrict__ out, int normalize,
                                                        float delta, const float* __restrict__ lg) {
  __shared__ float red[4];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const float* fq = phiq + bh * m;
  const float* fk = phik + bh * m;
  float* Sb = S + bh * static_cast<int64_t>(m) * dv;
  const float ga = GATED ? __expf(lg[bh]) : 1.f;
  float dpart = 0.f;
  for (int f = tid; f < m; f += 256) {
    const float zn = (GATED ? ga * z[bh * m + f] : z[bh * m + f]) + fk[f];
    z[bh * m + f] = zn;
    dpart = fmaf(fq[f], zn, dpart);
  }
  const float den = normalize ? block_sum(dpart, red) + delta : 1.f;
  for (int c = tid; c < dv; c += 256) {
    const float vc = load_v1<VBF16>(v, bh * dv + c);
    float acc = 0.f;
    for (int f = 0; f < m; ++f) {
      const float s0 = Sb[static_cast<int64_t>(f) * dv + c];
      const float s = fmaf(fk[f], vc, GATED ? ga * s0 : s0);
      Sb[static_cast<int64_t>(f) * dv + c] = s;
      acc = fmaf(fq[f], s, acc);
    }
    out[bh * dv + c] = normalize ? acc / den : acc;
  }
}


template <bool GATED>
hipError_t launch_decode_t(int64_t BH, int m, int dv, const float* phiq, const float* phik,
                           const void* v, int v_bf16, float* S, float* z, float* out,
                           int normalize, float delta, const float* lg, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(BH));
  const bool vec = (dv % 4 == 0) && (dv / 4 <= 256) && (256 % (dv / 4) == 0) && m <= kDecodeMaxM;
  if (vec) {
    if (v_bf16)
      LLOPS_LAUNCH("decode_state", st, (decode_state_vec<true, GATED>), grid, dim3(256), 0, st, m, dv,
                   phiq, phik, v, S, z, out, normalize, delta, lg);
    else
      LLOPS_LAUNCH("decode_state", st, (decode_state_vec<false, GATED>), grid, dim3(256), 0, st, m,
                   dv, phiq, phik, v, S, z, out, normalize, delta, lg);
  } else {
    if (v_bf16)
      LLOPS_LAUNCH("decode_state", st, (decode_state_gen<true, GATED>), grid, dim3(256), 0, st, m, dv,
                   phiq, phik, v, S, z, out, normalize, delta, lg);
    else
      LLOPS_LAUNCH("decode_state", st, (decode_state_gen<false, GATED>), grid, dim3(256), 0, st, m,
                   dv, phiq, phik, v, S, z, out, normalize, delta, lg);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_state(int64_t BH, int m, int dv, const float* phiq, const float* phik,
                               const void* v, int v_bf16, float* S, float* z, float* out,
                               int normalize, float delta, const float* log_gate, hipStream_t st) {
  if (BH <= 0) return hipSuccess;
  if (BH > 0x7fffffffLL) return hipErrorInvalidValue;
  if (log_gate)
    return launch_decode_t<true>(BH, m, dv, phiq, phik, v, v_bf16, S, z, out, normalize, delta,
                                 log_gate, st);
  return launch_decode_t<false>(BH, m, dv, phiq, phik, v, v_bf16, S, z, out, normalize, delta,
                                nullptr, st);
}

}  // namespace llops
