// Per-token absmax INT8 activation quantization, alone or after a parameter-free LayerNorm.
//
// "Microsoft BitNet 1.58: The Era of 1-Bit Large Language Models", section "The BitLinear
// Layer", operation 2 (BF16 -> INT8 by absmax scaling, scale kept for dequantization); "BitNet
// b1.58: How Ternary Weights Cut LLM Memory by 82% Without Losing Accuracy", section "How ternary
// quantization works during training" (per-token scale).
//
//   a'_t = max(max_k |x[t,k]|, 1e-5)          (exact: a maximum of bf16 magnitudes)
//   s_t  = fl32(127 / a'_t)                    (correctly rounded fp32 division)
//   q    = clamp(rne(fl32(x * s_t)), -127, 127)
//
// HBM-bound: 2 bytes read + 1 byte written per element. Each row is held in registers between
// the max pass and the quantize pass, so it is read from memory once. The max is taken on the
// bf16 bit patterns with the sign cleared (order-preserving for finite values), two per 32-bit
// lane op.
#include "sbn_internal.hpp"

namespace sbn {
namespace {

template <int TPR>
__device__ __forceinline__ uint32_t row_max(uint32_t v, uint32_t* red) {
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  if constexpr (TPR > 64) {
    const int wave = threadIdx.x >> 6, nw = TPR / 64;
    const int first = (threadIdx.x / TPR) * nw;  // first wave of this row
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    uint32_t r = 0;
    for (int i = 0; i < nw; ++i) r = max(r, red[first + i]);
    v = r;
  }
  return v;
}

// Vector path: x rows 16-byte aligned, K % 8 == 0, q rows 8-byte aligned.
template <int TPR, int VPT>
__global__ __launch_bounds__(256) void quantize_act_vec(const uint16_t* __restrict__ x, int64_t T,
                                                        int64_t K, int64_t ld_x,
                                                        int8_t* __restrict__ q, int64_t ld_q,
                                                        float* __restrict__ absmax) {
  constexpr int kRowsPerBlock = 256 / TPR;
  __shared__ uint32_t red[4];
  const int lt = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / TPR;
  const bool active = row < T;
  const int64_t nvec = K >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (active ? row : 0) * ld_x);
  uint4 v[VPT];
  uint32_t m2 = 0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t vi = lt + (int64_t)i * TPR;
    v[i] = (active && vi < nvec) ? xr[vi] : make_uint4(0, 0, 0, 0);
    m2 = max_abs_bf16x2(m2, v[i].x);
    m2 = max_abs_bf16x2(m2, v[i].y);
    m2 = max_abs_bf16x2(m2, v[i].z);
    m2 = max_abs_bf16x2(m2, v[i].w);
  }
  uint32_t mb = max(m2 & 0xFFFFu, m2 >> 16);
  mb = row_max<TPR>(mb, red);
  const float a = fmaxf(__uint_as_float(mb << 16), kAbsmaxFloor);
  const float s = 127.0f / a;
  if (!active) return;
  uint2* qr = reinterpret_cast<uint2*>(q + row * ld_q);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t vi = lt + (int64_t)i * TPR;
    if (vi < nvec) qr[vi] = make_uint2(quant4(v[i].x, v[i].y, s), quant4(v[i].z, v[i].w, s));
  }
  if (lt == 0) absmax[row] = a;
}

// General path: any alignment and K; the row is read twice (the second read hits cache).
__global__ __launch_bounds__(256) void quantize_act_any(const uint16_t* __restrict__ x, int64_t T,
                                                        int64_t K, int64_t ld_x,
                                                        int8_t* __restrict__ q, int64_t ld_q,
                                                        float* __restrict__ absmax) {
  __shared__ uint32_t red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * ld_x;
  uint32_t mb = 0;
  for (int64_t k = threadIdx.x; k < K; k += 256) mb = max(mb, (uint32_t)(xr[k] & 0x7FFFu));
  mb = row_max<256>(mb, red);
  const float a = fmaxf(__uint_as_float(mb << 16), kAbsmaxFloor);
  const float s = 127.0f / a;
  int8_t* qr = q + row * ld_q;
  for (int64_t k = threadIdx.x; k < K; k += 256) {
    const float f = __uint_as_float((uint32_t)xr[k] << 16);
    qr[k] = (int8_t)(int)__builtin_amdgcn_fmed3f(__builtin_rintf(f * s), -127.f, 127.f);
  }
  if (threadIdx.x == 0) absmax[row] = a;
}

// ---- Parameter-free LayerNorm in front of the quantizer ("The BitLinear Layer", operation 1) ----
//
//   mu = fl64(sum_k x / K),  var = fl64(sum_k (x - mu)^2 / K),  r = fl64(1 / sqrt(var + eps))
//   z  = bf16( fl32( fl32(x - fl32(mu)) * fl32(r) ) )     (round to nearest even)
// followed by the absmax quantization of z above. The statistics are fp64 (the sum of bf16 values
// is exact, so the mean does not depend on the summation order); the normalization is fp32 and
// its result is rounded to bf16, the type the quantizer takes.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ double pair_sum(uint32_t w) {
  return (double)bf16_lo(w) + (double)bf16_hi(w);
}

__device__ __forceinline__ double pair_dev2(uint32_t w, double mu) {
  const double d0 = (double)bf16_lo(w) - mu, d1 = (double)bf16_hi(w) - mu;
  return d0 * d0 + d1 * d1;
}

// Sum over the TPR threads of a row (xor butterfly: every lane ends with the same value), then
// over its waves in a fixed order.
template <int TPR>
__device__ __forceinline__ double row_sum(double v, double* red) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if constexpr (TPR > 64) {
    const int wave = threadIdx.x >> 6, nw = TPR / 64;
    const int first = (threadIdx.x / TPR) * nw;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    double r = 0.0;
    for (int i = 0; i < nw; ++i) r += red[first + i];
    v = r;
  }
  return v;
}

template <int TPR, int VPT>
__global__ __launch_bounds__(256) void ln_quantize_act_vec(const uint16_t* __restrict__ x,
                                                           int64_t T, int64_t K, int64_t ld_x,
                                                           float eps, int8_t* __restrict__ q,
                                                           int64_t ld_q,
                                                           float* __restrict__ absmax) {
  constexpr int kRowsPerBlock = 256 / TPR;
  __shared__ double red_s[4], red_d[4];
  __shared__ uint32_t red_m[4];
  const int lt = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / TPR;
  const bool active = row < T;
  const int64_t nvec = K >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (active ? row : 0) * ld_x);
  uint4 v[VPT];
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t vi = lt + (int64_t)i * TPR;
    v[i] = (active && vi < nvec) ? xr[vi] : make_uint4(0, 0, 0, 0);
    s += pair_sum(v[i].x) + pair_sum(v[i].y) + pair_sum(v[i].z) + pair_sum(v[i].w);
  }
  const double mu = row_sum<TPR>(s, red_s) / (double)K;
  double d = 0.0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    if (lt + (int64_t)i * TPR < nvec)
      d += pair_dev2(v[i].x, mu) + pair_dev2(v[i].y, mu) + pair_dev2(v[i].z, mu) +
           pair_dev2(v[i].w, mu);
  }
  const double var = row_sum<TPR>(d, red_d) / (double)K;
  const float mu32 = (float)mu, r32 = (float)(1.0 / sqrt(var + (double)eps));
  uint32_t m2 = 0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    if (lt + (int64_t)i * TPR < nvec) {
      v[i] = make_uint4(ln_pair(v[i].x, mu32, r32), ln_pair(v[i].y, mu32, r32),
                        ln_pair(v[i].z, mu32, r32), ln_pair(v[i].w, mu32, r32));
    }
    m2 = max_abs_bf16x2(m2, v[i].x);
    m2 = max_abs_bf16x2(m2, v[i].y);
    m2 = max_abs_bf16x2(m2, v[i].z);
    m2 = max_abs_bf16x2(m2, v[i].w);
  }
  uint32_t mb = max(m2 & 0xFFFFu, m2 >> 16);
  mb = row_max<TPR>(mb, red_m);
  const float a = fmaxf(__uint_as_float(mb << 16), kAbsmaxFloor);
  const float sc = 127.0f / a;
  if (!active) return;
  uint2* qr = reinterpret_cast<uint2*>(q + row * ld_q);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t vi = lt + (int64_t)i * TPR;
    if (vi < nvec) qr[vi] = make_uint2(quant4(v[i].x, v[i].y, sc), quant4(v[i].z, v[i].w, sc));
  }
  if (lt == 0) absmax[row] = a;
}

// General path (any alignment and K): one row per workgroup; the row is read four times (the
// later reads hit cache).
__global__ __launch_bounds__(256) void ln_quantize_act_any(const uint16_t* __restrict__ x,
                                                           int64_t T, int64_t K, int64_t ld_x,
                                                           float eps, int8_t* __restrict__ q,
                                                           int64_t ld_q,
                                                           float* __restrict__ absmax) {
  __shared__ double red_s[4], red_d[4];
  __shared__ uint32_t red_m[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * ld_x;
  double s = 0.0;
  for (int64_t k = threadIdx.x; k < K; k += 256) s += (double)bf16_lo(xr[k]);
  const double mu = row_sum<256>(s, red_s) / (double)K;
  double d = 0.0;
  for (int64_t k = threadIdx.x; k < K; k += 256) {
    const double e = (double)bf16_lo(xr[k]) - mu;
    d += e * e;
  }
  const double var = row_sum<256>(d, red_d) / (double)K;
  const float mu32 = (float)mu, r32 = (float)(1.0 / sqrt(var + (double)eps));
  auto z_of = [&](int64_t k) {
    return bf16_rne(__fmul_rn(__fsub_rn(bf16_lo(xr[k]), mu32), r32));
  };
  uint32_t mb = 0;
  for (int64_t k = threadIdx.x; k < K; k += 256) mb = max(mb, z_of(k) & 0x7FFFu);
  mb = row_max<256>(mb, red_m);
  const float a = fmaxf(__uint_as_float(mb << 16), kAbsmaxFloor);
  const float sc = 127.0f / a;
  int8_t* qr = q + row * ld_q;
  for (int64_t k = threadIdx.x; k < K; k += 256) {
    const float f = bf16_lo(z_of(k));
    qr[k] = (int8_t)(int)__builtin_amdgcn_fmed3f(__builtin_rintf(f * sc), -127.f, 127.f);
  }
  if (threadIdx.x == 0) absmax[row] = a;
}

template <int TPR, int VPT>
hipError_t launch_vec(const uint16_t* x, int64_t T, int64_t K, int64_t ld_x, int8_t* q,
                      int64_t ld_q, float* absmax, hipStream_t s) {
  constexpr int rpb = 256 / TPR;
  const int64_t blocks = (T + rpb - 1) / rpb;
  hipLaunchKernelGGL((quantize_act_vec<TPR, VPT>), dim3((unsigned)blocks), dim3(256), 0, s, x, T,
                     K, ld_x, q, ld_q, absmax);
  return hipGetLastError();
}

template <int TPR>
hipError_t dispatch_vpt(int vpt, const uint16_t* x, int64_t T, int64_t K, int64_t ld_x,
                        int8_t* q, int64_t ld_q, float* absmax, hipStream_t s) {
  switch (vpt) {
    case 1: return launch_vec<TPR, 1>(x, T, K, ld_x, q, ld_q, absmax, s);
    case 2: return launch_vec<TPR, 2>(x, T, K, ld_x, q, ld_q, absmax, s);
    case 3: return launch_vec<TPR, 3>(x, T, K, ld_x, q, ld_q, absmax, s);
    case 4: return launch_vec<TPR, 4>(x, T, K, ld_x, q, ld_q, absmax, s);
    case 5: return launch_vec<TPR, 5>(x, T, K, ld_x, q, ld_q, absmax, s);
    case 6: return launch_vec<TPR, 6>(x, T, K, ld_x, q, ld_q, absmax, s);
    case 7: return launch_vec<TPR, 7>(x, T, K, ld_x, q, ld_q, absmax, s);
    default: return launch_vec<TPR, 8>(x, T, K, ld_x, q, ld_q, absmax, s);
  }
}

template <int TPR, int VPT>
hipError_t launch_ln_vec(const uint16_t* x, int64_t T, int64_t K, int64_t ld_x, float eps,
                         int8_t* q, int64_t ld_q, float* absmax, hipStream_t s) {
  constexpr int rpb = 256 / TPR;
  const int64_t blocks = (T + rpb - 1) / rpb;
  hipLaunchKernelGGL((ln_quantize_act_vec<TPR, VPT>), dim3((unsigned)blocks), dim3(256), 0, s, x,
                     T, K, ld_x, eps, q, ld_q, absmax);
  return hipGetLastError();
}

template <int TPR>
hipError_t dispatch_ln_vpt(int vpt, const uint16_t* x, int64_t T, int64_t K, int64_t ld_x,
                           float eps, int8_t* q, int64_t ld_q, float* absmax, hipStream_t s) {
  switch (vpt) {
    case 1: return launch_ln_vec<TPR, 1>(x, T, K, ld_x, eps, q, ld_q, absmax, s);
    case 2: return launch_ln_vec<TPR, 2>(x, T, K, ld_x, eps, q, ld_q, absmax, s);
    case 3: return launch_ln_vec<TPR, 3>(x, T, K, ld_x, eps, q, ld_q, absmax, s);
    case 4: return launch_ln_vec<TPR, 4>(x, T, K, ld_x, eps, q, ld_q, absmax, s);
    case 5: return launch_ln_vec<TPR, 5>(x, T, K, ld_x, eps, q, ld_q, absmax, s);
    case 6: return launch_ln_vec<TPR, 6>(x, T, K, ld_x, eps, q, ld_q, absmax, s);
    case 7: return launch_ln_vec<TPR, 7>(x, T, K, ld_x, eps, q, ld_q, absmax, s);
    default: return launch_ln_vec<TPR, 8>(x, T, K, ld_x, eps, q, ld_q, absmax, s);
  }
}

}  // namespace

hipError_t launch_ln_quantize_act(const uint16_t* x, int64_t T, int64_t K, int64_t ld_x,
                                  float eps, int8_t* q, int64_t ld_q, float* absmax,
                                  hipStream_t s) {
  const bool aligned = ((uintptr_t)x % 16 == 0) && (ld_x % 8 == 0) && (K % 8 == 0) &&
                       ((uintptr_t)q % 8 == 0) && (ld_q % 8 == 0);
  const int64_t nvec = K / 8;
  if (aligned && nvec <= 64 * 8) {
    return dispatch_ln_vpt<64>((int)((nvec + 63) / 64), x, T, K, ld_x, eps, q, ld_q, absmax, s);
  }
  if (aligned && nvec <= 256 * 8) {
    return dispatch_ln_vpt<256>((int)((nvec + 255) / 256), x, T, K, ld_x, eps, q, ld_q, absmax,
                                s);
  }
  hipLaunchKernelGGL(ln_quantize_act_any, dim3((unsigned)T), dim3(256), 0, s, x, T, K, ld_x, eps,
                     q, ld_q, absmax);
  return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t* x, int64_t T, int64_t K, int64_t ld_x, int8_t* q,
                               int64_t ld_q, float* absmax, hipStream_t s) {
  const bool aligned = ((uintptr_t)x % 16 == 0) && (ld_x % 8 == 0) && (K % 8 == 0) &&
                       ((uintptr_t)q % 8 == 0) && (ld_q % 8 == 0);
  const int64_t nvec = K / 8;
  if (aligned && nvec <= 64 * 8) {
    return dispatch_vpt<64>((int)((nvec + 63) / 64), x, T, K, ld_x, q, ld_q, absmax, s);
  }
  if (aligned && nvec <= 256 * 8) {
    return dispatch_vpt<256>((int)((nvec + 255) / 256), x, T, K, ld_x, q, ld_q, absmax, s);
  }
  hipLaunchKernelGGL(quantize_act_any, dim3((unsigned)T), dim3(256), 0, s, x, T, K, ld_x, q,
                     ld_q, absmax);
  return hipGetLastError();
}

}  // namespace sbn
