// Measured ceilings of the GPU: a streaming read, loops of dense and structured-sparse INT8 MFMA
// instructions and an empty kernel, so that the library's rates can be reported against what this chip delivers beside its
// published peaks. Declared in include/sbn_ceilings.h.
#include "sbn_ceilings.h"
#include "sbn_internal.hpp"

namespace sbn {
namespace {

constexpr int kReadThreads = 256;

// Each lane reads 16 bytes per load, four loads in flight per step, grid-strided; the XOR of what
// it read is stored only if it equals the sentinel.
__global__ __launch_bounds__(kReadThreads) void ceiling_read(const uint4* __restrict__ p,
                                                             uint64_t n16, uint32_t sentinel,
                                                             uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kReadThreads;
  uint64_t i = (uint64_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == sentinel) sink[0] = acc;
}

typedef int v4i_t __attribute__((ext_vector_type(4)));

// Eight independent accumulator chains per wave, so the matrix core never waits on a result.
__global__ __launch_bounds__(256) void ceiling_mfma(int iters, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const v4i_t a = {lane, lane * 3, lane * 5, lane * 7};
  const v4i_t b = {lane * 11, lane * 13, lane * 17, lane * 19};
  // eight separate accumulators, each updated in place (with the builtin the compiler gave each
  // instruction a new destination and copied it back, an extra register move per product)
  v4i_t c0 = {0, 0, 0, 0}, c1 = {1, 0, 0, 0}, c2 = {2, 0, 0, 0}, c3 = {3, 0, 0, 0};
  v4i_t c4 = {4, 0, 0, 0}, c5 = {5, 0, 0, 0}, c6 = {6, 0, 0, 0}, c7 = {7, 0, 0, 0};
  for (int i = 0; i < iters; ++i) {
    asm volatile(
        "v_mfma_i32_16x16x64_i8 %0, %8, %9, %0\n\t"
        "v_mfma_i32_16x16x64_i8 %1, %8, %9, %1\n\t"
        "v_mfma_i32_16x16x64_i8 %2, %8, %9, %2\n\t"
        "v_mfma_i32_16x16x64_i8 %3, %8, %9, %3\n\t"
        "v_mfma_i32_16x16x64_i8 %4, %8, %9, %4\n\t"
        "v_mfma_i32_16x16x64_i8 %5, %8, %9, %5\n\t"
        "v_mfma_i32_16x16x64_i8 %6, %8, %9, %6\n\t"
        "v_mfma_i32_16x16x64_i8 %7, %8, %9, %7"
        : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7)
        : "v"(a), "v"(b));
  }
  const v4i_t x = c0 ^ c1 ^ c2 ^ c3 ^ c4 ^ c5 ^ c6 ^ c7;
  const int s = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (s == 0x7FFFFFFF && threadIdx.x == 0) sink[0] = (uint32_t)s;
}

typedef int v8i_t __attribute__((ext_vector_type(8)));

// The same loop on the structured-sparse instruction (2:4 kept weights of 128 K per row in the A
// operand, a 2-bit position index per kept weight): 16 x 16 x 128 dense-equivalent products each.
__global__ __launch_bounds__(256) void ceiling_smfmac(int iters, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const v4i_t a = {lane, lane * 3, lane * 5, lane * 7};
  const v8i_t b = {lane * 11, lane * 13, lane * 17, lane * 19, lane * 23, lane * 29, lane * 31,
                   lane * 37};
  const int idx = (int)0xE4E4E4E4u;  // positions 0, 1, 2, 3 ... of each group of 4 (valid pairs)
  v4i_t c0 = {0, 0, 0, 0}, c1 = {1, 0, 0, 0}, c2 = {2, 0, 0, 0}, c3 = {3, 0, 0, 0};
  v4i_t c4 = {4, 0, 0, 0}, c5 = {5, 0, 0, 0}, c6 = {6, 0, 0, 0}, c7 = {7, 0, 0, 0};
  for (int i = 0; i < iters; ++i) {
    asm volatile(
        "v_smfmac_i32_16x16x128_i8 %0, %8, %9, %10\n\t"
        "v_smfmac_i32_16x16x128_i8 %1, %8, %9, %10\n\t"
        "v_smfmac_i32_16x16x128_i8 %2, %8, %9, %10\n\t"
        "v_smfmac_i32_16x16x128_i8 %3, %8, %9, %10\n\t"
        "v_smfmac_i32_16x16x128_i8 %4, %8, %9, %10\n\t"
        "v_smfmac_i32_16x16x128_i8 %5, %8, %9, %10\n\t"
        "v_smfmac_i32_16x16x128_i8 %6, %8, %9, %10\n\t"
        "v_smfmac_i32_16x16x128_i8 %7, %8, %9, %10"
        : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
        : "v"(a), "v"(b), "v"(idx));
  }
  const v4i_t x = c0 ^ c1 ^ c2 ^ c3 ^ c4 ^ c5 ^ c6 ^ c7;
  const int s = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (s == 0x7FFFFFFF && threadIdx.x == 0) sink[0] = (uint32_t)s;
}

__global__ void ceiling_empty() {}

}  // namespace
}  // namespace sbn

extern "C" {

sbn_status sbn_ceiling_stream_read(const void* buf, size_t bytes, uint32_t sentinel,
                                   uint32_t* sink, void* stream) {
  if (!buf || !sink) return sbn::set_error(SBN_ERR_INVALID_ARG, "sbn_ceiling_stream_read: null pointer");
  if (bytes < 16 || bytes > ((size_t)1 << 40) || bytes % 16 != 0 || (uintptr_t)buf % 16 != 0)
    return sbn::set_error(SBN_ERR_INVALID_ARG,
                          "sbn_ceiling_stream_read: bytes=%zu must be a multiple of 16 in "
                          "[16, 2^40] on a 16-byte aligned buffer", bytes);
  // eight workgroups per CU of the 256, enough loads in flight to cover the HBM latency
  const unsigned blocks = 2048;
  hipLaunchKernelGGL(sbn::ceiling_read, dim3(blocks), dim3(sbn::kReadThreads), 0,
                     (hipStream_t)stream, static_cast<const uint4*>(buf), (uint64_t)(bytes / 16),
                     sentinel, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return sbn::set_error(SBN_ERR_HIP, "sbn_ceiling_stream_read launch: %s", hipGetErrorString(e));
  return SBN_OK;
}

sbn_status sbn_ceiling_mfma_i8(int64_t iters, int64_t waves, uint32_t* sink, double* ops,
                               void* stream) {
  if (!sink || !ops) return sbn::set_error(SBN_ERR_INVALID_ARG, "sbn_ceiling_mfma_i8: null pointer");
  if (iters < 1 || iters > (1 << 24) || waves < 4 || waves > (1 << 20) || waves % 4 != 0)
    return sbn::set_error(SBN_ERR_INVALID_ARG, "sbn_ceiling_mfma_i8: iters=%lld waves=%lld",
                          (long long)iters, (long long)waves);
  hipLaunchKernelGGL(sbn::ceiling_mfma, dim3((unsigned)(waves / 4)), dim3(256), 0,
                     (hipStream_t)stream, (int)iters, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return sbn::set_error(SBN_ERR_HIP, "sbn_ceiling_mfma_i8 launch: %s", hipGetErrorString(e));
  *ops = (double)waves * (double)iters * 8.0 * 32768.0;
  return SBN_OK;
}

sbn_status sbn_ceiling_smfmac_i8(int64_t iters, int64_t waves, uint32_t* sink, double* ops,
                                 void* stream) {
  if (!sink || !ops)
    return sbn::set_error(SBN_ERR_INVALID_ARG, "sbn_ceiling_smfmac_i8: null pointer");
  if (iters < 1 || iters > (1 << 24) || waves < 4 || waves > (1 << 20) || waves % 4 != 0)
    return sbn::set_error(SBN_ERR_INVALID_ARG, "sbn_ceiling_smfmac_i8: iters=%lld waves=%lld",
                          (long long)iters, (long long)waves);
  hipLaunchKernelGGL(sbn::ceiling_smfmac, dim3((unsigned)(waves / 4)), dim3(256), 0,
                     (hipStream_t)stream, (int)iters, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return sbn::set_error(SBN_ERR_HIP, "sbn_ceiling_smfmac_i8 launch: %s", hipGetErrorString(e));
  *ops = (double)waves * (double)iters * 8.0 * 65536.0;
  return SBN_OK;
}

sbn_status sbn_ceiling_empty(void* stream) {
  hipLaunchKernelGGL(sbn::ceiling_empty, dim3(1), dim3(64), 0, (hipStream_t)stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return sbn::set_error(SBN_ERR_HIP, "sbn_ceiling_empty launch: %s", hipGetErrorString(e));
  return SBN_OK;
}

}  // extern "C"
