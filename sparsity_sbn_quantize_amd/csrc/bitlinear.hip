// n:m-sparse ternary x INT8 matmul with int32 accumulation and fused dequantization.
//
// "Microsoft BitNet 1.58: The Era of 1-Bit Large Language Models", section "The BitLinear
// Layer", operations 4 (matmul of ternary weights and INT8 activations on quantized values) and 5
// (dequantize with the preserved scales); section "bitnet.cpp: Matrix-Free Inference" (2-bit
// packed weights streamed and unpacked on chip, integer dot products).
//
//   acc[t][r] = sum_k q[t][k] * code[r][k]                          (exact int32)
//   y[t][r]   = fl32( fl32( fl32(acc) * gamma ) * fl32(a'_t / 127) )
//
// Each lane decodes one brick (64 K positions of one weight row) from its packed mask + codes
// straight into the A operand of v_mfma_i32_16x16x64_i8: the brick's bytes [16j, 16j+16) feed
// MFMA j of the 256-K fragment. The B operand (activations) uses the same K assignment, so the
// products pair correctly whatever the instruction's internal K order. Decode is a lookup per
// 4 positions in a 4096-entry nibble table held in LDS (index: mask nibble, next 8 code bits).
//
//   GEMV (T <= 16): one workgroup per 16-row fragment row, its 4 waves split K; activations are
//   read straight from global memory (they are tiny and cache-resident).
//   GEMM (T > 16): a workgroup computes 256 rows x 128 tokens; the 128 x 256 activation tile of
//   each K step is staged in LDS and shared by the 4 waves, each wave owning 64 weight rows.
#include "sbn_internal.hpp"

namespace sbn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ const NibbleTable g_nibble_table = make_nibble_table();

__device__ __forceinline__ v4i mfma16(const uint32_t* a, v4i b, v4i c) {
  const v4i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3]};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, c, 0, 0, 0);
}

__device__ __forceinline__ void load_lut(uint32_t* lut) {
  const uint4* src = reinterpret_cast<const uint4*>(g_nibble_table.v);
  uint4* dst = reinterpret_cast<uint4*>(lut);
  for (int i = threadIdx.x; i < 1024; i += blockDim.x) dst[i] = src[i];
}

// Loads one brick's mask (8 bytes) and code bytes. CBB > 0: compile-time code bytes per brick.
template <int CBB>
__device__ __forceinline__ void load_brick(const Layout& L, const uint8_t* __restrict__ mask_plane,
                                           const uint8_t* __restrict__ code_plane, int64_t slot,
                                           uint32_t mask[2], uint32_t codes[4]) {
  mask[0] = mask[1] = 0;
  if (L.has_mask) {
    const uint2 m = *reinterpret_cast<const uint2*>(mask_plane + slot * 8);
    mask[0] = m.x;
    mask[1] = m.y;
  }
  codes[0] = codes[1] = codes[2] = codes[3] = 0;
  if constexpr (CBB == 16) {
    const uint4 c = *reinterpret_cast<const uint4*>(code_plane + slot * 16);
    codes[0] = c.x; codes[1] = c.y; codes[2] = c.z; codes[3] = c.w;
  } else if constexpr (CBB == 12) {
    const uint32_t* c = reinterpret_cast<const uint32_t*>(code_plane + slot * 12);
    codes[0] = c[0]; codes[1] = c[1]; codes[2] = c[2];
  } else if constexpr (CBB == 8) {
    const uint2 c = *reinterpret_cast<const uint2*>(code_plane + slot * 8);
    codes[0] = c.x; codes[1] = c.y;
  } else if constexpr (CBB == 4) {
    codes[0] = *reinterpret_cast<const uint32_t*>(code_plane + slot * 4);
  } else {
    const int cbb = L.code_brick_bytes;
    const uint8_t* c = code_plane + slot * cbb;
    for (int i = 0; i < cbb; ++i) codes[i >> 2] |= (uint32_t)c[i] << (8 * (i & 3));
  }
}

template <int N, int M>
__device__ __forceinline__ void decode(const Layout& L, const uint32_t* lut, const uint32_t mask[2],
                                       const uint32_t codes[4], uint32_t out[16]) {
  if constexpr (N > 0) {
    decode_brick_lut<N, M>(lut, mask, codes, out);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = 0;
    decode_brick_plain(mask, codes, L.n, L.m, L.has_mask, out);
  }
}

// 16 activation bytes of one token row at K offset k (zero beyond K).
__device__ __forceinline__ v4i load_x16(const int8_t* __restrict__ row, int64_t k, int64_t K,
                                        int vec) {
  if (vec && k + 16 <= K) return *reinterpret_cast<const v4i*>(row + k);
  uint32_t w[4] = {0, 0, 0, 0};
  for (int i = 0; i < 16; ++i) {
    if (k + i < K) w[i >> 2] |= (uint32_t)(uint8_t)row[k + i] << (8 * (i & 3));
  }
  return v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}

__device__ __forceinline__ void store_out(void* y, int64_t ld_y, int out_kind, int64_t t,
                                          int64_t r, int acc, float gamma, float step) {
  if (out_kind == SBN_OUT_I32_ACC) {
    reinterpret_cast<int32_t*>(y)[t * ld_y + r] = acc;
  } else {
    const float v = __fmul_rn(__fmul_rn((float)acc, gamma), step);
    reinterpret_cast<float*>(y)[t * ld_y + r] = v;
  }
}

template <int N, int M, int CBB>
__global__ __launch_bounds__(256) void bitlinear_gemv(
    const uint8_t* __restrict__ mask_plane, const uint8_t* __restrict__ code_plane, Layout L,
    const float* __restrict__ gamma_p, const int8_t* __restrict__ xq, int64_t ld_q, int xq_vec,
    const float* __restrict__ absmax, int64_t T, void* __restrict__ y, int64_t ld_y,
    int out_kind) {
  __shared__ uint32_t lut[N > 0 ? 4096 : 1];
  __shared__ v4i red[3][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rb = blockIdx.x;
  if constexpr (N > 0) {
    load_lut(lut);
    __syncthreads();
  }
  const int t = lane & 15, g = lane >> 4;
  const bool tok_ok = t < T;
  const int8_t* xrow = xq + (tok_ok ? t : 0) * ld_q;
  v4i acc = {0, 0, 0, 0};
  for (int64_t q = wave; q < L.quads; q += 4) {
    const int64_t slot = ((rb * L.quads + q) << 6) | lane;
    uint32_t mask[2], codes[4], a[16];
    load_brick<CBB>(L, mask_plane, code_plane, slot, mask, codes);
    const int64_t kb = (q * 4 + g) * kBrickK;
    v4i b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = tok_ok ? load_x16(xrow, kb + 16 * j, L.K, xq_vec) : v4i{0, 0, 0, 0};
    decode<N, M>(L, lut, mask, codes, a);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma16(a + 4 * j, b[j], acc);
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  acc += red[0][lane] + red[1][lane] + red[2][lane];
  if (!tok_ok) return;
  const float gamma = gamma_p[0];
  const float step = out_kind == SBN_OUT_F32 ? absmax[t] / 127.0f : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = rb * 16 + 4 * g + i;
    if (r < L.n_out) store_out(y, ld_y, out_kind, t, r, acc[i], gamma, step);
  }
}

constexpr int kRF = 4;    // 16-row fragments per wave
constexpr int kCF = 8;    // 16-token fragments per workgroup
constexpr int kXStride = 272;  // bytes per staged token row (256 + 16 to spread LDS banks)

template <int N, int M, int CBB>
__global__ __launch_bounds__(256) void bitlinear_gemm(
    const uint8_t* __restrict__ mask_plane, const uint8_t* __restrict__ code_plane, Layout L,
    const float* __restrict__ gamma_p, const int8_t* __restrict__ xq, int64_t ld_q, int xq_vec,
    const float* __restrict__ absmax, int64_t T, void* __restrict__ y, int64_t ld_y,
    int out_kind) {
  __shared__ uint32_t lut[N > 0 ? 4096 : 1];
  __shared__ __attribute__((aligned(16))) int8_t xs[kCF * 16 * kXStride];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rb0 = ((int64_t)blockIdx.x * 4 + wave) * kRF;  // this wave's first row fragment
  const int64_t t0 = (int64_t)blockIdx.y * kCF * 16;
  if constexpr (N > 0) load_lut(lut);
  v4i acc[kRF][kCF];
#pragma unroll
  for (int rf = 0; rf < kRF; ++rf)
#pragma unroll
    for (int cf = 0; cf < kCF; ++cf) acc[rf][cf] = v4i{0, 0, 0, 0};

  for (int64_t q = 0; q < L.quads; ++q) {
    // Stage the activation tile: tokens t0 + [0, 128), K = q*256 + [0, 256).
    for (int c = threadIdx.x; c < kCF * 16 * 16; c += 256) {
      const int tok = c >> 4, ch = c & 15;
      const int64_t tt = t0 + tok;
      v4i v = {0, 0, 0, 0};
      if (tt < T) v = load_x16(xq + tt * ld_q, q * kQuadK + ch * 16, L.K, xq_vec);
      *reinterpret_cast<v4i*>(xs + tok * kXStride + ch * 16) = v;
    }
    __syncthreads();
    uint32_t a[kRF][16];
#pragma unroll
    for (int rf = 0; rf < kRF; ++rf) {
      const int64_t rb = rb0 + rf;
      if (rb < L.row_blocks) {
        uint32_t mask[2], codes[4];
        load_brick<CBB>(L, mask_plane, code_plane, ((rb * L.quads + q) << 6) | lane, mask, codes);
        decode<N, M>(L, lut, mask, codes, a[rf]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) a[rf][i] = 0;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int cf = 0; cf < kCF; ++cf) {
        const v4i b = *reinterpret_cast<const v4i*>(xs + (cf * 16 + (lane & 15)) * kXStride +
                                                    (lane >> 4) * kBrickK + 16 * j);
#pragma unroll
        for (int rf = 0; rf < kRF; ++rf) acc[rf][cf] = mfma16(a[rf] + 4 * j, b, acc[rf][cf]);
      }
    }
    __syncthreads();
  }
  const float gamma = gamma_p[0];
  const int g = lane >> 4;
#pragma unroll
  for (int cf = 0; cf < kCF; ++cf) {
    const int64_t t = t0 + cf * 16 + (lane & 15);
    if (t >= T) continue;
    const float step = out_kind == SBN_OUT_F32 ? absmax[t] / 127.0f : 0.0f;
#pragma unroll
    for (int rf = 0; rf < kRF; ++rf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = (rb0 + rf) * 16 + 4 * g + i;
        if (r < L.n_out) store_out(y, ld_y, out_kind, t, r, acc[rf][cf][i], gamma, step);
      }
    }
  }
}

template <int N, int M, int CBB>
hipError_t launch_pattern(const sbn_packed* h, const int8_t* xq, int64_t ld_q, int xq_vec,
                          const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                          hipStream_t s) {
  const Layout& L = h->L;
  if (T <= 16) {
    hipLaunchKernelGGL((bitlinear_gemv<N, M, CBB>), dim3((unsigned)L.row_blocks), dim3(256), 0, s,
                       h->mask, h->codes, L, h->gamma, xq, ld_q, xq_vec, absmax, T, y, ld_y,
                       out_kind);
  } else {
    const int64_t gx = (L.row_blocks + 4 * kRF - 1) / (4 * kRF);
    const int64_t gy = (T + kCF * 16 - 1) / (kCF * 16);
    hipLaunchKernelGGL((bitlinear_gemm<N, M, CBB>), dim3((unsigned)gx, (unsigned)gy), dim3(256),
                       0, s, h->mask, h->codes, L, h->gamma, xq, ld_q, xq_vec, absmax, T, y,
                       ld_y, out_kind);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bitlinear(const sbn_packed* h, const int8_t* xq, int64_t ld_q,
                            const float* absmax, int64_t T, void* y, int64_t ld_y, int out_kind,
                            hipStream_t s) {
  const Layout& L = h->L;
  if (L.n_out == 0 || T == 0) return hipSuccess;
  const int xq_vec = ((uintptr_t)xq % 16 == 0) && (ld_q % 16 == 0);
  const int n = L.n, m = L.m;
#define SBN_CASE(NN, MM, CB)                                                                    \
  if (n == NN && m == MM)                                                                       \
    return launch_pattern<NN, MM, CB>(h, xq, ld_q, xq_vec, absmax, T, y, ld_y, out_kind, s);
  SBN_CASE(2, 4, 8)
  SBN_CASE(4, 4, 16)
  SBN_CASE(4, 8, 8)
  SBN_CASE(6, 8, 12)
  SBN_CASE(8, 8, 16)
  SBN_CASE(8, 16, 8)
  SBN_CASE(16, 16, 16)
#undef SBN_CASE
  return launch_pattern<0, 0, 0>(h, xq, ld_q, xq_vec, absmax, T, y, ld_y, out_kind, s);
}

}  // namespace sbn
