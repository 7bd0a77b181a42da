// Absmean ternary quantization with a dynamic n:m keep mask, written as packed bricks; and the
// export kernels that turn a handle back into canonical arrays.
//
// "Microsoft BitNet 1.58: The Era of 1-Bit Large Language Models", section "The BitLinear
// Layer", operation 3 (latent weights, scale = mean absolute value); "BitNet b1.58: How Ternary
// Weights Cut LLM Memory by 82% Without Losing Accuracy", section "How ternary quantization works
// during training" (divide by the mean absolute value, round to nearest, clamp to [-1, 1]);
// "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to Semi-Structured Sparsity", Abstract
// (dynamic N:M sparsification) and Figure 6 (keep the N largest normalized magnitudes of each
// M-block; since gamma > 0 scales every magnitude alike, ranking |w| gives the same choice).
//
//   gamma = fl32( sum |w| (fp64) / (n_out * K) )
//   keep  = the n largest |w| of each m-group along K, equal magnitudes to the lower position
//   code  = keep ? (|w| > gamma/2 ? sign(w) : 0) : 0
//
// gamma is a two-stage reduction with a fixed block count per shape and a fixed combine order,
// so it is identical run to run. The pack kernel reads gamma from device memory (no host sync).
#include "sbn_internal.hpp"

namespace sbn {
namespace {

constexpr int kAbsmeanThreads = 256;
constexpr int kMaxAbsmeanBlocks = 2048;

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double r = 0.0;
  if (threadIdx.x == 0) {
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r += red[i];
  }
  return r;  // valid in thread 0
}

// Stage 1: block b sums |w| over rows [b*n_out/B, (b+1)*n_out/B) in fp64.
__global__ __launch_bounds__(kAbsmeanThreads) void absmean_partial(const float* __restrict__ w,
                                                                   int64_t n_out, int64_t K,
                                                                   int64_t ld_w, int vec4,
                                                                   double* __restrict__ partials) {
  __shared__ double red[kAbsmeanThreads / 64];
  const int64_t B = gridDim.x;
  const int64_t r0 = n_out * blockIdx.x / B, r1 = n_out * (blockIdx.x + 1) / B;
  double acc = 0.0;
  if (vec4) {
    const int64_t kv = K >> 2;
    for (int64_t r = r0; r < r1; ++r) {
      const float4* row = reinterpret_cast<const float4*>(w + r * ld_w);
      for (int64_t i = threadIdx.x; i < kv; i += kAbsmeanThreads) {
        const float4 f = row[i];
        acc += (double)fabsf(f.x) + (double)fabsf(f.y) + (double)fabsf(f.z) + (double)fabsf(f.w);
      }
    }
  } else {
    for (int64_t r = r0; r < r1; ++r) {
      const float* row = w + r * ld_w;
      for (int64_t i = threadIdx.x; i < K; i += kAbsmeanThreads) acc += (double)fabsf(row[i]);
    }
  }
  const double s = block_sum_f64(acc, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

// Stage 2: one block combines the partials in a fixed order and writes gamma.
__global__ __launch_bounds__(kAbsmeanThreads) void absmean_finalize(
    const double* __restrict__ partials, int num, double count, float* __restrict__ gamma) {
  __shared__ double red[kAbsmeanThreads / 64];
  double acc = 0.0;
  for (int i = threadIdx.x; i < num; i += kAbsmeanThreads) acc += partials[i];
  const double s = block_sum_f64(acc, red);
  if (threadIdx.x == 0) gamma[0] = count > 0.0 ? (float)(s / count) : 0.0f;
}

// Ranks of one m-group: keep[i] iff fewer than n group members precede i in the order
// (|w| descending, position ascending). Magnitudes compare as their fp32 bit patterns.
template <int M>
__device__ __forceinline__ uint32_t keep_mask_group(const uint32_t (&a)[M], int n) {
  uint32_t keep = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    int rank = 0;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      if (j < i) rank += (a[j] >= a[i]) ? 1 : 0;
      if (j > i) rank += (a[j] > a[i]) ? 1 : 0;
    }
    keep |= (rank < n ? 1u : 0u) << i;
  }
  return keep;
}

// One thread per brick slot (slot order, so each wave writes one contiguous block of bricks).
template <int M>
__global__ __launch_bounds__(256) void pack_bricks(const float* __restrict__ w, int64_t ld_w,
                                                   Layout L, const float* __restrict__ gamma_p,
                                                   uint8_t* __restrict__ mask_plane,
                                                   uint8_t* __restrict__ code_plane) {
  const int64_t slot = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = L.row_blocks * L.quads * 64;
  if (slot >= total) return;
  const int lane = (int)(slot & 63);
  const int64_t frag = slot >> 6;
  const int64_t rb = frag / L.quads, bq = frag % L.quads;
  const int64_t row = rb * 16 + (lane & 15);
  const int64_t brick = bq * 4 + (lane >> 4);
  const int64_t k0 = brick * kBrickK;
  if (row >= L.n_out || k0 >= L.K) return;  // padding bricks stay zero
  const float half = 0.5f * gamma_p[0];
  const uint32_t half_bits = __float_as_uint(half);
  const int n = L.n;
  const float* wr = w + row * ld_w + k0;
  const int groups = (int)min<int64_t>(kBrickK / M, (L.K - k0) / M);

  uint64_t maskbits = 0;
  uint64_t pend = 0;  // code bits not yet stored (sequence order)
  int npend = 0;
  uint8_t* cdst = code_plane + slot * L.code_brick_bytes;
  const bool plane = plane_order(n, M);
  int cbyte = 0;
  for (int g = 0; g < groups; ++g) {
    uint32_t a[M], sgn[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const uint32_t u = __float_as_uint(wr[g * M + i]);
      a[i] = u & 0x7FFFFFFFu;
      sgn[i] = u >> 31;
    }
    const uint32_t keep = (n == M) ? ((1u << M) - 1u) : keep_mask_group<M>(a, n);
    maskbits |= (uint64_t)keep << (g * M);
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if ((keep >> i) & 1u) {
        const uint32_t c = a[i] > half_bits ? (sgn[i] ? 3u : 1u) : 0u;
        pend |= (uint64_t)c << npend;
        npend += 2;
      }
    }
    if (plane) {
      // plane order: store whole 16-code words (the code plane is 4-byte aligned per brick)
      while (npend >= 32) {
        reinterpret_cast<uint32_t*>(cdst)[cbyte >> 2] = seq_to_plane((uint32_t)pend);
        cbyte += 4;
        pend >>= 32;
        npend -= 32;
      }
    } else {
      while (npend >= 8) {
        cdst[cbyte++] = (uint8_t)(pend & 0xFFu);
        pend >>= 8;
        npend -= 8;
      }
    }
  }
  if (npend > 0) {
    if (plane) {
      reinterpret_cast<uint32_t*>(cdst)[cbyte >> 2] = seq_to_plane((uint32_t)pend);
    } else {
      cdst[cbyte++] = (uint8_t)(pend & 0xFFu);
    }
  }
  if (L.has_mask) {
    uint2* mdst = reinterpret_cast<uint2*>(mask_plane + slot * 8);
    *mdst = make_uint2((uint32_t)maskbits, (uint32_t)(maskbits >> 32));
  }
}

__device__ __forceinline__ void load_brick(const Layout& L, const uint8_t* mask_plane,
                                           const uint8_t* code_plane, int64_t slot,
                                           uint32_t mask[2], uint32_t codes[4]) {
  mask[0] = mask[1] = 0;
  if (L.has_mask) {
    const uint2 m = *reinterpret_cast<const uint2*>(mask_plane + slot * 8);
    mask[0] = m.x;
    mask[1] = m.y;
  }
  codes[0] = codes[1] = codes[2] = codes[3] = 0;
  const uint8_t* c = code_plane + slot * L.code_brick_bytes;
  for (int i = 0; i < L.code_brick_bytes; ++i) codes[i >> 2] |= (uint32_t)c[i] << (8 * (i & 3));
}

// Canonical export: codes int8 [n_out][K], keep uint8 [n_out][K].
__global__ __launch_bounds__(256) void export_canonical(Layout L, const uint8_t* mask_plane,
                                                        const uint8_t* code_plane,
                                                        int8_t* __restrict__ codes_out,
                                                        uint8_t* __restrict__ keep_out) {
  const int64_t nbricks = (L.K + kBrickK - 1) / kBrickK;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= L.n_out * nbricks) return;
  const int64_t row = idx / nbricks, brick = idx % nbricks;
  const int64_t slot = brick_slot(L, row, brick);
  uint32_t mask[2], codes[4], dec[16];
  load_brick(L, mask_plane, code_plane, slot, mask, codes);
  decode_brick_plain(mask, codes, L.n, L.m, L.has_mask, dec);
  const int64_t k0 = brick * kBrickK;
  const int cnt = (int)min<int64_t>(kBrickK, L.K - k0);
  for (int i = 0; i < cnt; ++i) {
    const int64_t o = row * L.K + k0 + i;
    if (codes_out) codes_out[o] = (int8_t)((dec[i >> 2] >> (8 * (i & 3))) & 0xFFu);
    if (keep_out) keep_out[o] = L.has_mask ? (uint8_t)((mask[i >> 5] >> (i & 31)) & 1u) : 1;
  }
}

// Reference packed format export: per row, code bytes [code_row_bytes] and mask bytes
// [mask_row_bytes]; brick b's bits are the row stream's bytes [b*cbb, (b+1)*cbb) and [8b, 8b+8).
__global__ __launch_bounds__(256) void export_rpf(Layout L, const uint8_t* mask_plane,
                                                  const uint8_t* code_plane, int64_t crb,
                                                  int64_t mrb, uint8_t* __restrict__ code_out,
                                                  uint8_t* __restrict__ mask_out) {
  const int64_t nbricks = (L.K + kBrickK - 1) / kBrickK;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= L.n_out * nbricks) return;
  const int64_t row = idx / nbricks, brick = idx % nbricks;
  const int64_t slot = brick_slot(L, row, brick);
  if (code_out) {
    const int64_t b0 = brick * L.code_brick_bytes;
    const int cnt = (int)min<int64_t>(L.code_brick_bytes, crb - b0);
    const uint8_t* src = code_plane + slot * L.code_brick_bytes;
    if (plane_order(L.n, L.m)) {
      for (int i = 0; i < cnt; i += 4) {
        const uint32_t seq = plane_to_seq(*reinterpret_cast<const uint32_t*>(src + i));
        for (int j = 0; j < 4 && i + j < cnt; ++j)
          code_out[row * crb + b0 + i + j] = (uint8_t)(seq >> (8 * j));
      }
    } else {
      for (int i = 0; i < cnt; ++i) code_out[row * crb + b0 + i] = src[i];
    }
  }
  if (mask_out && L.has_mask) {
    const int64_t b0 = brick * 8;
    const int cnt = (int)min<int64_t>(8, mrb - b0);
    for (int i = 0; i < cnt; ++i) mask_out[row * mrb + b0 + i] = mask_plane[slot * 8 + i];
  }
}

__global__ void copy_gamma(const float* src, float* dst) { dst[0] = src[0]; }

}  // namespace

int absmean_blocks(int64_t n_out) {
  if (n_out <= 0) return 1;
  return (int)std::min<int64_t>(n_out, kMaxAbsmeanBlocks);
}

hipError_t launch_pack(const float* w, int64_t ld_w, const sbn_packed* h, hipStream_t s) {
  const Layout& L = h->L;
  const int vec4 = ((uintptr_t)w % 16 == 0) && (ld_w % 4 == 0) && (L.K % 4 == 0);
  if (L.n_out > 0) {
    hipLaunchKernelGGL(absmean_partial, dim3(h->num_partials), dim3(kAbsmeanThreads), 0, s, w,
                       L.n_out, L.K, ld_w, vec4, h->partials);
  }
  hipLaunchKernelGGL(absmean_finalize, dim3(1), dim3(kAbsmeanThreads), 0, s, h->partials,
                     L.n_out > 0 ? h->num_partials : 0, (double)L.n_out * (double)L.K, h->gamma);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || L.n_out == 0) return e;
  const int64_t total = L.row_blocks * L.quads * 64;
  const dim3 grid((unsigned)((total + 255) / 256));
  switch (L.m) {
    case 4:
      hipLaunchKernelGGL(pack_bricks<4>, grid, dim3(256), 0, s, w, ld_w, L, h->gamma, h->mask,
                         h->codes);
      break;
    case 8:
      hipLaunchKernelGGL(pack_bricks<8>, grid, dim3(256), 0, s, w, ld_w, L, h->gamma, h->mask,
                         h->codes);
      break;
    default:
      hipLaunchKernelGGL(pack_bricks<16>, grid, dim3(256), 0, s, w, ld_w, L, h->gamma, h->mask,
                         h->codes);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_export(const sbn_packed* h, int8_t* codes, uint8_t* keep, float* gamma,
                         hipStream_t s) {
  const Layout& L = h->L;
  const int64_t nbricks = (L.K + kBrickK - 1) / kBrickK;
  const int64_t total = L.n_out * nbricks;
  if ((codes || keep) && total > 0) {
    hipLaunchKernelGGL(export_canonical, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       L, h->mask, h->codes, codes, keep);
  }
  if (gamma) hipLaunchKernelGGL(copy_gamma, dim3(1), dim3(1), 0, s, h->gamma, gamma);
  return hipGetLastError();
}

hipError_t launch_export_rpf(const sbn_packed* h, uint8_t* code_bytes, uint8_t* mask_bytes,
                             hipStream_t s) {
  const Layout& L = h->L;
  const int64_t nbricks = (L.K + kBrickK - 1) / kBrickK;
  const int64_t total = L.n_out * nbricks;
  if (total > 0 && (code_bytes || mask_bytes)) {
    hipLaunchKernelGGL(export_rpf, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, L,
                       h->mask, h->codes, (int64_t)h->code_row_bytes, (int64_t)h->mask_row_bytes,
                       code_bytes, mask_bytes);
  }
  return hipGetLastError();
}

}  // namespace sbn
